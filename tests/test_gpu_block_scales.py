"""GPU parity of the 128x128 block-scale rule on every legal scale.

The weight of a block is E4M3FN(code) * its own fp32 scale ("Gated DeltaNet
(+ FP8 MoE) -- AWS Neuron (NKI) kernels for Trainium2", section "FP8 MoE
decode kernel (moe_fused_w8_35b)", Validation paragraph: each 128x128 block
is mapped exactly).  These cases feed scales that the synthetic recipe
(block max / 448) never produces, with the codes left as drawn (nonzero):

* zero:      a zero scale on the first, a middle or the last K block of every
             scale row of every matrix, and experts whose whole down (or
             gate/up) projection has scale 0;
* wide:      adjacent K blocks scaled by 2^-100 and 2^20 in turn (a ratio of
             2^120 between neighbours);
* subnormal: one subnormal scale per gate/up row, and every down scale
             subnormal (the outputs are then around 1e-36).

Each runs through the self-routed fused decode kernel, the sorted fused
decode kernel, the split decode kernels, the bf16 prefill GEMMs and the
fp8-activation prefill, in both weight layouts and with both activations,
and every output row is compared with the unchanged float64 oracle at
2e-2 * RMS.  An expert whose down scales are all zero must add exactly 0.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8_amd import binding, synth

from _parity import assert_out_close, gpu_case, np_, oracle_rows, tiled_case

pytestmark = pytest.mark.gpu

# variant name -> (config, binding variant): the self-routed fused decode
# kernel needs >= 128 possible experts and <= 4096 routes; above 4096 routes
# the decode variant sorts first and runs the same fused kernel; with few
# experts it runs the split (expert, N-tile) kernels
VARIANTS = {
    "decode_fused": (synth.MoeConfig("bs_df", T=32, H=512, I=256, E=128, k=4, shared=True), "decode"),
    "decode_sorted": (synth.MoeConfig("bs_ds", T=1100, H=512, I=256, E=128, k=4, shared=True), "decode"),
    "decode_split": (synth.MoeConfig("bs_dp", T=40, H=512, I=256, E=16, k=4, shared=True), "decode"),
    "prefill": (synth.MoeConfig("bs_pf", T=300, H=512, I=256, E=16, k=4, shared=True), "prefill"),
    "prefill_a8": (synth.MoeConfig("bs_a8", T=300, H=512, I=256, E=16, k=4, shared=True), "prefill_a8"),
}
ZERO_DOWN_EXPERT = 1    # every down scale 0: its routes add exactly 0
ZERO_GATEUP_EXPERT = 2  # every gate/up scale 0: silu(0) * 0 = 0 and relu(0)^2 = 0


def _pattern_scales(s, pattern):
    """A copy of a scale tensor [..., rows, kblocks] with the pattern applied."""
    s = s.clone()
    nr, nk = s.shape[-2], s.shape[-1]
    if pattern == "zero":
        for r in range(nr):
            kb = (0, nk // 2, nk - 1)[r % 3]    # first, middle, last K block
            s[..., r, kb] = 0.0
    elif pattern == "wide":
        f = torch.tensor([2.0 ** -100 if kb % 2 == 0 else 2.0 ** 20 for kb in range(nk)],
                         dtype=torch.float32, device=s.device)
        s = s * f
    return s


def _make(pattern, name, activation):
    cfg, _ = VARIANTS[name]
    seed = zlib.crc32(f"{pattern}/{name}/{activation}".encode()) % 1000
    c = gpu_case(cfg, seed=seed, activation=activation)
    for key in ("w13_scale", "w2_scale"):
        c[key] = _pattern_scales(c[key], pattern)
    if c["shared"] is not None:
        sh = dict(c["shared"])
        for key in ("w13_scale", "w2_scale"):
            sh[key] = _pattern_scales(sh[key], pattern)
        c["shared"] = sh
    if pattern == "zero":
        c["w2_scale"][ZERO_DOWN_EXPERT] = 0.0
        c["w13_scale"][ZERO_GATEUP_EXPERT] = 0.0
    elif pattern == "subnormal":
        tiny = 2.0 ** -133                        # subnormal in fp32
        c["w13_scale"][..., 1] = tiny             # one K block of every gate/up row
        # every down scale subnormal: blockmax/448 (about 2^-13) times 2^-120
        c["w2_scale"] = (c["w2_scale"].double() * 2.0 ** -120).float()
        assert torch.all(c["w2_scale"] < 2.0 ** -126) and torch.all(c["w2_scale"] > 0)
        if c["shared"] is not None:
            c["shared"]["w13_scale"][..., 1] = tiny
            c["shared"]["w2_scale"] = (c["shared"]["w2_scale"].double() * 2.0 ** -120).float()
    return c


def _run(c, ids, aff, variant, layout, activation, shared=True):
    g = tiled_case(c) if layout == "tiled" else c
    return binding.fused_w8a16(g["x"], g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], ids, aff,
                               shared=g["shared"] if shared else None, variant=variant,
                               layout=layout, activation=activation)


def _xhat_rows(c, rows):
    codes, s = oracle.quantize_rows_e4m3(np_(c["x"][torch.as_tensor(rows, device=c["x"].device)].float()))
    return oracle.dequantize_rows(codes, s)


@pytest.mark.parametrize("activation", ["swiglu", "relu2"])
@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("name", list(VARIANTS))
@pytest.mark.parametrize("pattern", ["zero", "wide", "subnormal"])
def test_block_scales_parity(pattern, name, layout, activation):
    cfg, variant = VARIANTS[name]
    c = _make(pattern, name, activation)
    ids, aff = binding.route(c["logits"], cfg.k)
    out = np_(_run(c, ids, aff, variant, layout, activation))
    torch.cuda.synchronize()
    ref_ids, ref_aff = oracle.route_softmax_topk(np_(c["logits"]), cfg.k)
    assert np.array_equal(np_(ids), ref_ids)
    rows = np.arange(cfg.T)
    xr = _xhat_rows(c, rows) if variant == "prefill_a8" else None
    ref = oracle_rows(c, ref_ids, ref_aff, rows, xrows=xr)
    assert_out_close(out, ref, what=f"block scales {pattern} {name}/{layout}/{activation}")


@pytest.mark.parametrize("activation", ["swiglu", "relu2"])
@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("name", list(VARIANTS))
def test_zero_scale_experts_add_exactly_zero(name, layout, activation):
    """Every route on an expert whose down scales (or gate/up scales) are all
    zero, no shared expert: the output is exactly 0, whatever the codes."""
    cfg, variant = VARIANTS[name]
    c = _make("zero", name, activation)
    for e in (ZERO_DOWN_EXPERT, ZERO_GATEUP_EXPERT):
        ids = torch.full((cfg.T, cfg.k), e, dtype=torch.int32, device="cuda")
        # the other slots of each token on other experts, with zero affinity
        ids[:, 1:] = (e + 1 + torch.arange(cfg.k - 1, device="cuda", dtype=torch.int32)) % cfg.E
        aff = torch.zeros((cfg.T, cfg.k), dtype=torch.float32, device="cuda")
        aff[:, 0] = 1.0
        out = _run(c, ids, aff, variant, layout, activation, shared=False)
        torch.cuda.synchronize()
        nz = int(torch.count_nonzero(out).item())
        assert nz == 0, f"{name}/{layout}/{activation}: expert {e}: {nz} nonzero outputs"
