"""GPU parity of the MXFP4-weight path (moe_fused_mxfp4, W4A16) against the
float64 oracle on the same codes and scales.

MXFP4 as named by "Add gfx950 Q256 fused MXFP4 prefill pipeline" (ROCm/aiter
PR #5988) and "NKI Library Supported Kernel Reference" (Blockwise MM Block
MX), read as the OCP Microscaling format: E2M1 codes, one E8M0 scale per 32
consecutive elements of a row.  Same bar as the FP8 path: routing ids exact,
max |gpu - oracle| <= 2e-2 * RMS(oracle output), every row up to the
8192-token workload and the structured sample at 16384 tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scaled_fp8_amd import binding, synth

from _parity import assert_out_close, gpu_case, np_, oracle_rows, tiled_case
from test_gpu_parity import SEG_SIZES, TILE_M, _xhat_rows, check_rows

pytestmark = pytest.mark.gpu


def _x4hat_rows(c, rows):
    """The oracle's MXFP4 quantisation of the given rows of x, dequantised."""
    xr = np_(c["x"][torch.as_tensor(rows, device=c["x"].device)].float())
    return oracle.dequantize_mx(*oracle.quantize_rows_mxfp4(xr))


def _xq_rows(c, rows, variant):
    """The rows of x the variant's experts compute from (None: x itself)."""
    if variant == "prefill_a8":
        return _xhat_rows(c, rows)
    if variant in ("prefill_a4", "prefill_fp4"):
        return _x4hat_rows(c, rows)
    return None


# prefill_fp4 computes from the same MXFP4 operands as its oracle (x_hat, the
# weights and, away from quantisation flips, the hidden activation), so only
# fp32 sums and the block floating-point contributions separate the two:
# measured up to 3.3e-4 * RMS (scale bytes 1 and 140), 1.7e-6 at 8192 tokens.
FP4_TOL = 2e-3


def _tol(variant):
    return FP4_TOL if variant == "prefill_fp4" else 2e-2


def _ref(c, ids, aff, rows, variant, with_shared=True):
    """The oracle's rows for the variant and, for prefill_fp4 (the hidden
    activation quantised to MXFP4 as well), its per-element bound on what a
    kernel taking the quantisation decisions from fp32 sums may differ by
    (None for the other variants)."""
    xr = _xq_rows(c, rows, variant)
    if variant == "prefill_fp4":
        return oracle_rows(c, ids, aff, rows, with_shared=with_shared, xrows=xr, hidden="mxfp4")
    return oracle_rows(c, ids, aff, rows, with_shared=with_shared, xrows=xr), None

_cases = {}
_oracle = {}


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _case(name, activation):
    key = (name, activation)
    if key not in _cases:
        _cases.clear()
        _oracle.clear()
        torch.cuda.empty_cache()
        c = gpu_case(name, seed=1, activation=activation, weight_format="mxfp4")
        c["tiled"] = tiled_case(c)
        _cases[key] = c
    return _cases[key]


def _run(c, ids, aff, layout, activation, variant="auto", shared=True, status=None):
    g = c["tiled"] if layout == "tiled" else c
    return binding.fused_w8a16(g["x"], g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], ids, aff,
                               shared=g["shared"] if shared else None, variant=variant,
                               layout=layout, activation=activation, weight_format="mxfp4",
                               status=status)


# (AUTO: the decode kernels up to 16 routes per expert, the grouped GEMMs
# above; the large workloads also run the decode kernels' row-tile form and
# the grouped GEMMs with x quantised to E4M3 per token or to MXFP4)
@pytest.mark.parametrize("variant", ["auto", "decode", "prefill_a8", "prefill_a4", "prefill_fp4"])
@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("activation", ["swiglu", "relu2"])
@pytest.mark.parametrize("name", synth.CONFIG_ORDER)
def test_mxfp4_parity(name, activation, layout, variant):
    c = _case(name, activation)
    cfg = c["cfg"]
    if variant != "auto" and cfg.routes <= 16 * cfg.E:
        pytest.skip("decode-sized batch: AUTO runs the decode kernels")
    ids, aff = binding.route(c["logits"], cfg.k)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = _run(c, ids, aff, layout, activation, variant=variant, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref_ids, ref_aff = oracle.route_softmax_topk(np_(c["logits"]), cfg.k)
    assert np.array_equal(np_(ids), ref_ids)
    rows = check_rows(name, cfg, ref_ids)
    key = (activation, variant if variant.startswith("prefill_") else "x")
    if key not in _oracle:
        _oracle[key] = _ref(c, ref_ids, ref_aff, rows, variant)
    ref, bnd = _oracle[key]
    assert_out_close(np_(out)[rows], ref, bound=bnd, tol=_tol(variant),
                     what=f"mxfp4 {name}/{activation}/{layout}/{variant} ({len(rows)} rows)")


# the decode kernels: odd chunk counts (H/128 = 3, I/128 = 1 or 3), token
# boundaries and both self-routed (T*k <= 4096) and sorted (T*k > 4096) forms
@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("T,H,I,E,k", [(1, 384, 128, 16, 4), (17, 384, 384, 16, 4),
                                       (37, 256, 128, 8, 2), (130, 384, 256, 130, 8),
                                       (1100, 256, 128, 64, 4)])
def test_mxfp4_shapes(T, H, I, E, k, layout):
    cfg = synth.MoeConfig("mxs", T=T, H=H, I=I, E=E, k=k, shared=True)
    c = gpu_case(cfg, seed=T + H, weight_format="mxfp4")
    g = tiled_case(c) if layout == "tiled" else c
    ids, aff = binding.route(c["logits"], k)
    out = binding.fused_w8a16(g["x"], g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], ids, aff,
                              shared=g["shared"], layout=layout, weight_format="mxfp4",
                              variant="decode")
    torch.cuda.synchronize()
    ref_ids, ref_aff = oracle.route_softmax_topk(np_(c["logits"]), k)
    ref = oracle_rows(c, ref_ids, ref_aff, np.arange(T))
    assert_out_close(np_(out), ref, what=f"mxfp4 T={T} H={H} I={I} E={E} k={k}/{layout}")


@pytest.mark.parametrize("variant", ["decode", "prefill", "prefill_a8", "prefill_a4", "prefill_fp4"])
def test_mxfp4_scale_bytes_at_the_ends_and_zero_affinities(variant):
    """Scale bytes 1 (2^-126) and 140 (2^13) on some blocks, the rest as drawn;
    outputs stay finite and match the oracle; zero affinities give exactly 0."""
    cfg = synth.MoeConfig("mxe", T=24, H=256, I=256, E=8, k=2)
    c = gpu_case(cfg, seed=5, weight_format="mxfp4")
    c["w13_scale"][:, ::7, 1] = 1
    c["w2_scale"][:, ::5, 0] = 1
    c["w13_scale"][3, 0, 0] = 140   # one gate block of expert 3: 2^13 instead of about 2^-9
    ids, aff = binding.route(c["logits"], cfg.k)
    out = binding.fused_w8a16(c["x"], c["w13"], c["w13_scale"], c["w2"], c["w2_scale"], ids, aff,
                              weight_format="mxfp4", variant=variant)
    torch.cuda.synchronize()
    ref_ids, ref_aff = oracle.route_softmax_topk(np_(c["logits"]), cfg.k)
    rows = np.arange(cfg.T)
    ref, bnd = _ref(c, ref_ids, ref_aff, rows, variant)
    assert np.all(np.isfinite(ref))
    assert_out_close(np_(out), ref, bound=bnd, tol=_tol(variant),
                     what=f"mxfp4 {variant} scale bytes 1 and 140")
    zero = torch.zeros_like(aff)
    out0 = binding.fused_w8a16(c["x"], c["w13"], c["w13_scale"], c["w2"], c["w2_scale"], ids,
                               zero, weight_format="mxfp4", variant=variant)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out0).item()) == 0


# The grouped-GEMM (prefill) variant on MXFP4 weights: several 128-row tiles
# with ragged tails, down K = 128 (a single 128-wide chunk), 3 column blocks
# of 256, relu^2 up projections of an odd number of 128-column blocks (I = 384)
# and the shared expert's rows.
@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("activation", ["swiglu", "relu2"])
@pytest.mark.parametrize("T,H,I,E,k", [(300, 512, 256, 8, 2), (257, 256, 384, 16, 4),
                                       (129, 768, 128, 4, 1)])
def test_mxfp4_prefill_shapes(T, H, I, E, k, activation, layout):
    cfg = synth.MoeConfig("mxp", T=T, H=H, I=I, E=E, k=k, shared=True)
    c = gpu_case(cfg, seed=T + I, activation=activation, weight_format="mxfp4")
    g = tiled_case(c) if layout == "tiled" else c
    ids, aff = binding.route(c["logits"], k)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = binding.fused_w8a16(g["x"], g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], ids, aff,
                              shared=g["shared"], variant="prefill", layout=layout,
                              activation=activation, weight_format="mxfp4", status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    ref_ids, ref_aff = oracle.route_softmax_topk(np_(c["logits"]), k)
    ref = oracle_rows(c, ref_ids, ref_aff, np.arange(T))
    assert_out_close(np_(out), ref,
                     what=f"mxfp4 prefill T={T} H={H} I={I} E={E} k={k}/{activation}/{layout}")


def test_mxfp4_unaligned_scales_take_the_decode_kernels():
    """The prefill GEMMs stage E8M0 scales 4 bytes at a time: on scale arrays
    that are not 4-byte aligned AUTO runs the decode kernels (same result),
    and an explicit prefill variant is refused."""
    cfg = synth.MoeConfig("mxu", T=300, H=256, I=256, E=8, k=2)
    c = gpu_case(cfg, seed=9, weight_format="mxfp4")

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=torch.uint8, device=t.device)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    s13, s2 = shifted(c["w13_scale"]), shifted(c["w2_scale"])
    assert s13.data_ptr() % 4 != 0
    ids, aff = binding.route(c["logits"], cfg.k)
    out = binding.fused_w8a16(c["x"], c["w13"], s13, c["w2"], s2, ids, aff, weight_format="mxfp4")
    ref_out = binding.fused_w8a16(c["x"], c["w13"], c["w13_scale"], c["w2"], c["w2_scale"], ids,
                                  aff, weight_format="mxfp4", variant="decode")
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    ref_ids, ref_aff = oracle.route_softmax_topk(np_(c["logits"]), cfg.k)
    assert_out_close(np_(out), oracle_rows(c, ref_ids, ref_aff, np.arange(cfg.T)),
                     what="mxfp4 unaligned scales, auto")
    for v in ("prefill", "prefill_a8", "prefill_a4", "prefill_fp4"):
        with pytest.raises(binding.MoeError) as ei:
            binding.fused_w8a16(c["x"], c["w13"], s13, c["w2"], s2, ids, aff, variant=v,
                                weight_format="mxfp4")
        assert ei.value.code == binding.MOE_EINVAL


@pytest.mark.parametrize("shape", [(1, 16, 4), (3, 256, 64), (2, 1024, 16)])
def test_pack_mx_scales_matches_reference(shape):
    g = torch.Generator().manual_seed(sum(shape))
    sc = torch.randint(0, 256, shape, generator=g, dtype=torch.int64).to(torch.uint8)
    got = np_(binding.pack_mx_scales(sc.cuda()))
    n, R, C = shape
    ref = np.empty(n * R * C, np.uint8)
    src = sc.numpy()
    for m in range(n):
        for t in range(R // 16):
            for c in range(C // 4):
                for l in range(64):
                    ref[m * R * C + (t * (C // 4) + c) * 64 + l] = src[m, 16 * t + l % 16, 4 * c + l // 16]
    assert np.array_equal(got.reshape(-1), ref)


# x quantised to E4M3 per token (gate/up or up as E4M3 x E2M1) or to MXFP4
# (E2M1 x E2M1) on the scaled MFMA, with the E8M0 bytes as its per-lane
# scales: against the oracle run on the same quantised rows
# (MXFP4 x stages its scales from a per-tile table for H = 512 * 2^j <= 8192,
#  H = 512 and 8192 below and the large workloads; per step otherwise: H = 256,
#  768 and 8448)
@pytest.mark.parametrize("variant", ["prefill_a8", "prefill_a4", "prefill_fp4"])
@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("activation", ["swiglu", "relu2"])
@pytest.mark.parametrize("T,H,I,E,k", [(300, 512, 256, 8, 2), (257, 256, 384, 16, 4),
                                       (129, 768, 128, 4, 1), (41, 8192, 128, 4, 2),
                                       (37, 8448, 128, 4, 2)])
def test_mxfp4_prefill_quantised_x_shapes(T, H, I, E, k, activation, layout, variant):
    cfg = synth.MoeConfig("mxq", T=T, H=H, I=I, E=E, k=k, shared=True)
    c = gpu_case(cfg, seed=T + I + 1, activation=activation, weight_format="mxfp4")
    g = tiled_case(c) if layout == "tiled" else c
    ids, aff = binding.route(c["logits"], k)
    out = binding.fused_w8a16(g["x"], g["w13"], g["w13_scale"], g["w2"], g["w2_scale"], ids, aff,
                              shared=g["shared"], variant=variant, layout=layout,
                              activation=activation, weight_format="mxfp4")
    torch.cuda.synchronize()
    ref_ids, ref_aff = oracle.route_softmax_topk(np_(c["logits"]), k)
    rows = np.arange(T)
    ref, bnd = _ref(c, ref_ids, ref_aff, rows, variant)
    assert_out_close(np_(out), ref, bound=bnd, tol=_tol(variant),
                     what=f"mxfp4 {variant} T={T} H={H} I={I} E={E} k={k}/{activation}/{layout}")


@pytest.mark.parametrize("variant", ["prefill", "prefill_a8", "prefill_a4", "prefill_fp4"])
def test_mxfp4_nan_activation_row(variant):
    """A NaN in one token's activations gives that token an all-NaN output
    row (with MXFP4 activations through the E8M0 NaN byte of its run), as the
    oracle's; every other row still matches."""
    cfg = synth.MoeConfig("mxn", T=40, H=512, I=256, E=16, k=4, shared=True)
    c = gpu_case(cfg, seed=23, weight_format="mxfp4")
    t0 = 7
    c["x"][t0, 100] = float("nan")
    ids, aff = binding.route(c["logits"], cfg.k)
    out = np_(_run(c, ids, aff, "rowmajor", "swiglu", variant=variant))
    torch.cuda.synchronize()
    ref_ids, ref_aff = oracle.route_softmax_topk(np_(c["logits"]), cfg.k)
    ref0, _ = _ref(c, ref_ids, ref_aff, np.array([t0]), variant)
    assert np.all(np.isnan(ref0))
    assert np.all(np.isnan(out[t0])), f"{variant}: {int(np.sum(~np.isnan(out[t0])))} non-NaN values"
    rows = np.array([t for t in range(cfg.T) if t != t0])
    ref, bnd = _ref(c, ref_ids, ref_aff, rows, variant)
    assert_out_close(out[rows], ref, bound=bnd, tol=_tol(variant), what=f"mxfp4 nan row {variant}")


@pytest.mark.parametrize("variant", ["decode", "prefill", "prefill_a8", "prefill_a4", "prefill_fp4"])
def test_mxfp4_is_deterministic_and_graph_replays(variant):
    cfg = synth.MoeConfig("mxg", T=64, H=512, I=256, E=128, k=4, shared=True)
    c = gpu_case(cfg, seed=7, weight_format="mxfp4")
    ids, aff = binding.route(c["logits"], cfg.k)
    a = _run(c, ids, aff, "rowmajor", "swiglu", variant=variant)
    b = _run(c, ids, aff, "rowmajor", "swiglu", variant=variant)
    assert torch.equal(a, b)
    ws = torch.empty(binding.fused_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, True,
                                                   variant), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(a)

    def step():
        binding.fused_w8a16(c["x"], c["w13"], c["w13_scale"], c["w2"], c["w2_scale"], ids, aff,
                            shared=c["shared"], out=out, ws=ws, weight_format="mxfp4",
                            variant=variant)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, a)


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("activation", ["swiglu", "relu2"])
@pytest.mark.parametrize("variant", ["decode", "prefill", "prefill_a8", "prefill_a4", "prefill_fp4"])
def test_mxfp4_segment_size_sweep(variant, activation, layout, shared):
    """MXFP4 weights with crafted ids giving the experts exactly SEG_SIZES
    routes each (the edges of the 32-row MFMA row groups and 128-row tiles
    of the grouped GEMMs, and of the decode kernels' row tiles); every output
    row against the oracle."""
    E, k = len(SEG_SIZES), 2
    labels = np.repeat(np.arange(E, dtype=np.int32), SEG_SIZES)
    np.random.default_rng(33).shuffle(labels)
    T = labels.size // k
    ids_np = labels.reshape(T, k)
    assert T % TILE_M == 65
    cfg = synth.MoeConfig("mxseg", T=T, H=512, I=256, E=E, k=k, shared=shared)
    c = gpu_case(cfg, seed=33, activation=activation, weight_format="mxfp4")
    g = tiled_case(c) if layout == "tiled" else c
    aff_np = synth.random_affinities(T, k, seed=33).numpy()
    out = binding.fused_w8a16(g["x"], g["w13"], g["w13_scale"], g["w2"], g["w2_scale"],
                              torch.from_numpy(ids_np).cuda(), torch.from_numpy(aff_np).cuda(),
                              shared=g["shared"] if shared else None, variant=variant, layout=layout,
                              activation=activation, weight_format="mxfp4")
    torch.cuda.synchronize()
    rows = np.arange(T)
    ref, bnd = _ref(c, ids_np, aff_np, rows, variant, with_shared=shared)
    assert_out_close(np_(out), ref, bound=bnd, tol=_tol(variant),
                     what=f"mxfp4 segments {variant}/{activation}/{layout}/shared={shared}")
