"""moe_fused_w8a16_noalloc, the entry point for callers that cannot allocate,
against moe_fused_w8a16 with a caller workspace: the same kernels on the same
inputs, so the outputs must be identical bit for bit (stricter than the
2e-2 * RMS bar of the oracle comparisons).  Two calls in a row on the one
device scratch array, the second smaller, then a call too large for it."""
import pytest
import torch

from block_scaled_fp8_amd import binding, synth

from _parity import gpu_case

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _both(c, T, variant, activation, shared):
    x, ids, aff = c["x"][:T], c["ids"][:T], c["aff"][:T]
    sh = c["shared"] if shared else None
    ref = binding.fused_w8a16(x, c["w13"], c["w13_scale"], c["w2"], c["w2_scale"], ids, aff,
                              shared=sh, variant=variant, activation=activation)
    out = torch.full((T, x.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    binding.fused_w8a16_noalloc(x, c["w13"], c["w13_scale"], c["w2"], c["w2_scale"], ids, aff,
                                out, shared=sh, status=status, variant=variant,
                                activation=activation)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    return out, ref


@pytest.mark.parametrize("variant,activation", [("auto", "swiglu"), ("decode", "swiglu"),
                                                ("prefill", "swiglu"), ("prefill_a8", "swiglu"),
                                                ("auto", "relu2")])
def test_noalloc_matches_workspace_call(variant, activation):
    # decode64's geometry with a shared expert: 64 tokens, then 16 on the
    # same scratch array (which still holds the first call's data)
    cfg = synth.MoeConfig("na", T=64, H=2048, I=512, E=256, k=8, shared=True)
    c = gpu_case(cfg, seed=77, activation=activation)
    c["ids"], c["aff"] = binding.route(c["logits"], cfg.k)
    for T in (64, 16):
        for shared in (True, False):
            out, ref = _both(c, T, variant, activation, shared)
            assert torch.equal(out, ref), f"{variant}/{activation} T={T} shared={shared}"


def test_noalloc_rejects_a_call_beyond_the_scratch_array():
    cfg = synth.MoeConfig("na_big", T=8192, H=2048, I=512, E=8, k=8)
    c = gpu_case(cfg, seed=78)
    ids, aff = binding.route(c["logits"], cfg.k)
    need = binding.fused_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, variant="prefill")
    assert need > binding.MOE_NOALLOC_SCRATCH_BYTES
    out = torch.zeros((cfg.T, cfg.H), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.MoeError) as ei:
        binding.fused_w8a16_noalloc(c["x"], c["w13"], c["w13_scale"], c["w2"], c["w2_scale"],
                                    ids, aff, out, variant="prefill")
    assert ei.value.code == binding.MOE_EUNSUPPORTED
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out).item()) == 0   # nothing was launched
