"""Helpers for GPU-vs-oracle parity tests (inputs on the GPU, oracle on the CPU)."""
import os

import numpy as np
import torch

import oracle
from block_scaled_fp8_amd import synth

OUT_TOL = 2e-2          # max |gpu - oracle| <= OUT_TOL * RMS(oracle output)
AFF_RTOL = 2e-6         # fp32 exp/sum/divide against float64


def gpu_case(name_or_cfg, seed=0, activation="swiglu", weight_format="e4m3_128"):
    cfg = synth.CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    dev = "cuda"
    # tiny geometries are drawn on the CPU; the large ones on the GPU
    gen_dev = "cpu" if cfg.E * 3 * cfg.H * cfg.I < (64 << 20) else dev
    case = synth.make_case(cfg, seed, gen_dev, activation, weight_format)
    case["activation"] = activation
    for n in ("x", "logits", "w13", "w13_scale", "w2", "w2_scale"):
        case[n] = case[n].to(dev)
    if case["shared"] is not None:
        case["shared"] = {n: t.to(dev) for n, t in case["shared"].items()}
    return case


def np_(t):
    return t.detach().cpu().numpy()


def oracle_rows(case, ids, aff, rows, with_shared=True, xrows=None, hidden="exact"):
    """Oracle output for the given token rows, copying only the experts they use.

    The case's "activation" entry selects the expert MLP; xrows, when given,
    replaces the activation rows, e.g. by their fp8 quantisation.  With
    hidden="mxfp4" the down GEMM takes the MXFP4-quantised hidden activation
    and the result is (out, bound): bound per element on how far a kernel
    that takes the quantisation decisions from fp32 sums can be from out on
    that account (oracle.moe_ffn, bound=True)."""
    rows = np.asarray(rows)
    sub_ids = np.asarray(ids)[rows]
    uniq = np.unique(sub_ids)
    sel = torch.as_tensor(uniq, dtype=torch.long, device=case["w13"].device)
    w13 = np_(case["w13"].index_select(0, sel))
    w13s = np_(case["w13_scale"].index_select(0, sel))
    w2 = np_(case["w2"].index_select(0, sel))
    w2s = np_(case["w2_scale"].index_select(0, sel))
    remap = np.searchsorted(uniq, sub_ids)
    sh = None
    if with_shared and case.get("shared") is not None:
        sh = {n: np_(t) for n, t in case["shared"].items()}
    x = np_(case["x"].double())[rows] if xrows is None else np.asarray(xrows, dtype=np.float64)
    return oracle.moe_ffn(x, w13, w13s, w2, w2s, remap, np.asarray(aff)[rows], sh,
                          activation=case.get("activation", "swiglu"),
                          weight_format=case.get("weight_format", "e4m3_128"),
                          hidden=hidden, bound=hidden != "exact")


# With a flip bound, at most this fraction of the outputs may need it (be
# more than tol * RMS from the oracle): a kernel's fp32 sums land on the other
# side of a quantisation midpoint only rarely, and a wrong kernel misses
# everywhere.
FLIP_FRAC = 1e-3


def assert_out_close(got, ref, tol=OUT_TOL, what="", bound=None):
    """max |got - ref| <= tol * RMS(ref); with bound (per element, from the
    oracle), |got - ref| - bound <= tol * RMS(ref) element by element, and
    at most FLIP_FRAC of the elements beyond OUT_TOL * RMS at all."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite GPU output"
    rms = float(np.sqrt(np.mean(ref ** 2)))
    d = np.abs(got - ref)
    extra = ""
    if bound is not None:
        bound = np.asarray(bound, dtype=np.float64)
        assert bound.shape == ref.shape
        over = int(np.count_nonzero(d > OUT_TOL * rms))
        extra = (f" flip-bound: {np.count_nonzero(bound)} elements, max {bound.max() / max(rms, 1e-300):.3g} rms,"
                 f" max|d| there {d[bound > 0].max() / max(rms, 1e-300) if np.any(bound > 0) else 0:.3g} rms,"
                 f" {over} beyond tol")
        assert over <= FLIP_FRAC * d.size, f"{what}: {over} of {d.size} outputs beyond {OUT_TOL} * RMS"
        d = d - bound
    err = float(np.max(d)) if got.size else 0.0
    line = f"[parity] {what}: max|d|={err:.4g} rms={rms:.4g} ratio={err / max(rms, 1e-300):.4g}{extra}"
    print(line, flush=True)
    log = os.environ.get("MOE_PARITY_LOG")
    if log:
        with open(log, "a") as f:
            f.write(line + "\n")
    assert err <= tol * rms, f"{what}: max|gpu-oracle| = {err:.4g} > {tol} * RMS {rms:.4g}"


def sample_rows(T, n, seed=0):
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=n - 2, replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick))


def pack_reference(w):
    """numpy statement of the tile-coalesced layout: out[((t*(C/64)+c)*64+l)*16+b] =
    w[16t + l%16, 64c + 16(l//16) + b] for each matrix."""
    w = np.asarray(w)
    *lead, R, C = w.shape
    v = w.reshape(*lead, R // 16, 16, C // 64, 4, 16)          # [.., t, l%16, c, l//16, b]
    v = np.moveaxis(v, -2, -4)                                    # [.., t, l//16, l%16, c, b]
    v = np.moveaxis(v, -2, -4)                                    # [.., t, c, l//16, l%16, b]
    return np.ascontiguousarray(v).reshape(w.shape)


def tiled_case(case):
    """A copy of a GPU case whose expert weights are packed for the tiled
    layout (MXFP4 scales too)."""
    from block_scaled_fp8_amd import binding
    return binding.pack_weights(case, case.get("weight_format", "e4m3_128"))
