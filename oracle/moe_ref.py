"""Plain float64 reference of the routed MoE expert FFN (test infrastructure).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may use this module.

Sources (page title, then section):

* [NKI] "Gated DeltaNet (+ FP8 MoE) -- AWS Neuron (NKI) kernels for
  Trainium2", section "FP8 MoE decode kernel (moe_fused_w8_35b)": the fused
  path is gate/up GEMM -> SwiGLU -> down GEMM -> affinity scale -> expert-sum,
  on official E4M3FN weights with per 128x128 block scales ("maps each 128x128
  block exactly", Validation paragraph); the router is softmax -> top-8 ->
  normalise and the shared expert is added after the routed sum (Serving
  contract paragraph); the result is [B, H] fp32 (Interface paragraph).
* [NEMO] "nemo_automodel.components.models.qwen3_5.layers", ``_silu_mul``:
  the SwiGLU product is silu(gate) * up; ``Qwen3_5FusedMLP``: a dense SwiGLU
  MLP projects, applies silu(gate)*up and projects back.
* [SPARK] "spark_model/layers/nemotron_moe.rs", module documentation
  ("Forward: ... weighted_sum ... sum routed+shared") and the sorted prefill
  path (sort by expert, grouped GEMM, unpermute-reduce).
* [AITER] "Add gfx950 Q256 fused MXFP4 prefill pipeline" (ROCm/aiter
  PR #5988), description: tokens sorted by expert with an inverse route map,
  an FP32 route reduction, and one always-on shared expert.
* [NKILIB] "NKI Library Supported Kernel Reference", Router Top-K: the router
  computes its logits from the hidden states and then selects the top K.

Readings where the pages are silent:

* selection is taken on the fp32 logits (softmax is strictly increasing, so the
  chosen set is the same as on the probabilities), ties go to the lower expert
  index, and -0.0 equals +0.0;
* slot j of a token holds its j-th expert in that order;
* "normalise" divides each selected probability by the sum of the k selected
  probabilities;
* within one expert's segment of the sorted map, routes keep ascending flat
  route index r = t*k + j (stable order); offsets are not padded;
* the output is overwritten, fp32-or-better, summed over routes then the shared
  expert (affinity exactly 1).
"""
from __future__ import annotations

import numpy as np

BLOCK = 128
E4M3FN_MAX = 448.0


# --------------------------------------------------------------------------
# E4M3FN decoding and block dequantisation  ([NKI] weight format paragraph)
# --------------------------------------------------------------------------
def _e4m3fn_value(code: int) -> float:
    """Value of one E4M3FN byte: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits, no infinities, and only S.1111.111 reserved for NaN."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:                       # subnormal: 0.m * 2^(1-7)
        mag = (m / 8.0) * 2.0 ** (1 - 7)
    else:                            # normal: 1.m * 2^(e-7)
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e4m3fn_table() -> np.ndarray:
    """The value of every one of the 256 codes, float64 (NaN for 0x7F, 0xFF)."""
    return np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3fn_table()


def e4m3fn_decode(codes) -> np.ndarray:
    """Decode an array of E4M3FN bytes to float64."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def dequantize_blocks(codes, scales, block: int = BLOCK) -> np.ndarray:
    """W[r, c] = decode(codes[r, c]) * scales[r // 128, c // 128] (float64).

    ``codes`` is [..., R, C] uint8, ``scales`` [..., R/128, C/128] float32."""
    vals = e4m3fn_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    s = np.repeat(np.repeat(s, block, axis=-2), block, axis=-1)
    assert s.shape == vals.shape, (s.shape, vals.shape)
    return vals * s


def e4m3fn_encode_rne(v) -> np.ndarray:
    """E4M3FN codes of values with |v| <= 448: the nearest finite value of the
    format, a tie going to the code with an even mantissa (round half to even);
    the sign bit is copied, so -0.0 and small negatives give 0x80."""
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.abs(v) <= E4M3FN_MAX)
    mags = _TABLE[:0x7F]                      # codes 0x00..0x7E, increasing
    a = np.abs(v)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    return (code | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_rows_e4m3(x):
    """Per-token E4M3 quantisation of activations, decided in fp32 like the
    weights' recipe ([NKI] FP8 weights with a scale of block max / 448, here
    per token row): s = fp32(amax / 448), code = RNE(fp32(x / s)) clamped to
    +-448; a row of zeros gets s = 0 and zero codes.  Returns (codes uint8
    [T, H], scales float32 [T]); the GEMM uses decode(code) * s."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.abs(x32).max(axis=1)
    s = (amax / np.float32(E4M3FN_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    v = (x32 / safe[:, None]).astype(np.float32)
    v = np.clip(v, -E4M3FN_MAX, E4M3FN_MAX)
    codes = e4m3fn_encode_rne(v)
    codes[s == 0] = 0
    return codes, s


def dequantize_rows(codes, scales) -> np.ndarray:
    """x_hat[t, h] = decode(codes[t, h]) * scales[t] (float64)."""
    return e4m3fn_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


# --------------------------------------------------------------------------
# Routing: softmax -> top-k -> normalise  ([NKI] Serving contract)
# --------------------------------------------------------------------------
def route_softmax_topk(logits, k: int):
    """ids int32 [T, k] and renormalised affinities float64 [T, k]."""
    l32 = np.asarray(logits, dtype=np.float32)
    T, E = l32.shape
    assert 1 <= k <= E
    l = l32.astype(np.float64)
    # softmax over all E experts
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    # top-k: order by (logit descending, expert index ascending) and keep k
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -l), axis=1)
    ids = order[:, :k].astype(np.int32)
    # normalise the k selected probabilities to sum to one
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    aff = sel / sel.sum(axis=1, keepdims=True)
    return ids, aff


# --------------------------------------------------------------------------
# Sigmoid routing  ([SPARK] module documentation: "sigmoid topK routing"; the
# routed weighted sum is scaled by the configuration's routed scaling factor)
# --------------------------------------------------------------------------
def route_sigmoid_topk(logits, k: int, normalize: bool = False, scale: float = 1.0):
    """ids int32 [T, k] and affinities float64 [T, k] of sigmoid routing.

    The kept experts are the k largest sigmoid scores sigma(l) = 1/(1+exp(-l));
    sigma is strictly increasing, so they are the k largest fp32 logits, ties
    to the lower expert index and -0.0 equal to +0.0, slot j the j-th.  The
    affinity is scale * sigma(l_j), or scale * sigma(l_j) / (sum of the k kept
    sigma) when ``normalize`` (the pages do not say whether the kept scores are
    renormalised; both readings are offered)."""
    l32 = np.asarray(logits, dtype=np.float32)
    T, E = l32.shape
    assert 1 <= k <= E
    l = l32.astype(np.float64)
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -l), axis=1)
    ids = order[:, :k].astype(np.int32)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-np.take_along_axis(l, ids.astype(np.int64), axis=1)))
    if normalize:
        sig = sig / sig.sum(axis=1, keepdims=True)
    return ids, float(scale) * sig


# --------------------------------------------------------------------------
# Router projection  ([SPARK] prefill forward: a batched gate GEMM takes the
# normalised hidden states [N, H] and the gate weights [E, H] to gate logits
# [N, E], which the top-K routing consumes; [NKILIB] Router Top-K: router
# logits, then top-K selection)
# --------------------------------------------------------------------------
def router_logits(x, wg):
    """logits[t, e] = sum over h of x[t, h] * wg[e, h], in float64.

    x is [T, H] and wg [E, H] (bf16 values given as float32/float64).  The
    router itself is route_softmax_topk on these logits; a device that sums in
    fp32 routes on its own fp32 logits, so the two agree exactly only where no
    two candidate logits lie within the fp32 summation error of each other."""
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(wg, dtype=np.float64)
    assert x.ndim == 2 and wg.ndim == 2 and x.shape[1] == wg.shape[1]
    return x @ wg.T


# --------------------------------------------------------------------------
# Sort by expert  ([SPARK] sorted prefill path; [AITER] inverse route map)
# --------------------------------------------------------------------------
def sort_by_expert(ids, E: int):
    """counts[E], offsets[E+1], sorted_route[R], inv_route[R] (all int32).

    Route r = t*k + j.  Expert e's segment is sorted_route[offsets[e]:offsets[e+1]]
    and holds, in ascending r, every route whose id is e; inv_route[r] is the
    position of route r in sorted_route."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    R = flat.size
    assert flat.size == 0 or (flat.min() >= 0 and flat.max() < E)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_route = np.argsort(flat, kind="stable")
    inv_route = np.empty(R, dtype=np.int64)
    inv_route[sorted_route] = np.arange(R)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_route.astype(np.int32), inv_route.astype(np.int32))


# --------------------------------------------------------------------------
# Expert FFN  ([NKI] fused path; [NEMO] _silu_mul / fused dense MLP)
# --------------------------------------------------------------------------
def swiglu(g, u):
    """silu(g) * u with silu(g) = g * sigmoid(g) = g / (1 + exp(-g))."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g)) * u


def relu2(u):
    """relu(u)^2 = max(u, 0)^2."""
    return np.maximum(u, 0.0) ** 2


def expert_mlp(xrows, w13, w13_scale, w2, w2_scale, activation="swiglu"):
    """One expert on rows of x (float64 [M, H]) -> float64 [M, H].

    SwiGLU: w13 [2I, H] (gate rows first, then up rows); relu2 ([SPARK] module
    documentation: up projection, then relu^2 and the down projection): w13
    [I, H] is the up projection alone.  w2 [H, I]; all block-scaled."""
    W13 = dequantize_blocks(w13, w13_scale)
    if activation == "relu2":
        a = relu2(xrows @ W13.T)
    else:
        I = W13.shape[0] // 2
        g = xrows @ W13[:I].T
        u = xrows @ W13[I:].T
        a = swiglu(g, u)
    W2 = dequantize_blocks(w2, w2_scale)
    return a @ W2.T


def moe_ffn(x, w13, w13_scale, w2, w2_scale, ids, aff, shared=None, activation="swiglu"):
    """out[t] = sum_j aff[t, j] * MLP_{ids[t, j]}(x[t]) (+ shared MLP(x[t])).

    x is [T, H] (bf16 values given as float32/float64), ids [T, k], aff [T, k].
    The routed terms are added expert by expert in ascending expert index, then
    the shared expert with affinity exactly 1."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    aff = np.asarray(aff, dtype=np.float64)
    T, H = x.shape
    out = np.zeros((T, H), dtype=np.float64)
    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        y = expert_mlp(x[t_idx], w13[e], w13_scale[e], w2[e], w2_scale[e], activation)
        np.add.at(out, t_idx, aff[t_idx, j_idx][:, None] * y)
    if shared is not None:
        out += expert_mlp(x, shared["w13"], shared["w13_scale"],
                          shared["w2"], shared["w2_scale"], activation)
    return out


def moe_forward(x, logits, k, w13, w13_scale, w2, w2_scale, shared=None):
    """Route then run the expert FFN: returns (ids, aff, out)."""
    ids, aff = route_softmax_topk(logits, k)
    out = moe_ffn(x, w13, w13_scale, w2, w2_scale, ids, aff, shared)
    return ids, aff, out
