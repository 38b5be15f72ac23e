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
    +-448; a row of zeros gets s = 0 and zero codes.  A row holding a NaN or
    an infinity (out of contract, but never made finite) gets a NaN scale and
    zero codes, so its x_hat is NaN.  Returns (codes uint8 [T, H], scales
    float32 [T]); the GEMM uses decode(code) * s."""
    x32 = np.asarray(x, dtype=np.float32)
    bad = ~np.all(np.isfinite(x32), axis=1)
    x32 = np.where(bad[:, None], np.float32(0.0), x32)
    amax = np.abs(x32).max(axis=1)
    s = (amax / np.float32(E4M3FN_MAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    v = (x32 / safe[:, None]).astype(np.float32)
    v = np.clip(v, -E4M3FN_MAX, E4M3FN_MAX)
    codes = e4m3fn_encode_rne(v)
    codes[s == 0] = 0
    s[bad] = np.float32(np.nan)
    return codes, s


def dequantize_rows(codes, scales) -> np.ndarray:
    """x_hat[t, h] = decode(codes[t, h]) * scales[t] (float64)."""
    return e4m3fn_decode(codes) * np.asarray(scales, dtype=np.float64)[:, None]


# --------------------------------------------------------------------------
# MXFP4 weights  ([AITER] description: the prefill pipeline's weights are
# MXFP4; [NKILIB] Blockwise MM Block MX: MXFP4/MXFP8 MoE).  The pages name the
# format without spelling it out; this follows the OCP Microscaling (MX)
# definition: FP4 E2M1 elements, one E8M0 scale per 32 consecutive elements.
# --------------------------------------------------------------------------
MX_BLOCK = 32


def _e2m1_value(code: int) -> float:
    """Value of one E2M1 code (4 bits): 1 sign bit, 2 exponent bits (bias 1),
    1 mantissa bit, subnormal at exponent 0, no infinities or NaN."""
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:                       # subnormal: 0.m * 2^(1-1)
        mag = m / 2.0
    else:                            # normal: 1.m * 2^(e-1)
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


def e2m1_table() -> np.ndarray:
    """The value of each of the 16 E2M1 codes, float64."""
    return np.array([_e2m1_value(c) for c in range(16)], dtype=np.float64)


_E2M1 = e2m1_table()


def e8m0_value(s) -> np.ndarray:
    """E8M0 scale bytes: 2^(s - 127) for s = 0..254; 255 is NaN."""
    s = np.asarray(s, dtype=np.int64)
    v = np.ldexp(1.0, s - 127)
    return np.where(s == 255, np.nan, v)


def unpack_fp4(packed) -> np.ndarray:
    """[..., C/2] bytes -> [..., C] E2M1 codes: element 2j is the low nibble of
    byte j and element 2j+1 its high nibble."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def dequantize_mx(packed, scales, block: int = MX_BLOCK) -> np.ndarray:
    """W[r, c] = E2M1(code[r, c]) * 2^(scales[r, c // 32] - 127) (float64).

    ``packed`` is [..., R, C/2] uint8 (two codes a byte), ``scales`` [..., R,
    C/32] uint8 E8M0."""
    vals = _E2M1[unpack_fp4(packed)]
    s = np.repeat(e8m0_value(scales), block, axis=-1)
    assert s.shape == vals.shape, (s.shape, vals.shape)
    return vals * s


def quantize_rows_mxfp4(x):
    """MXFP4 quantisation of activation rows (x of bf16 values, [T, H], H % 32
    == 0), by the OCP rule the synthetic MXFP4 weights use: each run of 32
    consecutive elements of a row shares the E8M0 exponent
    X = floor(log2(max |x|)) - 2, clamped to [-127, 127] (an all-zero run
    takes X = -127), so that the run's largest magnitude lands in [4, 8); each
    element becomes the E2M1 value nearest to |x| / 2^X, a tie going to the
    even code and magnitudes above 6 saturating to 6, with the sign bit of x
    (a negative element that rounds to 0 keeps its sign bit).  Every step is
    exact for bf16 inputs: the division is a power-of-two scaling and the
    rounding compares with the midpoints of the E2M1 grid.  A run holding a
    NaN or an infinity (out of contract, but never made finite) takes the
    E8M0 NaN byte 255 and zero codes, so its x_hat is NaN.

    Returns (codes uint8 [T, H/2], two a byte as the weights, scales uint8
    [T, H/32] E8M0); dequantize_mx of the pair gives x_hat."""
    xf = np.asarray(x, dtype=np.float64)
    T, H = xf.shape
    assert H % MX_BLOCK == 0, H
    blk = xf.reshape(T, H // MX_BLOCK, MX_BLOCK)
    bad = ~np.all(np.isfinite(blk), axis=2)
    blk = np.where(bad[..., None], 0.0, blk)
    amax = np.abs(blk).max(axis=2)
    _, e = np.frexp(amax)  # amax = m * 2^e with m in [0.5, 1): floor(log2 amax) = e - 1
    X = np.clip(np.where(amax > 0, e - 1 - 2, -127), -127, 127)
    v = np.abs(blk) / np.ldexp(1.0, X)[..., None]
    # the grid 0, 1/2, 1, 3/2, 2, 3, 4, 6: a code counts the midpoints below
    # |x| / 2^X; at a midpoint the even code wins, so 1/4, 5/4, 5/2 and 5 round
    # down and 3/4, 7/4 and 7/2 up
    mag = ((v > 0.25).astype(np.uint8) + (v >= 0.75) + (v > 1.25) + (v >= 1.75) +
           (v > 2.5) + (v >= 3.5) + (v > 5.0)).astype(np.uint8)
    codes = (mag | (np.signbit(blk).astype(np.uint8) << 3))
    codes[bad] = 0
    codes = codes.reshape(T, H)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, np.where(bad, 255, X + 127).astype(np.uint8)


def round_bf16(v) -> np.ndarray:
    """Each float64 value rounded once to the nearest bfloat16 value (8
    significant bits, exponent range of fp32, subnormals spaced 2^-133), ties
    to the even significand; NaN and infinities pass through, magnitudes that
    round past the largest bf16 value become infinities."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)  # v = m * 2^e, |m| in [0.5, 1)
    e = np.maximum(e, -125)  # below 2^-126 the grid is the subnormal spacing 2^-133
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)
        r = np.where(np.abs(r) > 3.3895313892515355e38, np.copysign(np.inf, v), r)
    return np.where(np.isfinite(v), r, v)


def quantize_hidden_mxfp4(a):
    """The hidden activation before the down GEMM when it runs on MXFP4
    activations: rows of float64 values (the SwiGLU or relu^2 output, [M, I])
    rounded to bf16 as every variant does before the down GEMM, then
    quantised by the MXFP4 activation rule of quantize_rows_mxfp4 (runs of 32
    along I).  Returns the dequantised float64 rows."""
    q, s = quantize_rows_mxfp4(round_bf16(a))
    return dequantize_mx(q, s)


def _e2m1_dequant_at(b, X):
    """b (float64) quantised to E2M1 at the E8M0 exponent X by the grid rule
    of quantize_rows_mxfp4 (nearest grid value of |b| / 2^X, ties to the even
    code, saturating at 6, sign kept), then dequantised."""
    sc = np.ldexp(1.0, X)
    v = np.abs(b) / sc
    mag = ((v > 0.25).astype(np.int64) + (v >= 0.75) + (v > 1.25) + (v >= 1.75) +
           (v > 2.5) + (v >= 3.5) + (v > 5.0))
    return np.copysign(_E2M1[mag] * sc, b)


def _mx_exponent(amax):
    """The run exponent of quantize_rows_mxfp4 for a largest magnitude amax."""
    _, e = np.frexp(amax)
    return np.clip(np.where(amax > 0, e - 1 - 2, -127), -127, 127)


def hidden_mxfp4_deviation(a, delta):
    """How far the quantised hidden activation can move when the value it is
    taken from is only known to within +-delta: an upper bound, per element,
    on |dq(b)_i - dq(bf16(a))_i| over bf16 vectors b whose element i lies in
    [bf16(a_i - delta_i), bf16(a_i + delta_i)] (bf16 rounding is monotone,
    so these are all the values the rounding can give), dq being
    quantize_rows_mxfp4 then dequantize_mx.  A run's exponent can then take
    any value between those of its smallest and largest possible maximum
    magnitude; at a fixed exponent the E2M1 value of an element is monotone
    in it, so the extremes sit at the ends of its interval.  The bound is the
    largest distance over those exponents and ends; it is exact when the
    exponent cannot move.  a, delta: float64 [M, I], delta >= 0; returns
    float64 [M, I].  A run holding a non-finite value quantises to NaN
    whatever its neighbours do (quantize_rows_mxfp4), so it gets no bound."""
    a = np.asarray(a, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.float64)
    M, I = a.shape
    delta = np.where(np.isnan(delta), 0.0, delta)
    assert I % MX_BLOCK == 0 and np.all(delta >= 0), (I,)
    nb = I // MX_BLOCK
    ref = quantize_hidden_mxfp4(a).reshape(M, nb, MX_BLOCK)
    lo = round_bf16(a - delta).reshape(M, nb, MX_BLOCK)
    hi = round_bf16(a + delta).reshape(M, nb, MX_BLOCK)
    least = np.where((lo <= 0) & (hi >= 0), 0.0, np.minimum(np.abs(lo), np.abs(hi)))
    most = np.maximum(np.abs(lo), np.abs(hi))
    X_lo = _mx_exponent(least.max(axis=2))[..., None]
    X_hi = _mx_exponent(most.max(axis=2))[..., None]
    moving = (X_hi > X_lo) | (hi > lo)
    dev = np.zeros_like(ref)
    for dx in range(int((X_hi - X_lo).max()) + 1 if M * nb else 0):
        X = np.minimum(X_lo + dx, X_hi)
        for b in (lo, hi):
            d = np.abs(_e2m1_dequant_at(b, X) - ref)
            dev = np.maximum(dev, np.where(moving, d, 0.0))
    return np.where(np.isfinite(ref), dev, 0.0).reshape(M, I)


def mx_gemm_error_bound(xrows, W, step: int = 64):
    """An upper bound on |fl32(xrows @ W.T) - xrows @ W.T| for a product of
    MXFP4 values (E2M1 codes times powers of two, on both sides) taken the
    way the scaled FP4 MFMA takes it: K in steps of 64, each step adding its
    two 32-element blocks to an fp32 accumulator.  A block's 32 products are
    multiples of one power of two (a quarter of the product of its two
    scales) of magnitude at most 32 * 36, so their sum is exact in fp32; a
    step then rounds at most twice in whatever order it adds its two block
    sums B0, B1 to the accumulator, each time by at most 2^-24 of the result.
    With S_j the exact running sum after step j, the error is at most
    2 * 2^-24 * sum_j (|S_j| + |S_{j-1}| + |B0_j| + |B1_j|) (the factor 2
    covering the second-order terms).  xrows [M, K], W [N, K] float64,
    K % 64 == 0; returns [M, N]."""
    xrows = np.asarray(xrows, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    M, K = xrows.shape
    assert K % step == 0 and W.shape[1] == K
    h = step // 2
    S = np.zeros((M, W.shape[0]))
    tot = np.zeros_like(S)
    for j in range(K // step):
        k0 = j * step
        B0 = xrows[:, k0:k0 + h] @ W[:, k0:k0 + h].T
        B1 = xrows[:, k0 + h:k0 + step] @ W[:, k0 + h:k0 + step].T
        Sn = S + B0 + B1
        tot += np.abs(Sn) + np.abs(S) + np.abs(B0) + np.abs(B1)
        S = Sn
    return 2.0 * 2.0 ** -24 * tot


def hidden_delta(g, u, eg, eu, activation: str = "swiglu"):
    """An upper bound on how far a kernel's fp32 hidden value can be from the
    exact one, used with hidden_mxfp4_deviation.  g, u: the exact gate and up
    sums (float64; g unused for relu^2), eg, eu: bounds on the fp32 error of
    those sums (mx_gemm_error_bound), all [M, I].  The kernel evaluates
    g / (1 + exp(-g)) * u in fp32 with an exponential whose argument error
    grows with |g|, within (8 + |g|) * 2^-22 of the value (and flushes it to
    zero below g = -80); relu^2 squares the rounded u.  The result is twice
    the first-order propagation of eg and eu, plus that evaluation error and
    2^-140."""
    u, eu = np.asarray(u, dtype=np.float64), np.asarray(eu, dtype=np.float64)
    if activation == "relu2":
        h = relu2(u)
        return 2.0 * (2.0 * np.maximum(u, 0.0) * eu + eu * eu) + 2.0 ** -20 * h + 2.0 ** -140
    g, eg = np.asarray(g, dtype=np.float64), np.asarray(eg, dtype=np.float64)
    h = np.abs(swiglu(g, u))
    rel = np.where(g > -80.0, (8.0 + np.abs(g)) * 2.0 ** -22, 1.0)
    return 2.0 * (1.1 * np.abs(u) * eg + np.abs(g) * eu + eg * eu) + rel * h + 2.0 ** -140


def dequantize_weights(codes, scales, weight_format: str = "e4m3_128") -> np.ndarray:
    """Dequantised float64 weights of either stored format: "e4m3_128"
    (E4M3FN codes, fp32 128x128 block scales) or "mxfp4" (E2M1 codes two a
    byte, E8M0 scales per 32 elements of a row)."""
    if weight_format == "mxfp4":
        return dequantize_mx(codes, scales)
    assert weight_format == "e4m3_128", weight_format
    return dequantize_blocks(codes, scales)


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


def expert_mlp(xrows, w13, w13_scale, w2, w2_scale, activation="swiglu",
               weight_format="e4m3_128", hidden="exact", bound=False):
    """One expert on rows of x (float64 [M, H]) -> float64 [M, H].

    SwiGLU: w13 [2I, H] (gate rows first, then up rows); relu2 ([SPARK] module
    documentation: up projection, then relu^2 and the down projection): w13
    [I, H] is the up projection alone.  w2 [H, I]; all block-scaled (see
    dequantize_weights for the two formats).

    hidden="mxfp4": the down GEMM takes the hidden activation quantised by
    quantize_hidden_mxfp4 ([AITER] description: the producer quantises the
    hidden activation to MXFP4 and runs the down projection in MXFP4).  With
    bound=True (x rows of MXFP4 values and MXFP4 weights, as on that path)
    also returns, per output element, an upper bound on how far a kernel that
    takes the same quantisation decision from fp32 sums can be from this
    result on that account: |W2| times hidden_mxfp4_deviation under
    hidden_delta of the gate/up sums' mx_gemm_error_bound."""
    W13 = dequantize_weights(w13, w13_scale, weight_format)
    if activation == "relu2":
        g = None
        u = xrows @ W13.T
        a = relu2(u)
    else:
        I = W13.shape[0] // 2
        g = xrows @ W13[:I].T
        u = xrows @ W13[I:].T
        a = swiglu(g, u)
    W2 = dequantize_weights(w2, w2_scale, weight_format)
    if hidden == "exact":
        assert not bound
        return a @ W2.T
    assert hidden == "mxfp4", hidden
    y = quantize_hidden_mxfp4(a) @ W2.T
    if not bound:
        return y
    if activation == "relu2":
        delta = hidden_delta(None, u, None, mx_gemm_error_bound(xrows, W13), "relu2")
    else:
        delta = hidden_delta(g, u, mx_gemm_error_bound(xrows, W13[:I]), mx_gemm_error_bound(xrows, W13[I:]))
    return y, hidden_mxfp4_deviation(a, delta) @ np.abs(W2).T


def moe_ffn(x, w13, w13_scale, w2, w2_scale, ids, aff, shared=None, activation="swiglu",
            weight_format="e4m3_128", hidden="exact", bound=False):
    """out[t] = sum_j aff[t, j] * MLP_{ids[t, j]}(x[t]) (+ shared MLP(x[t])).

    x is [T, H] (bf16 values given as float32/float64), ids [T, k], aff [T, k].
    The routed terms are added expert by expert in ascending expert index, then
    the shared expert with affinity exactly 1.  hidden and bound as in
    expert_mlp; with bound=True returns (out, bound) where bound[t] sums
    |aff[t, j]| times each route's bound."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    aff = np.asarray(aff, dtype=np.float64)
    T, H = x.shape
    out = np.zeros((T, H), dtype=np.float64)
    bnd = np.zeros((T, H), dtype=np.float64)

    def mlp(rows, w):
        r = expert_mlp(rows, *w, activation, weight_format, hidden, bound)
        return r if bound else (r, None)

    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        y, b = mlp(x[t_idx], (w13[e], w13_scale[e], w2[e], w2_scale[e]))
        np.add.at(out, t_idx, aff[t_idx, j_idx][:, None] * y)
        if bound:
            np.add.at(bnd, t_idx, np.abs(aff[t_idx, j_idx])[:, None] * b)
    if shared is not None:
        y, b = mlp(x, (shared["w13"], shared["w13_scale"], shared["w2"], shared["w2_scale"]))
        out += y
        if bound:
            bnd += b
    return (out, bnd) if bound else out


def moe_forward(x, logits, k, w13, w13_scale, w2, w2_scale, shared=None):
    """Route then run the expert FFN: returns (ids, aff, out)."""
    ids, aff = route_softmax_topk(logits, k)
    out = moe_ffn(x, w13, w13_scale, w2, w2_scale, ids, aff, shared)
    return ids, aff, out
