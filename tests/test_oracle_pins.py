"""Pins for the CPU oracle: each checks it against something other than itself.

* torch's own float8_e4m3fn conversion (an independent library routine),
* hand-derived closed forms stored under tests/golden/ with their citations,
* brute-force enumeration on tiny inputs,
* dense SwiGLU MLPs written with torch CPU fp64 library calls,
* invariants the method must satisfy (zero affinities, token permutation,
  linearity, sort-map structure).
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from block_scaled_fp8_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ----------------------------------------------------------------- MXFP4
def _e2m1_golden():
    out = {}
    for ln in _golden_lines("e2m1_values.txt"):
        code, val = ln.split()[:2]
        out[int(code, 16)] = float(val)
    return out


def test_e2m1_table_matches_hand_values():
    gold = _e2m1_golden()
    assert sorted(gold) == list(range(16))
    got = oracle.e2m1_table()
    for c, v in gold.items():
        assert got[c] == v and np.signbit(got[c]) == np.signbit(v), hex(c)


def test_e2m1_structure():
    t = oracle.e2m1_table()
    assert np.all(np.diff(t[:8]) > 0)               # magnitudes increase with the code
    assert np.array_equal(t[8:], -t[:8])            # the sign bit mirrors them
    # every value is exact in bf16 (8 significant bits) and in E4M3FN
    bf = torch.tensor(t, dtype=torch.float64).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf, t)
    f8 = torch.tensor(t, dtype=torch.float64).to(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(f8, t)


def test_e8m0_matches_torch_cast():
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_value(codes.numpy())
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_unpack_fp4_nibble_order():
    # byte j holds element 2j in its low nibble and 2j+1 in its high nibble
    packed = np.array([[0x71, 0x0F, 0xA3]], np.uint8)
    assert oracle.unpack_fp4(packed).tolist() == [[1, 7, 15, 0, 3, 10]]
    vals = oracle.dequantize_mx(np.tile(packed, (1, 32 // 3 + 1))[:, :16],
                                np.array([[127]], np.uint8))
    assert vals[0, :6].tolist() == [0.5, 6.0, -6.0, 0.0, 1.5, -1.0]


def test_dequantize_mx_block_indexing():
    # one scale byte 130 (x8) among 127s (x1): exactly that row's 32-element block scales
    R, C = 4, 128
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 256, (R, C // 2), dtype=np.uint8)
    sc = np.full((R, C // 32), 127, np.uint8)
    sc[2, 1] = 130
    got = oracle.dequantize_mx(packed, sc)
    g = _e2m1_golden()
    codes = np.empty((R, C), np.int64)
    codes[:, 0::2], codes[:, 1::2] = packed & 15, packed >> 4
    ref = np.vectorize(lambda c: g[c])(codes)
    ref[2, 32:64] *= 8.0
    assert np.array_equal(got, ref)


def test_mx_quantiser_round_trip():
    w = torch.randn(3, 64, 256, generator=torch.Generator().manual_seed(9)) * 0.02
    packed, sc = synth.quantize_mx(w)
    d = oracle.dequantize_mx(packed.numpy(), sc.numpy())
    step = np.repeat(oracle.e8m0_value(sc.numpy()), 32, -1)     # 2^X of each block
    q = w.double().numpy() / step
    # inside the E2M1 range the error is at most half a grid spacing (<= 1 unit
    # of 2^X between 4 and 6); beyond 6 the value saturates at 6
    inside = np.abs(q) <= 6
    assert np.all(np.abs(d - w.double().numpy())[inside] <= 1.0 * step[inside])
    assert np.all(np.abs(d[~inside]) == 6 * step[~inside])
    # values on the grid times a power of two come back exactly
    gridw = torch.tensor(oracle.e2m1_table()[[1, 2, 3, 4, 5, 6, 7, 9, 15]] * 2.0 ** -9,
                         dtype=torch.float32).repeat(1, 32)[:, :32 * 4].reshape(1, 1, -1)
    gridw[..., 0] = 6 * 2.0 ** -9          # every block holds the largest value
    gridw[..., 32] = gridw[..., 64] = gridw[..., 96] = 6 * 2.0 ** -9
    p2, s2 = synth.quantize_mx(gridw)
    assert np.array_equal(oracle.dequantize_mx(p2.numpy(), s2.numpy()), gridw.double().numpy())


def _mx_act_cases():
    out = []
    for ln in _golden_lines("mxfp4_rounding.txt"):
        v, code = ln.split()[:2]
        out.append((float(v), int(code, 16)))
    return out


@pytest.mark.parametrize("X", [-9, 0, 100, -120])
def test_mxfp4_activation_quantiser_hand_cases(X):
    """Each hand-worked case as element 1 of its own 32-element run whose
    element 0 is 4 * 2^X, so the run's exponent is X (a saturating case is
    itself the run's largest, still below 8 * 2^X)."""
    cases = _mx_act_cases()
    x = np.zeros((1, 32 * len(cases)))
    for i, (v, _) in enumerate(cases):
        x[0, 32 * i] = 4.0 * 2.0 ** X
        x[0, 32 * i + 1] = v * 2.0 ** X
    packed, sc = oracle.quantize_rows_mxfp4(x)
    codes = oracle.unpack_fp4(packed)[0]
    assert np.all(sc == X + 127)
    for i, (v, code) in enumerate(cases):
        assert codes[32 * i] == 0x6
        assert codes[32 * i + 1] == code, (v, codes[32 * i + 1], code)
        assert np.all(codes[32 * i + 2:32 * i + 32] == 0)


def test_mxfp4_activation_quantiser_zero_and_clamped_runs():
    """An all-zero run takes the byte 0 (X = -127) and zero codes; a run whose
    exponent would fall below -127 is clamped there (2^-126 / 2^-127 = 2)."""
    x = np.zeros((2, 64))
    x[1, 32] = 2.0 ** -126
    x[1, 33] = -(2.0 ** -127)
    packed, sc = oracle.quantize_rows_mxfp4(x)
    assert sc.tolist() == [[0, 0], [0, 0]]
    codes = oracle.unpack_fp4(packed)
    assert np.all(codes[0] == 0) and np.all(codes[1, :32] == 0)
    assert codes[1, 32] == 0x4 and codes[1, 33] == 0xA       # 2 and -1
    assert np.array_equal(oracle.dequantize_mx(packed, sc)[1, 32:34], x[1, 32:34])


def test_e4m3_row_quantiser_marks_non_finite_rows():
    """A row holding a NaN or an infinity gets a NaN scale and zero codes (its
    x_hat is NaN); the finite rows are quantised as before."""
    x = np.ones((3, 16), np.float32)
    x[0, 3] = np.nan
    x[2, 7] = -np.inf
    codes, s = oracle.quantize_rows_e4m3(x)
    assert np.isnan(s[0]) and np.isnan(s[2]) and s[1] == np.float32(1.0 / 448.0)
    assert np.all(codes[[0, 2]] == 0) and np.all(codes[1] == 0x7E)      # 448
    xh = oracle.dequantize_rows(codes, s)
    assert np.all(np.isnan(xh[[0, 2]])) and np.allclose(xh[1], 1.0, rtol=1e-6)


def test_mxfp4_activation_quantiser_marks_non_finite_runs():
    """A run holding a NaN or an infinity takes the E8M0 NaN byte 255 and zero
    codes (its x_hat is NaN); the other runs of the row are unaffected."""
    x = np.full((1, 96), 1.5)
    x[0, 3] = np.nan
    x[0, 40] = -np.inf
    packed, sc = oracle.quantize_rows_mxfp4(x)
    assert sc.tolist() == [[255, 255, 125]]
    codes = oracle.unpack_fp4(packed)[0]
    assert np.all(codes[:64] == 0) and np.all(codes[64:] == 0x7)   # 1.5 / 2^-2 = 6
    xh = oracle.dequantize_mx(packed, sc)[0]
    assert np.all(np.isnan(xh[:64])) and np.all(xh[64:] == 1.5)


def test_mxfp4_activation_quantiser_matches_brute_force():
    """Random bf16 rows, many of them on E2M1 midpoints: the exponent by a
    search over integers and each code by enumerating the 8 magnitudes
    (nearest, a tie to the even code) give the same bytes."""
    g = torch.Generator().manual_seed(21)
    base = torch.randn(3, 256, generator=g) * torch.tensor([1.0, 1e-3, 30.0])[:, None]
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])
    pick = mids[torch.randint(0, 8, (3, 256), generator=g)]
    sgn = torch.where(torch.rand(3, 256, generator=g) < 0.5, -1.0, 1.0)
    x = torch.where(torch.rand(3, 256, generator=g) < 0.4, pick * sgn * 2.0 ** -3, base)
    x[:, ::32] = 4.0 * 2.0 ** -3 * (torch.arange(3)[:, None] + 1)   # vary the runs' largest
    x[2, 64:96] = 0.0
    x = x.to(torch.bfloat16).double().numpy()
    packed, sc = oracle.quantize_rows_mxfp4(x)
    mags = oracle.e2m1_table()[:8]
    codes = oracle.unpack_fp4(packed)
    for t in range(x.shape[0]):
        for b in range(x.shape[1] // 32):
            run = x[t, 32 * b:32 * b + 32]
            amax = float(np.max(np.abs(run)))
            X = -127
            if amax > 0:
                k = -200
                while 2.0 ** (k + 1) <= amax:
                    k += 1
                X = max(-127, min(127, k - 2))
            assert sc[t, b] == X + 127
            for j, xv in enumerate(run):
                v = abs(xv) / 2.0 ** X
                d = np.abs(mags - v)
                best = [c for c in range(8) if d[c] == d.min()]
                c = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
                if np.signbit(xv):
                    c |= 8
                assert codes[t, 32 * b + j] == c, (t, b, j, xv)


def _torch_deq_mx(packed, sc):
    """MXFP4 dequantisation with the hand-worked E2M1 values and torch's
    float8_e8m0fnu cast (independent of the oracle's code)."""
    g = _e2m1_golden()
    lut = torch.tensor([g[c] for c in range(16)], dtype=torch.float64)
    p = torch.as_tensor(packed).to(torch.int64)
    codes = torch.stack([p & 15, p >> 4], dim=-1).flatten(-2)
    s = torch.as_tensor(sc).view(torch.float8_e8m0fnu).to(torch.float64)
    return lut[codes] * s.repeat_interleave(32, -1)


def test_ffn_mxfp4_single_expert_and_mixture_are_dense_mlps():
    E, T = 3, 5
    cfg = synth.MoeConfig("mx", T=T, H=256, I=128, E=E, k=1)
    c = synth.make_case(cfg, 12, weight_format="mxfp4")
    x = c["x"].float().numpy()
    w = {n: c[n].numpy() for n in ("w13", "w13_scale", "w2", "w2_scale")}
    xx = torch.as_tensor(x, dtype=torch.float64)

    def dense(e):
        W13 = _torch_deq_mx(c["w13"][e], c["w13_scale"][e])
        W2 = _torch_deq_mx(c["w2"][e], c["w2_scale"][e])
        I = W13.shape[0] // 2
        return (torch.nn.functional.silu(xx @ W13[:I].T) * (xx @ W13[I:].T)) @ W2.T

    got = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"],
                         np.full((T, 1), 1, np.int32), np.ones((T, 1)), weight_format="mxfp4")
    ref = dense(1).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    logits = c["logits"].numpy()
    ids, aff = oracle.route_softmax_topk(logits, E)
    got = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, aff,
                         weight_format="mxfp4")
    p = torch.softmax(torch.as_tensor(logits, dtype=torch.float64), dim=1)
    ref = sum(p[:, e:e + 1] * dense(e) for e in range(E)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


# ------------------------------------------------- MXFP4 hidden activation
def test_round_bf16_matches_torch_cast():
    """fp32 values (sweeps, exact ties between bf16 neighbours, subnormals,
    the largest finite values): one rounding to bf16 equals torch's
    float32 -> bfloat16 conversion."""
    g = torch.Generator().manual_seed(5)
    v = torch.cat([torch.randn(4000, generator=g) * 10.0 ** torch.randint(-30, 30, (4000,), generator=g),
                   torch.randn(500, generator=g) * 2.0 ** -130])
    bits = v.view(torch.int32)
    ties = ((bits & ~0xFFFF) | 0x8000).view(torch.float32)  # halfway between bf16 neighbours
    v = torch.cat([v, ties, torch.tensor([3.3895e38, -3.3895e38, 0.0, -0.0, 2.0 ** -133])])
    got = oracle.round_bf16(v.double().numpy())
    ref = v.to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(np.signbit(got), np.signbit(ref))


def test_hidden_quantiser_rounds_to_bf16_first():
    """1.25 + 2^-9 is bf16 1.25, an E2M1 tie at exponent 0 that goes to the
    even code (1.0); quantised directly it would be 1.5.  Worked by hand."""
    a = np.zeros((1, 32))
    a[0, 0] = 6.0
    a[0, 1] = 1.25 + 2.0 ** -9
    a[0, 2] = 2.25
    a[0, 3] = -0.3
    got = oracle.quantize_hidden_mxfp4(a)
    assert got[0, 0] == 6.0 and got[0, 1] == 1.0 and got[0, 2] == 2.0 and got[0, 3] == -0.5
    assert np.all(got[0, 4:] == 0.0)


def test_hidden_deviation_hand_cases():
    """Worked by hand.  (1) The tie above: within 2^-8 the bf16 value can
    also be 1.2578125, which rounds to 1.5, so only that element can move,
    by 0.5; within 2^-12 nothing can.  (2) A run whose largest element can be
    bf16 3.984375 (exponent -1: it saturates to 3.0, 1.0 stays 1.0, 0.30078125
    gives 0.25) or 4.0 (exponent 0: 4.0, 1.0 and 0.5): deviations 1, 0, 0.25."""
    a = np.zeros((1, 32))
    a[0, 0], a[0, 1] = 6.0, 1.25 + 2.0 ** -9
    d = np.zeros_like(a)
    d[0, 1] = 2.0 ** -8
    dev = oracle.hidden_mxfp4_deviation(a, d)
    assert dev[0, 1] == 0.5 and np.count_nonzero(dev) == 1
    d[0, 1] = 2.0 ** -12
    assert not np.any(oracle.hidden_mxfp4_deviation(a, d))
    a = np.zeros((1, 32))
    a[0, :3] = [3.99, 1.0, 0.3]
    d = np.zeros_like(a)
    d[0, 0] = 0.01
    dev = oracle.hidden_mxfp4_deviation(a, d)
    np.testing.assert_array_equal(dev[0, :3], [1.0, 0.0, 0.25])
    assert not np.any(dev[0, 3:])


def test_hidden_deviation_bounds_brute_force():
    """Random runs with a few elements near bf16 rounding points: enumerate
    every bf16 vector the intervals allow, quantise each with
    quantize_rows_mxfp4, and take the largest distance from the reference.
    The oracle's bound covers it, and equals it wherever the run's exponent
    was the same for every vector."""
    rng = np.random.default_rng(8)
    tab = oracle.e2m1_table()
    for trial in range(60):
        a = rng.standard_normal((1, 32)) * 2.0 ** rng.integers(-6, 6)
        a[0, rng.integers(0, 32)] *= 3.0
        if trial % 3 == 0:  # push some elements onto E2M1 ties of their run
            X = int(np.frexp(np.abs(a).max())[1]) - 3
            for i in rng.choice(32, 4, replace=False):
                a[0, i] = np.sign(a[0, i]) * rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * 2.0 ** X
        d = np.zeros_like(a)
        idx = rng.choice(32, 3, replace=False)
        d[0, idx] = np.abs(a[0, idx]) * 2.0 ** -8.5
        dev = oracle.hidden_mxfp4_deviation(a, d)[0]
        ref = oracle.quantize_hidden_mxfp4(a)[0]
        cands = []
        for i in range(32):
            lo = float(torch.tensor(a[0, i] - d[0, i]).float().to(torch.bfloat16).float())
            hi = float(torch.tensor(a[0, i] + d[0, i]).float().to(torch.bfloat16).float())
            vals = [lo]
            while vals[-1] < hi:  # the next bf16 value up, from its bit pattern
                bits = int(torch.tensor([vals[-1]]).to(torch.bfloat16).view(torch.int16)) & 0xFFFF
                bits = bits + 1 if vals[-1] > 0 or bits == 0 else (1 if bits == 0x8000 else bits - 1)
                nxt = torch.tensor([bits if bits < 0x8000 else bits - 0x10000],
                                   dtype=torch.int16).view(torch.bfloat16).float()
                vals.append(float(nxt))
            cands.append(vals)
        brute = np.zeros(32)
        exps = set()
        for vec in itertools.product(*cands):
            q, sc = oracle.quantize_rows_mxfp4(np.array([vec]))
            exps.add(int(sc[0, 0]))
            codes = oracle.unpack_fp4(q)[0]
            dq = tab[codes] * 2.0 ** (int(sc[0, 0]) - 127)
            brute = np.maximum(brute, np.abs(dq - ref))
        assert np.all(brute <= dev), trial
        if len(exps) == 1:
            np.testing.assert_array_equal(brute, dev)


def test_mx_gemm_error_bound_covers_simulated_fp32_steps():
    """mx_gemm_error_bound against a float32 simulation of the K loop it
    describes (each 32-element block summed exactly, then the two blocks of
    a 64-K step added to the accumulator in either order, every addition
    rounded to fp32): random MXFP4 operands with wide exponent spreads and
    near-cancelling rows stay within the bound."""
    rng = np.random.default_rng(3)
    tab = oracle.e2m1_table()
    for K in (64, 512, 2048):
        x = tab[rng.integers(0, 16, (6, K))] * 2.0 ** rng.integers(-20, 20, (6, K // 32)).repeat(32, 1)
        w = tab[rng.integers(0, 16, (5, K))] * 2.0 ** rng.integers(-20, 20, (5, K // 32)).repeat(32, 1)
        x[0] = -x[1]  # a row whose sums cancel against the next one's
        bound = oracle.mx_gemm_error_bound(x, w)
        exact = x @ w.T
        for order in (0, 1):
            acc = np.zeros((6, 5), np.float32)
            for j in range(K // 64):
                b0 = (x[:, 64 * j:64 * j + 32] @ w[:, 64 * j:64 * j + 32].T).astype(np.float32)
                b1 = (x[:, 64 * j + 32:64 * j + 64] @ w[:, 64 * j + 32:64 * j + 64].T).astype(np.float32)
                # the block sums are exact in fp32 (checked), the step rounds its additions
                assert np.array_equal(b0.astype(np.float64), x[:, 64 * j:64 * j + 32] @ w[:, 64 * j:64 * j + 32].T)
                acc = (acc + b0) + b1 if order == 0 else acc + (b0 + b1)
            assert np.all(np.abs(acc.astype(np.float64) - exact) <= bound), (K, order)


def test_ffn_hidden_mxfp4_one_hot_closed_form():
    """relu^2 expert with one-hot x rows and E2M1 weights of 1.0 and 1.5
    (scale byte 127): the up sums u are the weight values, relu(u)^2 is
    1 or 2.25, and a run holding 2.25 with largest value 2.25 takes exponent
    -1 (2.25 / 0.5 = 4.5 -> 4, i.e. 2.0) -- the down weights (identity)
    return the quantised hidden values themselves.  Worked by hand."""
    I = H = 64
    # up rows: row i reads x column i with weight 1.5 (i even) or 1.0 (i odd)
    codes = np.zeros((I, H), np.uint8)
    for i in range(I):
        codes[i, i] = 3 if i % 2 == 0 else 2   # E2M1 1.5 and 1.0
    w13 = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)[None]
    eye = np.zeros((H, I), np.uint8)
    eye[np.arange(H), np.arange(H)] = 2
    w2 = (eye[:, 0::2] | (eye[:, 1::2] << 4)).astype(np.uint8)[None]
    s13 = np.full((1, I, H // 32), 127, np.uint8)
    s2 = np.full((1, H, I // 32), 127, np.uint8)
    x = np.ones((1, H))
    y = oracle.moe_ffn(x, w13, s13, w2, s2, np.zeros((1, 1), np.int64), np.ones((1, 1)),
                       activation="relu2", weight_format="mxfp4", hidden="mxfp4")
    # relu(u)^2 = 2.25 (even i), 1.0 (odd i); run amax 2.25 -> X = -1: 2.25/0.5 = 4.5 -> 4
    # (midpoint 5 above), 1.0/0.5 = 2 -> 2
    want = np.where(np.arange(H) % 2 == 0, 2.0, 1.0)
    np.testing.assert_array_equal(y[0], want)
    y_exact = oracle.moe_ffn(x, w13, s13, w2, s2, np.zeros((1, 1), np.int64), np.ones((1, 1)),
                             activation="relu2", weight_format="mxfp4")
    np.testing.assert_array_equal(y_exact[0], np.where(np.arange(H) % 2 == 0, 2.25, 1.0))
    y2, b = oracle.moe_ffn(x, w13, s13, w2, s2, np.zeros((1, 1), np.int64), np.ones((1, 1)),
                           activation="relu2", weight_format="mxfp4", hidden="mxfp4", bound=True)
    np.testing.assert_array_equal(y2, y)
    assert not np.any(b)  # exact sums of one product: no element near a rounding point


# ----------------------------------------------------------------- E4M3FN
def test_e4m3fn_all_codes_match_torch_cast():
    codes = torch.arange(256, dtype=torch.int64).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_decode(codes.numpy())
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zero agree too
    assert np.signbit(got[0x80]) and not np.signbit(got[0x00])


def test_e4m3fn_spot_values():
    for ln in _golden_lines("e4m3fn_spot_values.txt"):
        code_s, val_s = ln.split()
        code, val = int(code_s, 16), float(val_s)
        got = oracle.e4m3fn_decode(np.array([code], np.uint8))[0]
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)


def test_e4m3fn_structure():
    t = oracle.e4m3fn_table()
    assert np.isfinite(t).sum() == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # 0x00..0x7E strictly increasing
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])   # sign bit mirrors
    assert t[0x7E] == oracle.E4M3FN_MAX == 448.0
    # every finite value is exactly representable in bf16
    fin = t[np.isfinite(t)]
    rt = torch.tensor(fin, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(rt, fin)


def test_dequant_block_indexing():
    rng = np.random.default_rng(0)
    R, C = 384, 256
    scales = (2.0 ** rng.integers(-6, 6, size=(R // 128, C // 128))).astype(np.float32)
    codes = np.full((R, C), 0x38, np.uint8)              # every code is 1.0
    got = oracle.dequantize_blocks(codes, scales)
    assert np.array_equal(got, np.kron(scales.astype(np.float64), np.ones((128, 128))))
    codes[5, 200] = 0x40                                  # one element is 2.0
    got = oracle.dequantize_blocks(codes, scales)
    assert got[5, 200] == 2.0 * scales[0, 1]


def test_quantiser_round_trip_bound():
    g = torch.Generator().manual_seed(3)
    w = torch.randn((2, 256, 384), generator=g) * 0.02
    w[1, :128, :128] = 0.0                                # an all-zero block
    codes, scales = synth.quantize_blocks(w)
    deq = oracle.dequantize_blocks(codes.numpy(), scales.numpy())
    wn = w.double().numpy()
    s = np.repeat(np.repeat(scales.double().numpy(), 128, -2), 128, -1)
    v = np.abs(wn) / np.where(s > 0, s, 1)
    # half an E4M3 spacing at the magnitude of w/s (2^-10 below the normal range)
    ulp = np.where(v >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(v, 1e-300))) - 3), 2.0 ** -9)
    assert np.all(np.abs(deq - wn) <= 0.5 * ulp * s * (1 + 1e-6) + 1e-30)
    assert np.all(deq[1, :128, :128] == 0.0)
    # the largest magnitude of each block lands on code +-448
    blk = np.abs(codes.numpy().reshape(2, 2, 128, 3, 128).astype(np.int64) & 0x7F)
    assert np.all((blk.max(axis=(2, 4)) == 0x7E) | (scales.numpy() == 0))


# ----------------------------------------------------------------- routing
def _brute_topk(row, k):
    """The unique ordered k-subset whose members all precede the others in
    (logit descending, index ascending); found by enumeration."""
    E = len(row)

    def before(a, b):
        return row[a] > row[b] or (row[a] == row[b] and a < b)

    found = []
    for sub in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in sub]
        if all(before(a, b) for a in sub for b in rest):
            found.append(sub)
    assert len(found) == 1
    sub = list(found[0])
    # order inside the subset
    out = []
    while sub:
        best = sub[0]
        for e in sub[1:]:
            if before(e, best):
                best = e
        out.append(best)
        sub.remove(best)
    return out


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(1)
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 1.0, 2.5], dtype=np.float32)
    for _ in range(300):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, min(E, 3) + 1))
        T = 3
        logits = rng.choice(vals, size=(T, E)).astype(np.float32)
        ids, aff = oracle.route_softmax_topk(logits, k)
        for t in range(T):
            assert list(ids[t]) == _brute_topk(list(logits[t]), k), (logits[t], k)


def test_route_golden_rows():
    for ln in _golden_lines("route_closed_form.txt"):
        k_s, l_s, i_s, a_s = [p.strip() for p in ln.split("|")]
        logits = np.array([[float(v) for v in l_s.split()]], dtype=np.float32)
        ids, aff = oracle.route_softmax_topk(logits, int(k_s))
        assert list(ids[0]) == [int(v) for v in i_s.split()]
        np.testing.assert_allclose(aff[0], [float(v) for v in a_s.split()], rtol=1e-14, atol=0)


# ------------------------------------------------- activation quantisation (E4M3)
def test_e4m3_encoder_matches_torch_cast_on_ties_and_sweeps():
    mags = oracle.e4m3fn_table()[:0x7F]
    mids = (mags[:-1] + mags[1:]) / 2             # every tie between neighbours
    rng = np.random.default_rng(21)
    vals = np.concatenate([mags, mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20),
                           rng.uniform(-448, 448, 200000), rng.standard_normal(50000) * 1e-2,
                           [0.0, -0.0, 448.0, -448.0, 2.0 ** -10, -(2.0 ** -10)]])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    vals = vals[np.abs(vals) <= 448]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_encode_rne(vals), ref)


def test_quantize_rows_matches_torch_and_closed_forms():
    x = torch.randn(64, 512, generator=torch.Generator().manual_seed(22)).to(torch.bfloat16).float()
    x[3] = 0.0
    x[5, :] = 0.0
    x[5, 17] = -3.0
    xn = x.numpy()
    codes, s = oracle.quantize_rows_e4m3(xn)
    # the same recipe through torch's own fp32 ops and E4M3 cast
    amax = x.abs().amax(dim=1)
    ts = amax / 448.0
    safe = torch.where(ts > 0, ts, torch.ones_like(ts))
    ref = (x / safe[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8)
    ref[ts == 0] = 0
    assert np.array_equal(s, ts.numpy()) and np.array_equal(codes, ref.numpy())
    # closed forms: the row maximum maps to +-448 (0x7E / 0xFE); a zero row to
    # scale 0 and code 0; row [1, -2, 0.5, 4]: x/s = 112, -224, 56, 448
    assert s[3] == 0 and np.all(codes[3] == 0)
    assert codes[5, 17] == 0xFE and np.all(np.delete(codes[5], 17) == 0)
    c4, s4 = oracle.quantize_rows_e4m3(np.array([[1.0, -2.0, 0.5, 4.0]], np.float32))
    assert c4.tolist() == [[0x6E, 0xF6, 0x66, 0x7E]] and s4[0] == np.float32(4.0) / np.float32(448)
    # dequantised values within half an E4M3 step (relative 2^-4) of x, plus the
    # subnormal step 2^-10 * s near zero
    xh = oracle.dequantize_rows(codes, s)
    err = np.abs(xh - xn.astype(np.float64))
    assert np.all(err <= 2.0 ** -4 * np.abs(xn) + 2.0 ** -10 * s[:, None] + 1e-30)


# ----------------------------------------------------------- sigmoid routing
def _sigmoid_golden_rows():
    rows = []
    for ln in _golden_lines("route_sigmoid_closed_form.txt"):
        k_s, n_s, sc_s, l_s, i_s, a_s = [p.strip() for p in ln.split("|")]
        rows.append((int(k_s), bool(int(n_s)), float(sc_s),
                     np.array([[float(v) for v in l_s.split()]], dtype=np.float32),
                     [int(v) for v in i_s.split()], [float(v) for v in a_s.split()]))
    return rows


def test_route_sigmoid_golden_rows():
    for k, norm, scale, logits, ids, aff in _sigmoid_golden_rows():
        i, a = oracle.route_sigmoid_topk(logits, k, norm, scale)
        assert list(i[0]) == ids
        np.testing.assert_allclose(a[0], aff, rtol=1e-14, atol=0)


def test_route_sigmoid_invariants():
    rng = np.random.default_rng(13)
    vals = np.array([-2.0, -0.0, 0.0, 0.5, 3.0], dtype=np.float32)
    logits = rng.choice(vals, size=(64, 9)).astype(np.float32)        # many ties
    logits[:8] = rng.standard_normal((8, 9)).astype(np.float32) * 4
    for k in (1, 3, 9):
        ids_s, _ = oracle.route_softmax_topk(logits, k)
        ids, aff = oracle.route_sigmoid_topk(logits, k)
        # the same experts as the softmax router: both keep the k largest logits
        assert np.array_equal(ids, ids_s)
        sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1)
        # sigma(0) = 1/2, and the scale multiplies exactly
        assert np.all((aff > 0) & (aff < 1))
        np.testing.assert_allclose(oracle.route_sigmoid_topk(logits, k, scale=3.0)[1], 3.0 * aff,
                                   rtol=1e-15)
        assert np.all(aff[sel == 0] == 0.5)
        # normalised: sums to the scale and keeps the ratios
        _, an = oracle.route_sigmoid_topk(logits, k, normalize=True, scale=0.75)
        np.testing.assert_allclose(an.sum(axis=1), 0.75, rtol=1e-14)
        np.testing.assert_allclose(an / an[:, :1], aff / aff[:, :1], rtol=1e-13)
    # sigma(l) + sigma(-l) = 1 on single experts
    l1 = np.array([[1.25], [-7.0], [0.0]], dtype=np.float32)
    np.testing.assert_allclose(oracle.route_sigmoid_topk(l1, 1)[1] + oracle.route_sigmoid_topk(-l1, 1)[1],
                               1.0, rtol=1e-15)


# ----------------------------------------------------------- router projection
def _proj_golden_rows():
    rows = []
    for ln in _golden_lines("router_proj_closed_form.txt"):
        w_s, k_s, x_s, l_s, i_s, a_s = [p.strip() for p in ln.split("|")]
        wg = np.array([[float(v) for v in r.split()] for r in w_s.split(";")])
        rows.append((wg, int(k_s), np.array([float(v) for v in x_s.split()]),
                     [float(v) for v in l_s.split()], [int(v) for v in i_s.split()],
                     [float(v) for v in a_s.split()]))
    return rows


def test_router_projection_golden_rows():
    for wg, k, x, logits, ids, aff in _proj_golden_rows():
        got = oracle.router_logits(x[None, :], wg)
        assert got[0].tolist() == logits
        i, a = oracle.route_softmax_topk(got, k)
        assert list(i[0]) == ids
        np.testing.assert_allclose(a[0], aff, rtol=1e-14, atol=0)


def test_router_projection_basis_rows_read_weight_columns():
    # x = the h-th unit vector selects column h of the gate weights: a
    # transposed or mis-indexed operand fails here (T != E != H)
    rng = np.random.default_rng(11)
    H, E = 7, 5
    wg = rng.standard_normal((E, H))
    got = oracle.router_logits(np.eye(H), wg)
    assert got.shape == (H, E)
    assert np.array_equal(got, wg.T)


def test_router_projection_brute_force_and_linearity():
    rng = np.random.default_rng(12)
    T, H, E = 3, 6, 4
    x = rng.integers(-3, 4, size=(T, H)).astype(np.float64)
    wg = rng.integers(-3, 4, size=(E, H)).astype(np.float64)
    got = oracle.router_logits(x, wg)
    for t in range(T):
        for e in range(E):
            assert got[t, e] == sum(int(x[t, h]) * int(wg[e, h]) for h in range(H))
    # linear in x
    x2 = rng.standard_normal((T, H))
    np.testing.assert_allclose(oracle.router_logits(2.5 * x - x2, wg),
                               2.5 * got - oracle.router_logits(x2, wg), rtol=1e-13, atol=1e-12)


def test_affinities_closed_forms():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((16, 12)).astype(np.float32)
    ids, aff = oracle.route_softmax_topk(logits, 4)
    np.testing.assert_allclose(aff.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # renormalised softmax == softmax over the selected logits alone
    sel = np.take_along_axis(logits.astype(np.float64), ids.astype(np.int64), axis=1)
    np.testing.assert_allclose(aff, scipy.special.softmax(sel, axis=1), rtol=1e-13)
    # k = E: the full softmax, in rank order
    ids_all, aff_all = oracle.route_softmax_topk(logits, 12)
    full = scipy.special.softmax(logits.astype(np.float64), axis=1)
    np.testing.assert_allclose(aff_all, np.take_along_axis(full, ids_all.astype(np.int64), 1),
                               rtol=1e-13)
    # slots are in descending logit order
    assert np.all(np.diff(np.take_along_axis(logits, ids_all.astype(np.int64), 1), axis=1) <= 0)


# ----------------------------------------------------------------- sort
def _brute_sort(flat, E):
    sorted_route = [r for e in range(E) for r in range(len(flat)) if flat[r] == e]
    counts = [sum(1 for v in flat if v == e) for e in range(E)]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    inv = [0] * len(flat)
    for p, r in enumerate(sorted_route):
        inv[r] = p
    return counts, offsets, sorted_route, inv


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (5, 2, 4), (13, 3, 7), (0, 2, 3), (40, 4, 9)])
def test_sort_brute_force(T, k, E):
    rng = np.random.default_rng(T * 100 + E)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    got = oracle.sort_by_expert(ids, E)
    exp = _brute_sort(list(ids.reshape(-1)), E)
    for g, e in zip(got, exp):
        assert list(g) == list(e)


def test_sort_invariants_large():
    rng = np.random.default_rng(7)
    T, k, E = 4096, 8, 256
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route_softmax_topk(logits, k)
    counts, offsets, sr, inv = oracle.sort_by_expert(ids, E)
    flat = ids.reshape(-1)
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
    assert np.all(np.diff(offsets) == counts)
    assert np.array_equal(np.sort(sr), np.arange(T * k))
    assert np.array_equal(inv[sr], np.arange(T * k))
    assert np.all(np.diff(flat[sr]) >= 0)
    for e in range(E):
        seg = sr[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)


# ----------------------------------------------------------------- FFN
def _torch_deq(codes, scales):
    c = torch.as_tensor(codes).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.as_tensor(scales).to(torch.float64)
    return c * s.repeat_interleave(128, -2).repeat_interleave(128, -1)


def _torch_mlp(x, w13, w13s, w2, w2s):
    """Dense SwiGLU MLP, torch CPU fp64: down(silu(gate x) * up x)."""
    W13 = _torch_deq(w13, w13s)
    I = W13.shape[0] // 2
    W1, W3 = W13[:I], W13[I:]
    W2 = _torch_deq(w2, w2s)
    xx = torch.as_tensor(x, dtype=torch.float64)
    return (torch.nn.functional.silu(xx @ W1.T) * (xx @ W3.T)) @ W2.T


def _small_case(E=4, T=6, H=256, I=128, seed=0, shared=False):
    cfg = synth.MoeConfig("t", T=T, H=H, I=I, E=E, k=1, shared=shared)
    c = synth.make_case(cfg, seed)
    np_w = {n: c[n].numpy() for n in ("w13", "w13_scale", "w2", "w2_scale")}
    sh = None
    if shared:
        sh = {n: c["shared"][n].numpy() for n in ("w13", "w13_scale", "w2", "w2_scale")}
    x = c["x"].float().numpy()
    return c, x, np_w, sh


def test_ffn_single_expert_is_dense_swiglu_mlp():
    c, x, w, _ = _small_case(E=1, T=7, H=384, I=256, seed=4)
    ids = np.zeros((7, 1), np.int32)
    aff = np.ones((7, 1))
    got = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, aff)
    ref = _torch_mlp(x, c["w13"][0], c["w13_scale"][0], c["w2"][0], c["w2_scale"][0]).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def _torch_mlp_relu2(x, w1, w1s, w2, w2s):
    """Dense non-gated MLP, torch CPU fp64: down(relu(up x)^2)."""
    W1 = _torch_deq(w1, w1s)
    W2 = _torch_deq(w2, w2s)
    xx = torch.as_tensor(x, dtype=torch.float64)
    return torch.nn.functional.relu(xx @ W1.T).square() @ W2.T


def test_ffn_relu2_single_expert_and_mixture_are_dense_mlps():
    cfg = synth.MoeConfig("t", T=7, H=384, I=256, E=3, k=1, shared=True)
    c = synth.make_case(cfg, 14, activation="relu2")
    assert tuple(c["w13"].shape) == (3, 256, 384)
    w = {n: c[n].numpy() for n in ("w13", "w13_scale", "w2", "w2_scale")}
    sh = {n: c["shared"][n].numpy() for n in ("w13", "w13_scale", "w2", "w2_scale")}
    x = c["x"].float().numpy()
    dense = [_torch_mlp_relu2(x, c["w13"][e], c["w13_scale"][e], c["w2"][e], c["w2_scale"][e])
             for e in range(3)]
    # one expert, affinity 1
    got = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"],
                         np.full((7, 1), 2, np.int32), np.ones((7, 1)), activation="relu2")
    ref = dense[2].numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # k = E: the softmax mixture, plus the shared expert's own MLP
    logits = c["logits"].numpy()
    ids, aff = oracle.route_softmax_topk(logits, 3)
    got = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, aff, sh,
                         activation="relu2")
    p = torch.softmax(torch.as_tensor(logits, dtype=torch.float64), dim=1)
    ref = (sum(p[:, e:e + 1] * dense[e] for e in range(3)) +
           _torch_mlp_relu2(x, c["shared"]["w13"], c["shared"]["w13_scale"], c["shared"]["w2"],
                            c["shared"]["w2_scale"])).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_ffn_relu2_closed_form():
    # Worked by hand.  H = 256, I = 128, one expert.  Up codes 0x38 (1.0) with
    # block scales 0.5 (rows 0..127, columns 0..127) and 4.0 (columns 128..255);
    # down codes 0x30 (0.5) with scales 2.0 (rows 0..127) and 0.25 (rows 128..255).
    #   token 0, x = e_3:     u_i = 0.5, a_i = 0.25, y_h = 128 * 0.25 * w2 =
    #                         32 (h < 128, w2 = 1) and 4 (h >= 128, w2 = 1/8);
    #   token 1, x = -e_200:  u_i = -4, a_i = relu(-4)^2 = 0, y = 0 exactly
    #                         (SwiGLU would not give 0 here);
    #   token 2, x = 2 e_0 - e_130: u_i = 2*0.5 - 4 = -3 -> 0.
    H, I = 256, 128
    w1 = np.full((1, I, H), 0x38, np.uint8)
    w1s = np.array([[[0.5, 4.0]]], np.float32)
    w2 = np.full((1, H, I), 0x30, np.uint8)
    w2s = np.array([[[2.0], [0.25]]], np.float32)
    x = np.zeros((3, H), np.float32)
    x[0, 3] = 1.0
    x[1, 200] = -1.0
    x[2, 0], x[2, 130] = 2.0, -1.0
    out = oracle.moe_ffn(x, w1, w1s, w2, w2s, np.zeros((3, 1), np.int32), np.ones((3, 1)),
                         activation="relu2")
    assert np.all(out[0, :128] == 32.0) and np.all(out[0, 128:] == 4.0)
    assert np.all(out[1:] == 0.0)
    assert oracle.relu2(np.array([-0.0, 0.0, -2.0, 3.0])).tolist() == [0.0, 0.0, 0.0, 9.0]


def test_ffn_all_experts_is_softmax_mixture():
    E, T = 4, 5
    c, x, w, _ = _small_case(E=E, T=T, seed=5)
    logits = c["logits"].numpy()
    ids, aff = oracle.route_softmax_topk(logits, E)
    got = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, aff)
    p = torch.softmax(torch.as_tensor(logits, dtype=torch.float64), dim=1)
    ref = sum(p[:, e:e + 1] * _torch_mlp(x, c["w13"][e], c["w13_scale"][e], c["w2"][e],
                                         c["w2_scale"][e]) for e in range(E)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_ffn_golden_closed_form():
    H, I = 256, 128
    w13 = np.zeros((2, 2 * I, H), np.uint8)
    w13[0, :I] = 0x38
    w13[0, I:] = 0x40
    w13[1] = 0xB8
    w13s = np.ones((2, 2, 2), np.float32)
    w13s[0] = [[0.5, 0.125], [0.25, 4.0]]
    w2 = np.zeros((2, H, I), np.uint8)
    w2[0] = 0x30
    w2[1] = 0x38
    w2s = np.ones((2, 2, 1), np.float32)
    w2s[0] = [[2.0], [0.5]]
    x = np.zeros((2, H), np.float32)
    x[0, 3] = 1.0
    x[1, 200] = -2.0
    logits = np.array([[3.0, 1.0], [2.0, -1.0]], np.float32)
    ids, aff, out = oracle.moe_forward(x, logits, 1, w13, w13s, w2, w2s)
    assert ids.tolist() == [[0], [0]] and aff.tolist() == [[1.0], [1.0]]
    for ln in _golden_lines("ffn_closed_form.txt"):
        t_s, lo_s, hi_s = [p.strip() for p in ln.split("|")]
        t = int(t_s)
        np.testing.assert_allclose(out[t, :128], float(lo_s), rtol=1e-14)
        np.testing.assert_allclose(out[t, 128:], float(hi_s), rtol=1e-14)


def test_ffn_zero_affinities_and_shared_expert():
    c, x, w, sh = _small_case(E=4, T=6, seed=6, shared=True)
    ids = synth.random_ids(6, 2, 4, 6).numpy()
    zero = np.zeros((6, 2))
    out = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, zero)
    assert np.all(out == 0.0)
    out_sh = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, zero, sh)
    ref = _torch_mlp(x, c["shared"]["w13"], c["shared"]["w13_scale"], c["shared"]["w2"],
                     c["shared"]["w2_scale"]).numpy()
    np.testing.assert_allclose(out_sh, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # shared expert adds exactly its own MLP on top of the routed sum
    aff = synth.random_affinities(6, 2, 6).numpy()
    r = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, aff)
    rs = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, aff, sh)
    np.testing.assert_allclose(rs - r, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_ffn_token_permutation_and_linearity():
    c, x, w, _ = _small_case(E=8, T=9, seed=8)
    logits = c["logits"].numpy()
    ids, aff, out = oracle.moe_forward(x, logits, 2, w["w13"], w["w13_scale"], w["w2"],
                                       w["w2_scale"])
    perm = np.random.default_rng(8).permutation(9)
    ids_p, aff_p, out_p = oracle.moe_forward(x[perm], logits[perm], 2, w["w13"],
                                             w["w13_scale"], w["w2"], w["w2_scale"])
    assert np.array_equal(ids_p, ids[perm])
    assert np.array_equal(aff_p, aff[perm])
    assert np.array_equal(out_p, out[perm])
    out2 = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, 2 * aff)
    assert np.array_equal(out2, 2 * out)
    # each route contributes aff * MLP_e(x): compare one token against torch
    t = 4
    ref = sum(aff[t, j] * _torch_mlp(x[t:t + 1], c["w13"][ids[t, j]], c["w13_scale"][ids[t, j]],
                                     c["w2"][ids[t, j]], c["w2_scale"][ids[t, j]]).numpy()[0]
              for j in range(2))
    np.testing.assert_allclose(out[t], ref, rtol=1e-11, atol=1e-12 * np.abs(ref).max())


def test_ffn_block_scale_is_local():
    """Doubling one down-projection block scale changes the output by exactly that
    block's contribution (powers of two keep it exact)."""
    c, x, w, _ = _small_case(E=1, T=3, H=256, I=256, seed=9)
    ids = np.zeros((3, 1), np.int32)
    aff = np.ones((3, 1))
    base = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], w["w2_scale"], ids, aff)
    s2 = w["w2_scale"].copy()
    s2[0, 1, 0] *= 2.0          # rows 128..255 of W2, K block 0
    bumped = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], s2, ids, aff)
    assert np.array_equal(bumped[:, :128], base[:, :128])
    only = np.zeros_like(s2)
    only[0, 1, 0] = w["w2_scale"][0, 1, 0]
    block = oracle.moe_ffn(x, w["w13"], w["w13_scale"], w["w2"], only, ids, aff)
    np.testing.assert_allclose(bumped - base, block, rtol=1e-12, atol=1e-12 * np.abs(base).max())
