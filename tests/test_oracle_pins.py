"""Pins of the CPU oracle to facts fixed outside it (no GPU).

Each test ties one oracle function to something other than its own formula:
a value a page prints, a closed form, an invariant, brute force on tiny inputs,
or a special case that reduces to a library routine.  Together they are
chosen so that a plausible slip (wrong rounding mode, multiply instead of
divide, /128 instead of /127, the smoothing vector applied to the wrong axis or
inverted, a dropped term in the epilogue, a transposed GEMM operand, outlier
columns counted in the per-token scale) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng0 = np.random.default_rng(1234)


# --------------------------------------------------------------------------
# fp16 <-> fp32 conversions: special case = numpy's IEEE conversions
# --------------------------------------------------------------------------

def test_half_to_float_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    ours = orc.half_to_float(h)
    ref = h.astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_float_to_half_matches_numpy_rne(orc):
    rng = np.random.default_rng(7)
    parts = [
        rng.standard_normal(200000).astype(np.float32) * np.float32(100),
        (rng.random(100000) * 7e-5).astype(np.float32),                    # binary16 subnormal range
        rng.uniform(60000, 70000, 20000).astype(np.float32),               # overflow edge
        rng.integers(0, 2**32, 200000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ]
    # exact ties: midpoints between neighbouring binary16 values
    h = np.arange(0, 0x7bff, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    parts += [mid, -mid, np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, np.inf, -np.inf],
                                  np.float32)]
    f = np.concatenate(parts)
    f = f[~np.isnan(f)]
    ours = orc.float_to_half(f)
    ref = f.astype(np.float16)
    assert np.array_equal(ours.view(np.uint16), ref.view(np.uint16))


# --------------------------------------------------------------------------
# Quantizer: the page's worked example, ties, bounds and invariants
# --------------------------------------------------------------------------

def test_worked_example_outlier_channel_scale(orc):
    """SmoothQuant page, section 1.2: one +-50 channel among [-1,1] values forces
    scale 50/127 ~ 0.39 and leaves the [-1,1] values 2-3 bits."""
    g = json.load(open(os.path.join(GOLDEN, "smoothquant_s12_outlier_channel.json")))
    rng = np.random.default_rng(0)
    x = rng.uniform(-1, 1, 64).astype(np.float32)
    x[:4] = [1.0, -1.0, 0.5, 0.25]
    x[37] = 50.0
    Xq, xs = orc.quantize_per_token(x[None, :])
    pv = g["page_values"]
    assert abs(float(xs[0]) - pv["scale_approx"]) < pv["scale_tolerance"]
    assert np.float32(xs[0]) == np.float32(g["derived_exact"]["scale_fp32"])
    for v, q in g["derived_exact"]["q_of"].items():
        row = np.zeros(64, np.float32)
        row[37] = 50.0
        row[0] = float(v)
        qq, _ = orc.quantize_per_token(row[None, :])
        assert int(qq[0, 0]) == q, v
    levels = np.unique(Xq[0][np.abs(x) <= 1.0])
    assert set(levels.tolist()) <= set(range(-3, 4))
    assert pv["bits_low"] <= math.log2(g["derived_exact"]["levels_in_unit_range"]) <= pv["bits_high"]


def test_ties_round_half_to_even(orc):
    """A row whose absmax is exactly 127 has scale 1.0, so x/scale = x exactly and
    the code is x rounded half to even (torch.round semantics)."""
    row = np.array([127.0, 2.5, 3.5, -2.5, -3.5, 0.5, 1.5, -0.5, 126.5, -126.5, 4.4999995, 0.0],
                   np.float32)
    Xq, xs = orc.quantize_per_token(row[None, :])
    assert xs[0] == np.float32(1.0)
    assert Xq[0].tolist() == [127, 2, 4, -2, -4, 0, 2, 0, 126, -126, 4, 0]


def _brute_code(v):
    """Nearest integer in [-128,127] by exhaustive search, ties to the even one."""
    best = None
    for q in range(-128, 128):
        d = abs(Fraction(float(v)) - q)
        if best is None or d < best[0] or (d == best[0] and q % 2 == 0):
            best = (d, q)
    return best[1]


def test_quantizer_brute_force_tiny(orc):
    rng = np.random.default_rng(3)
    X = (rng.standard_normal((6, 10)) * rng.uniform(0.01, 100, (6, 1))).astype(np.float32)
    X[2, 4] = X[2].max() * 1.5
    Xq, xs = orc.quantize_per_token(X)
    for m in range(6):
        a = max(abs(Fraction(float(v))) for v in X[m])
        # scale is the correctly rounded a/127 (a library division, numpy IEEE fp32)
        assert xs[m] == np.float32(np.float32(a) / np.float32(127.0))
        for j in range(10):
            v = np.float32(X[m, j]) / np.float32(xs[m])
            assert Xq[m, j] == _brute_code(v)


def test_roundtrip_error_bound_and_full_range(orc):
    """|x - q*scale| <= scale/2 (plus the rounding of x/scale) for every element,
    |q| <= 127, and every non-zero row reaches |q| = 127."""
    rng = np.random.default_rng(5)
    X = rng.standard_normal((64, 300)).astype(np.float32) * rng.uniform(1e-3, 1e3, (64, 1)).astype(np.float32)
    X[3] = 0.0
    Xq, xs = orc.quantize_per_token(X)
    err = np.abs(X.astype(np.float64) - Xq.astype(np.float64) * xs[:, None].astype(np.float64))
    assert np.all(err <= xs[:, None].astype(np.float64) * (0.5 + 1e-5))
    assert np.abs(Xq.astype(np.int32)).max() <= 127
    nz = np.any(X != 0, axis=1)
    assert np.all(np.abs(Xq[nz].astype(np.int32)).max(axis=1) == 127)
    assert xs[3] == 0 and np.all(Xq[3] == 0)


def test_scale_and_sign_invariance(orc):
    rng = np.random.default_rng(6)
    X = rng.standard_normal((32, 128)).astype(np.float32)
    Xq, xs = orc.quantize_per_token(X)
    for k in (-7, -1, 3, 11):
        Xq2, xs2 = orc.quantize_per_token(X * np.float32(2.0 ** k))
        assert np.array_equal(Xq, Xq2)
        assert np.array_equal(xs2, xs * np.float32(2.0 ** k))
    Xq3, xs3 = orc.quantize_per_token(-X)
    assert np.array_equal(Xq3, -Xq) and np.array_equal(xs3, xs)


def test_fp16_input_equals_widened_fp32(orc):
    X, _, _ = workloads.random_layer(11, 24, 256, 8, np.float16, n_outliers=3)
    a = orc.quantize_per_token(X)
    b = orc.quantize_per_token(X.astype(np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# --------------------------------------------------------------------------
# Weight quantization granularities
# --------------------------------------------------------------------------

def test_per_channel_weight_is_per_output_row(orc):
    """Each output channel (row of the [out, in] weight) gets its own absmax scale:
    the same computation as per-token quantization of those rows."""
    _, W, _ = workloads.random_layer(12, 1, 200, 48, np.float32)
    W[5] *= 40
    Wq, ws = orc.quantize_weight(W, None, 0)
    Wq2, ws2 = orc.quantize_per_token(W)
    assert np.array_equal(Wq, Wq2) and np.array_equal(ws, ws2)
    assert np.all(np.abs(Wq.astype(int)).max(axis=1) == 127)


def test_per_tensor_weight_is_one_row(orc):
    """Per-tensor quantization = one scale for the whole matrix: the special
    case of absmax quantization over one flattened row."""
    _, W, _ = workloads.random_layer(13, 1, 96, 40, np.float32)
    Wq, ws = orc.quantize_weight(W, None, 1)
    Wq1, ws1 = orc.quantize_per_token(W.reshape(1, -1))
    assert ws.shape == (1,) and ws[0] == ws1[0]
    assert np.array_equal(Wq.reshape(1, -1), Wq1)
    assert np.abs(Wq.astype(int)).max() == 127
    assert (np.abs(Wq.astype(int)).max(axis=1) < 127).sum() > 0


# --------------------------------------------------------------------------
# Smoothing factors (SmoothQuant page, sections 1.3, 2.1, 3.3)
# --------------------------------------------------------------------------

def _ulps(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b) / np.spacing(np.abs(b).astype(np.float32)).astype(np.float64)


def test_smooth_alpha_half_balances_maxima(orc):
    """alpha = 0.5: max|X'_j| = a_j/s_j and max|W'_j| = w_j*s_j both equal
    sqrt(a_j*w_j) -- the difficulty is split evenly."""
    X, W, _ = workloads.random_layer(21, 128, 256, 64, np.float32, n_outliers=4)
    amax, s = orc.smooth_scales(X, W, 0.5)
    a = np.abs(X).max(0).astype(np.float64)
    w = np.abs(W).max(0).astype(np.float64)
    assert np.array_equal(amax, np.abs(X).max(0))
    g = np.sqrt(a * w)
    assert np.all(_ulps(a / s.astype(np.float64), g) <= 2)
    assert np.all(_ulps(w * s.astype(np.float64), g) <= 2)


def test_smooth_alpha_extremes(orc):
    X, W, _ = workloads.random_layer(22, 64, 128, 32, np.float32, n_outliers=2)
    _, s1 = orc.smooth_scales(X, W, 1.0)
    assert np.array_equal(s1, np.abs(X).max(0))               # s = a: max|X'_j| = 1 exactly
    Xq, xs = orc.quantize_per_token(X, s1)
    Xs = X / s1                                               # numpy IEEE division
    assert np.all(np.abs(Xs).max(0) == 1.0)
    _, s0 = orc.smooth_scales(X, W, 0.0)
    w = np.abs(W).max(0).astype(np.float64)
    assert np.all(_ulps(w * s0.astype(np.float64), np.ones_like(w)) <= 1)   # max|W'_j| ~ 1


def test_smooth_floor_and_running_max(orc):
    X, W, _ = workloads.random_layer(23, 16, 32, 8, np.float32)
    X[:, 5] = 0.0
    W[:, 7] = 0.0
    amax, s = orc.smooth_scales(X, W, 0.5)
    w5 = float(np.abs(W[:, 5]).max())
    assert abs(float(s[5]) - math.sqrt(1e-8) / math.sqrt(w5)) <= 1e-6 * abs(float(s[5]))
    a7 = float(np.abs(X[:, 7]).max())
    assert abs(float(s[7]) - math.sqrt(a7) / math.sqrt(float(np.float32(1e-8)))) <= 1e-6 * float(s[7])
    # running maximum across calibration batches == maximum over the union
    amax2, _ = orc.smooth_scales(X[8:], W, 0.5, act_max=orc.smooth_scales(X[:8], W, 0.5)[0])
    assert np.array_equal(amax2, amax)


def test_smoothing_axis_and_direction_power_of_two(orc):
    """With s_j powers of two, X/s and W*s are exact, so smoothing inside the
    oracle must equal quantizing the numpy-scaled tensors: divides X's columns,
    multiplies W's columns (input channels), never rows."""
    X, W, _ = workloads.random_layer(24, 20, 64, 12, np.float32, n_outliers=3)
    s = (2.0 ** np.random.default_rng(0).integers(-6, 7, 64)).astype(np.float32)
    assert np.array_equal(orc.quantize_per_token(X, s)[0], orc.quantize_per_token(X / s)[0])
    for g in (0, 1):
        a, b = orc.quantize_weight(W, s, g), orc.quantize_weight(W * s, None, g)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_smoothing_identity_fp64():
    """(X diag(s)^-1)(diag(s) W) = X W exactly in exact arithmetic; in fp64 the
    difference is rounding only (SmoothQuant page, section 1.3)."""
    X, W, _ = workloads.random_layer(25, 32, 256, 48, np.float64, n_outliers=4)
    s = np.random.default_rng(1).uniform(0.01, 50, 256)
    ref = X @ W.T
    sm = (X / s) @ (W * s).T
    assert np.max(np.abs(sm - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_normalisation_is_invariant_power_of_two(orc):
    """Scaling s by a power of two (the optional s/max(s)*127 normalisation of the
    calibration sample, restricted to exact multipliers) changes no int8 code."""
    X, W, _ = workloads.random_layer(26, 24, 128, 16, np.float32, n_outliers=3)
    _, s = orc.smooth_scales(X, W, 0.5)
    c = np.float32(2.0 ** 5)
    for g in (0, 1):
        Wa, wa = orc.quantize_weight(W, s, g)
        Wb, wb = orc.quantize_weight(W, s * c, g)
        assert np.array_equal(Wa, Wb) and np.array_equal(wb, wa * c)
    Xa, xa = orc.quantize_per_token(X, s)
    Xb, xb = orc.quantize_per_token(X, s * c)
    assert np.array_equal(Xa, Xb) and np.array_equal(xb, xa / c)


# --------------------------------------------------------------------------
# int8 GEMM
# --------------------------------------------------------------------------

def test_gemm_brute_force_tiny(orc):
    rng = np.random.default_rng(31)
    for M, N, K in ((1, 1, 1), (3, 5, 7), (8, 4, 16), (5, 9, 33)):
        A = rng.integers(-128, 128, (M, K)).astype(np.int8)
        B = rng.integers(-128, 128, (N, K)).astype(np.int8)
        A[0, :] = -128
        B[0, :] = -128
        acc = orc.gemm_i8(A, B)
        for m in range(M):
            for n in range(N):
                assert acc[m, n] == sum(int(A[m, k]) * int(B[n, k]) for k in range(K))


def test_gemm_vs_fp64_blas_and_identity(orc):
    """fp64 matmul of int8-valued matrices is exact (partial sums < 2^53), an
    independent check at a larger size; Wq = 127 I gives acc = 127 Xq."""
    rng = np.random.default_rng(32)
    A = rng.integers(-127, 128, (70, 1040)).astype(np.int8)
    B = rng.integers(-127, 128, (90, 1040)).astype(np.int8)
    acc = orc.gemm_i8(A, B)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    assert np.array_equal(acc.astype(np.float64), ref)
    I = (np.eye(1040) * 127).astype(np.int8)
    assert np.array_equal(orc.gemm_i8(A, I), A.astype(np.int32) * 127)
    rows = rng.integers(0, 70, 500)
    cols = rng.integers(0, 90, 500)
    assert np.array_equal(orc.gemm_i8_sampled(A, B, rows, cols), acc[rows, cols])


def test_gemm_extreme_values_and_overflow_guard(orc):
    K = 20480
    A = np.full((2, K), 127, np.int8)
    B = np.full((2, K), -127, np.int8)
    assert np.all(orc.gemm_i8(A, B) == -127 * 127 * K)
    K = 133200                                                 # 127^2 * K > 2^31 - 1
    with pytest.raises(OverflowError):
        orc.gemm_i8(np.full((1, K), 127, np.int8), np.full((1, K), 127, np.int8))


# --------------------------------------------------------------------------
# Dequantization epilogue
# --------------------------------------------------------------------------

def test_dequant_closed_form(orc):
    rng = np.random.default_rng(41)
    acc = rng.integers(-2**23, 2**23, (8, 12)).astype(np.int32)
    xs = (2.0 ** rng.integers(-12, -4, 8)).astype(np.float32)       # exact products
    ws = (2.0 ** rng.integers(-10, -3, 12)).astype(np.float32)
    bias = (rng.integers(-64, 64, 12) / 8.0).astype(np.float32)
    y = orc.dequant(acc, xs, ws, 0, bias)
    for m in range(8):
        for n in range(12):
            ex = Fraction(int(acc[m, n])) * Fraction(float(xs[m])) * Fraction(float(ws[n])) + Fraction(float(bias[n]))
            assert Fraction(float(y[m, n])) == ex or abs(float(y[m, n]) - float(ex)) <= 2 ** -23 * abs(float(ex))
    yt = orc.dequant(acc, xs, ws[:1], 1, None)
    assert np.allclose(yt, acc.astype(np.float64) * xs[:, None] * float(ws[0]), rtol=0, atol=0)


def test_dequant_rounding_bound_general(orc):
    rng = np.random.default_rng(42)
    acc = rng.integers(-3 * 10**8, 3 * 10**8, (16, 16)).astype(np.int32)
    xs = rng.uniform(1e-4, 1e-1, 16).astype(np.float32)
    ws = rng.uniform(1e-5, 1e-2, 16).astype(np.float32)
    y = orc.dequant(acc, xs, ws, 0, None).astype(np.float64)
    ref = acc.astype(np.float64) * xs.astype(np.float64)[:, None] * ws.astype(np.float64)[None, :]
    assert np.all(np.abs(y - ref) <= 3 * 2.0 ** -24 * np.abs(ref))
    rows = rng.integers(0, 16, 40)
    cols = rng.integers(0, 16, 40)
    assert np.array_equal(orc.dequant_sampled(acc[rows, cols], xs, ws, 0, None, rows, cols),
                          orc.dequant(acc, xs, ws, 0, None)[rows, cols])


def test_half_store_is_numpy_rne(orc):
    y = np.random.default_rng(43).standard_normal(5000).astype(np.float32) * 30
    assert np.array_equal(orc.float_to_half(y).view(np.uint16), y.astype(np.float16).view(np.uint16))


# --------------------------------------------------------------------------
# Whole W8A8 layer: error bounded by the quantization steps
# --------------------------------------------------------------------------

def test_w8a8_layer_error_bound(orc):
    """|Y - X W^T| is bounded by the propagated quantization errors,
    sum_k (xs/2 |W'| + |X'| ws/2 + xs ws / 4); a smoothing applied to the wrong
    axis or a dequant missing a factor breaks it by orders of magnitude."""
    X, W, _ = workloads.random_layer(51, 32, 512, 64, np.float32, n_outliers=4)
    _, s = orc.smooth_scales(X, W, 0.5)
    Wq, ws = orc.quantize_weight(W, s, 0)
    _, xs, _, Y = orc.w8a8_linear(X, s, Wq, ws, 0, None, np.float32)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    Xs = X.astype(np.float64) / s
    Ws = W.astype(np.float64) * s
    xs64, ws64 = xs.astype(np.float64)[:, None], ws.astype(np.float64)[None, :]
    bound = (xs64 / 2) * np.abs(Ws).sum(1)[None, :] + np.abs(Xs).sum(1)[:, None] * (ws64 / 2) \
        + xs64 * ws64 / 4 * X.shape[1]
    assert np.all(np.abs(Y - ref) <= bound * 1.001 + 1e-6)
    snr = 10 * np.log10(np.var(ref) / np.var(Y - ref))
    assert snr > 20


# --------------------------------------------------------------------------
# LLM.int8() decomposition
# --------------------------------------------------------------------------

def _small_llm_case(seed=61, M=48, K=256, N=40, n_out=3):
    X, W, idx = workloads.random_layer(seed, M, K, N, np.float16, n_outliers=n_out, factor=20.0)
    return X, W, idx


def test_outlier_columns_are_numpy_column_max(orc):
    X, _, idx = _small_llm_case()
    mask, got = orc.outlier_columns(X, 6.0)
    ref = np.abs(X.astype(np.float32)).max(0) > 6.0
    assert np.array_equal(mask.astype(bool), ref)
    assert np.array_equal(got, np.nonzero(ref)[0])
    X2 = X.copy()
    X2[0, 0] = np.float16(6.0)                     # equal to the threshold: not an outlier
    X2[1:, 0] = 0
    assert orc.outlier_columns(X2, 6.0)[0][0] == 0


def test_llm_int8_no_outliers_reduces_to_w8a8(orc):
    X, W, _ = _small_llm_case()
    Wq, ws = orc.quantize_weight(W, None, 0)
    mask, idx, Xq, xs, acc, Y = orc.llm_int8_linear(X, W, Wq, ws, np.inf)
    assert idx.size == 0
    Xq2, xs2, acc2, Y2 = orc.w8a8_linear(X, None, Wq, ws, 0, None, np.float16)
    assert np.array_equal(Xq, Xq2) and np.array_equal(xs, xs2) and np.array_equal(acc, acc2)
    assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16))


def test_llm_int8_all_outliers_is_fp16_gemm(orc):
    X, W, _ = _small_llm_case()
    X = np.where(X == 0, np.float16(0.5), X)
    Wq, ws = orc.quantize_weight(W, None, 0)
    _, idx, Xq, xs, acc, Y = orc.llm_int8_linear(X, W, Wq, ws, 0.0)
    assert idx.size == X.shape[1]
    assert np.all(Xq == 0) and np.all(xs == 0) and np.all(acc == 0)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(Y.astype(np.float64), ref, rtol=1e-3, atol=1e-3 * np.abs(ref).mean())


def test_llm_int8_outlier_magnitude_does_not_touch_int8_part(orc):
    """The per-token scale is taken over normal columns only: scaling the outlier
    columns changes neither Xq nor x_scale, and the fp16 side product carries them."""
    X, W, idx = _small_llm_case()
    Wq, ws = orc.quantize_weight(W, None, 0)
    r1 = orc.llm_int8_linear(X, W, Wq, ws, 6.0)
    X2 = X.copy()
    X2[:, r1[1]] *= np.float16(2)
    r2 = orc.llm_int8_linear(X2, W, Wq, ws, 6.0)
    assert np.array_equal(r1[1], r2[1])
    assert np.array_equal(r1[2], r2[2]) and np.array_equal(r1[3], r2[3])
    assert np.all(r1[2][:, r1[1]] == 0)
    # decomposition = int8 part + exact side product over the listed columns
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    err = np.abs(r1[5].astype(np.float64) - ref)
    assert np.median(err / (np.abs(ref) + np.abs(ref).mean())) < 2e-2


def test_side_product_vs_numpy(orc):
    X, W, _ = _small_llm_case()
    idx = np.array([3, 17, 100, 255], np.int32)
    M, N = X.shape[0], W.shape[0]
    rr = np.repeat(np.arange(M), N)
    cc = np.tile(np.arange(N), M)
    side = orc.side_product_sampled(X, W, idx, rr, cc).reshape(M, N)
    ref = X[:, idx].astype(np.float64) @ W[:, idx].astype(np.float64).T
    assert np.allclose(side, ref, rtol=1e-14, atol=0)


def test_quantize_divides_by_scale(orc):
    """The basics notes and the SmoothQuant page divide by scale = max/127 (the
    LLM.int8() page's multiply-by-127/max form is not taken).  Rows built so that
    x/scale and x*(1/scale) round to different codes must follow the division
    (numpy IEEE fp32 division and rint, library routines)."""
    rng = np.random.default_rng(0)
    rows = []
    while len(rows) < 8:
        a = np.float32(rng.uniform(1, 100))
        sc = np.float32(a / np.float32(127))
        r = np.float32(np.float32(1) / sc)
        x = np.float32((rng.integers(-126, 126) + 0.5) * float(sc))
        for d in range(-3, 4):
            xx = x
            for _ in range(abs(d)):
                xx = np.nextafter(xx, np.float32(np.inf) if d > 0 else np.float32(-np.inf))
            if abs(xx) < a and np.rint(xx / sc) != np.rint(xx * r):
                rows.append((a, xx, np.rint(xx / sc)))
                break
    X = np.array([[a, xx] for a, xx, _ in rows], np.float32)
    Xq, xs = orc.quantize_per_token(X)
    assert Xq[:, 0].tolist() == [127] * len(rows)
    assert Xq[:, 1].tolist() == [int(q) for _, _, q in rows]


# --------------------------------------------------------------------------
# LayerNorm with the smoothing folded in, fused with per-token quantization
# ("SmoothQuant量化实战", sections 2.3, 4.2, 4.5).  Statistics are exact
# integer sums of binary16 values (the reading for this step).
# --------------------------------------------------------------------------

def _ln_rows(seed, M, K, scale=1.0):
    r = np.random.default_rng(seed)
    X = (r.standard_normal((M, K)) * scale + r.standard_normal((M, 1)) * scale).astype(np.float16)
    return X


def test_layernorm_stats_vs_exact_rationals(orc):
    """mu and the population variance against exact rational arithmetic with the
    two-pass definition sum((x - mean)^2) / K (not the oracle's K*S2 - S1^2)."""
    X = _ln_rows(11, 24, 48, scale=3.0)
    X[0] = np.float16(65504.0) * np.sign(X[0]).astype(np.float16)     # extreme magnitudes
    X[1, ::2] = np.float16(6e-8)                                        # subnormals
    X[2] = np.float16(-0.0)
    _, _, mu64, var64 = orc.layernorm_stats(X, 1e-5)
    for m in range(X.shape[0]):
        xs = [Fraction(float(v)) for v in X[m].astype(np.float64)]
        mu = sum(xs) / len(xs)
        var = sum((x - mu) ** 2 for x in xs) / len(xs)
        assert mu64[m] == float(mu) or abs(mu64[m] - float(mu)) <= math.ulp(float(mu)), m
        assert abs(var64[m] - float(var)) <= 2 * math.ulp(float(var)) + 0.0, m
    # small integer-valued rows: the sums stay below 2^53, so the definition is the
    # correctly rounded exact value
    Xs = np.array([[1, 2, 3, 4, 5, 6, 7, 9], [0.5, -0.25, 8, 8, 8, 8, -3, 1]], np.float16)
    _, _, mu64, var64 = orc.layernorm_stats(Xs, 0.0)
    for m in range(2):
        xs = [Fraction(float(v)) for v in Xs[m].astype(np.float64)]
        mu = sum(xs) / 8
        assert mu64[m] == float(mu)
        assert var64[m] == float(sum((x - mu) ** 2 for x in xs) / 8)


def test_layernorm_vs_torch_fp64(orc):
    """The normalised, scaled and shifted output against torch's layer_norm in fp64:
    biased variance, eps inside the square root, y = z * gamma + beta."""
    torch = pytest.importorskip("torch")
    M, K = 64, 1040
    X = _ln_rows(12, M, K, scale=2.0)
    r = np.random.default_rng(13)
    g = r.uniform(0.2, 3.0, K).astype(np.float32)
    b = r.standard_normal(K).astype(np.float32)
    eps = 1e-5
    y = orc.layernorm(X, g, b, eps)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(X.astype(np.float64)), (K,),
                                         weight=torch.from_numpy(g.astype(np.float64)),
                                         bias=torch.from_numpy(b.astype(np.float64)), eps=eps).numpy()
    err = np.abs(y.astype(np.float64) - ref)
    assert err.max() <= 1e-5 * np.abs(ref).max(), err.max()
    # without beta: no shift at all
    y0 = orc.layernorm(X, g, None, eps)
    assert np.array_equal(y0 + b, y)  # fl32(z*g) + b is exactly the with-beta result


def test_layernorm_special_rows(orc):
    K = 64
    X = np.zeros((4, K), np.float16)
    X[0] = np.float16(3.5)                       # constant row: var = 0
    X[1, ::2], X[1, 1::2] = np.float16(-2.0), np.float16(2.0)   # mean 0, var 4
    X[2] = np.float16(0.0)                       # zero row
    X[3, :4] = np.array([1, 2, 3, 4], np.float16)
    eps = 1e-5
    e64 = float(np.float32(eps))                 # the entry point takes eps as binary32
    mu32, r32, mu64, var64 = orc.layernorm_stats(X, eps)
    assert mu64[0] == 3.5 and var64[0] == 0.0 and r32[0] == np.float32(1.0 / math.sqrt(e64))
    assert mu64[1] == 0.0 and var64[1] == 4.0 and r32[1] == np.float32(1.0 / math.sqrt(4.0 + e64))
    assert mu64[2] == 0.0 and var64[2] == 0.0
    b = np.linspace(-1, 1, K).astype(np.float32)
    y = orc.layernorm(X, np.full(K, 1.5, np.float32), b, eps)
    assert np.array_equal(y[0], b) and np.array_equal(y[2], b)      # z == 0 exactly
    # hand-worked: [1,2,3,4] over K = 4 has mean 2.5 and variance 1.25
    X4 = np.array([[1, 2, 3, 4]], np.float16)
    mu32, r32, mu64, var64 = orc.layernorm_stats(X4, eps)
    assert mu64[0] == 2.5 and var64[0] == 1.25
    q, xs = orc.layernorm_quantize(X4, np.ones(4, np.float32), None, eps)
    z = np.float32(1.5) * np.float32(1.0 / math.sqrt(1.25 + e64))
    assert xs[0] == np.float32(z / np.float32(127.0))
    assert q.tolist() == [[-127, -42, 42, 127]]       # 0.5/1.5 * 127 = 42.33
    # zero row without beta: scale 0, codes 0
    q, xs = orc.layernorm_quantize(X[2:3], np.ones(K, np.float32), None, eps)
    assert xs[0] == 0.0 and not q.any()


def test_fold_layernorm_direction_and_axis(orc):
    """LayerNorm with gamma/s, beta/s equals LayerNorm followed by X / s: bit-exact for
    power-of-two s (every division exact), close for general s."""
    M, K = 16, 256
    X = _ln_rows(14, M, K)
    r = np.random.default_rng(15)
    g = r.uniform(0.5, 2.0, K).astype(np.float32)
    b = r.standard_normal(K).astype(np.float32)
    s2 = np.exp2(r.integers(-6, 7, K)).astype(np.float32)
    g2, b2 = orc.fold_layernorm(g, b, s2)
    assert np.array_equal(g2, g / s2) and np.array_equal(b2, b / s2)
    y = orc.layernorm(X, g, b, 1e-5)
    assert np.array_equal(orc.layernorm(X, g2, b2, 1e-5), y / s2[None, :])
    s = r.uniform(0.05, 20.0, K).astype(np.float32)
    gs, bs = orc.fold_layernorm(g, b, s)
    ys = orc.layernorm(X, gs, bs, 1e-5).astype(np.float64)
    ref = y.astype(np.float64) / s[None, :]
    assert np.abs(ys - ref).max() <= 4 * np.finfo(np.float32).eps * np.abs(ref).max()
    gn, bn = orc.fold_layernorm(g, None, s)
    assert bn is None and np.array_equal(gn, gs)


def test_layernorm_quantize_invariants(orc):
    """Every non-zero row reaches |q| = 127, and |y - q*xs| <= xs/2 elementwise."""
    M, K = 48, 4112
    X = _ln_rows(16, M, K, scale=4.0)
    r = np.random.default_rng(17)
    g = r.uniform(0.1, 5.0, K).astype(np.float32)
    b = (r.standard_normal(K) * 0.1).astype(np.float32)
    q, xs = orc.layernorm_quantize(X, g, b, 1e-5)
    y = orc.layernorm(X, g, b, 1e-5).astype(np.float64)
    assert np.all(np.abs(q).max(axis=1) == 127)
    assert np.all(xs == (np.abs(y).max(axis=1) / 127.0).astype(np.float32)) or \
        np.all(xs == (np.abs(y).max(axis=1).astype(np.float32) / np.float32(127.0)))
    err = np.abs(y - q.astype(np.float64) * xs[:, None].astype(np.float64))
    assert np.all(err <= xs[:, None].astype(np.float64) * (0.5 + 1e-6))


def test_layernorm_workload_shape_vs_fp64(orc):
    """The C2 activation shape (2048 x 4096 fp16, outlier channels), fold with a
    real smoothing vector, against fp64 within the fp32 error of the steps."""
    torch = pytest.importorskip("torch")
    wl = workloads.prefill_7b(which=("qkv",))
    X = wl.X[:256]
    K = X.shape[1]
    r = np.random.default_rng(18)
    g = r.uniform(0.5, 1.5, K).astype(np.float32)
    b = (r.standard_normal(K) * 0.05).astype(np.float32)
    s = r.uniform(0.2, 8.0, K).astype(np.float32)
    gs, bs = orc.fold_layernorm(g, b, s)
    y = orc.layernorm(X, gs, bs, 1e-5).astype(np.float64)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(X.astype(np.float64)), (K,),
                                         weight=torch.from_numpy(g.astype(np.float64)),
                                         bias=torch.from_numpy(b.astype(np.float64)), eps=1e-5).numpy() / s
    assert np.abs(y - ref).max() <= 1e-5 * np.abs(ref).max()


# --------------------------------------------------------------------------
# Static per-tensor activation scale (basics notes, 静态量化; the percentile
# calibrator of the deployment page).  Nearest-rank percentile of |x'|.
# --------------------------------------------------------------------------

def test_percentile_is_numpy_inverted_cdf(orc):
    """The nearest-rank percentile is numpy's 'inverted_cdf' method; p = 100 is the max."""
    r = np.random.default_rng(31)
    X = (r.standard_normal((96, 160)) * 3).astype(np.float16)
    X[:, 5] = np.float16(7.0)                                  # many ties
    s = r.uniform(0.2, 5.0, 160).astype(np.float32)
    for sv in (None, s):
        a = np.abs(X.astype(np.float32) if sv is None else X.astype(np.float32) / sv[None, :]).ravel()
        for p in (0.5, 10.0, 50.0, 90.0, 99.0, 99.9, 99.99, 100.0):
            ref = np.percentile(a, p, method="inverted_cdf")
            assert orc.abs_percentile(X, sv, p) == np.float32(ref), (p, sv is None)
        assert orc.abs_percentile(X, sv, 100.0) == a.max()
    assert orc.percentile_rank(10, 100.0) == 10 and orc.percentile_rank(10, 0.001) == 1
    assert orc.percentile_rank(10000, 99.99) == 9999


def test_static_scale_closed_form(orc):
    X = np.arange(1, 101, dtype=np.float32).reshape(10, 10)
    assert orc.abs_percentile(X, None, 50.0) == 50.0
    assert orc.abs_percentile(X, None, 99.0) == 99.0
    assert orc.static_scale(X, None, 100.0) == np.float32(np.float32(100.0) / np.float32(127.0))
    assert orc.static_scale(np.zeros((3, 16), np.float32), None, 99.9) == 0.0


def test_static_quantize_with_row_scale_is_per_token(orc):
    """Quantizing a row with its own dynamic scale as the static one reproduces the
    (pinned) per-token quantizer exactly, with and without smoothing."""
    r = np.random.default_rng(32)
    X = (r.standard_normal((12, 272)) * 5).astype(np.float16)
    s = r.uniform(0.1, 9.0, 272).astype(np.float32)
    for sv in (None, s):
        q_dyn, xs_dyn = orc.quantize_per_token(X, sv)
        for m in range(X.shape[0]):
            q = orc.quantize_static(X[m:m + 1], sv, xs_dyn[m])
            assert np.array_equal(q[0], q_dyn[m])


def test_static_quantize_saturates_and_bounds(orc):
    """Beyond the calibrated threshold codes saturate at 127 / -128; inside it the
    round trip is within half a step."""
    r = np.random.default_rng(33)
    X = (r.standard_normal((64, 512)) * 2).astype(np.float32)
    xs = orc.static_scale(X, None, 99.0)
    T = xs * np.float32(127.0)
    q = orc.quantize_static(X, None, xs)
    big = X > T * 1.01
    assert big.any() and np.all(q[big] == 127)
    neg = X < -T * 1.02
    assert neg.any() and np.all(q[neg] <= -127)
    assert np.all(q[X <= -T * 128.6 / 127.0] == -128)
    inside = np.abs(X) <= T
    err = np.abs(X[inside].astype(np.float64) - q[inside].astype(np.float64) * float(xs))
    assert err.max() <= float(xs) * (0.5 + 1e-6)


# --------------------------------------------------------------------------
# INT8 KV cache with per-head scales ("SmoothQuant量化实战", section 5.2)
# --------------------------------------------------------------------------

def _kv(seed, T, H, D, dt=np.float16):
    r = np.random.default_rng(seed)
    KV = r.standard_normal((T, H, D)) * r.uniform(0.2, 8.0, (1, H, 1))    # heads differ in range
    return KV.astype(dt)


def test_kv_calibration_is_numpy_head_max(orc):
    KV = _kv(41, 64, 8, 128)
    for margin in (1.0, 1.25):
        ref = (np.float32(margin) * np.abs(KV.astype(np.float32)).max(axis=(0, 2))) / np.float32(127.0)
        assert np.array_equal(orc.kv_calibrate_per_head(KV, margin), ref.astype(np.float32))
    assert not orc.kv_calibrate_per_head(np.zeros((4, 2, 16), np.float16)).any()


def test_kv_per_head_is_static_quantization_per_head(orc):
    """Each head is quantized exactly like a static per-tensor quantization of its
    own [T x D] slice with its own scale (the pinned N3 quantizer)."""
    T, H, D = 40, 4, 64
    KV = _kv(42, T, H, D)
    sc = orc.kv_calibrate_per_head(KV[: T // 2], 1.0)                     # later tokens can saturate
    q = orc.kv_quantize_per_head(KV, sc)
    for h in range(H):
        assert np.array_equal(q[:, h, :], orc.quantize_static(KV[:, h, :], None, sc[h]))
    assert np.abs(q.astype(np.int32)).max() >= 127


def test_dequantize_closed_form_and_round_trip(orc):
    T, H, D = 32, 4, 64
    KV = _kv(43, T, H, D, np.float32)
    sc = orc.kv_calibrate_per_head(KV, 1.0)
    q = orc.kv_quantize_per_head(KV, sc)
    y = orc.dequantize(q.reshape(T, H * D), sc, 0, D).reshape(T, H, D)
    assert np.array_equal(y, q.astype(np.float32) * sc[None, :, None])    # one fp32 product
    err = np.abs(KV.astype(np.float64) - y.astype(np.float64))
    assert np.all(err <= sc[None, :, None].astype(np.float64) * (0.5 + 1e-6))
    # power-of-two scales: exact
    s2 = np.exp2(np.arange(-3, 1)).astype(np.float32)
    y2 = orc.dequantize(q.reshape(T, H * D), s2, 0, D).reshape(T, H, D)
    assert np.array_equal(y2, q.astype(np.float32) * s2[None, :, None])
    # per-token-per-head (dynamic) scales: rows of D with the per-token quantizer, row-indexed dequant
    qd, xs = orc.quantize_per_token(KV.reshape(T * H, D), None)
    yd = orc.dequantize(qd, xs, 1, D)
    assert np.all(np.abs(KV.reshape(T * H, D) - yd) <= xs[:, None] * (0.5 + 1e-6))


# --------------------------------------------------------------------------
# FP8 E4M3 W8A8 variant (SmoothQuant page, section 6.1)
# --------------------------------------------------------------------------
def _torch_e4m3(v):
    import torch
    return torch.from_numpy(np.ascontiguousarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_decode_closed_form_and_torch(orc):
    """All 256 codes: (-1)^s 2^(E-7) (1 + m/8), subnormals m 2^-9, NaN at S.1111.111;
    and torch's float8_e4m3fn widening agrees."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    d = orc.fp8_decode(codes)
    for c in range(256):
        s, E, m = c >> 7, (c >> 3) & 15, c & 7
        if E == 15 and m == 7:
            assert np.isnan(d[c])
            continue
        v = Fraction(m, 512) if E == 0 else Fraction(8 + m, 8) * Fraction(2) ** (E - 7)
        assert Fraction(float(d[c])) == (-v if s else v), c
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    ok = np.isnan(t) & np.isnan(d) | (t == d)
    assert ok.all()
    assert d[0x7E] == 448.0 and d[0x01] == 2.0 ** -9 and d[0x08] == 2.0 ** -6


def test_fp8_encode_rne_against_torch(orc):
    """Nearest-even rounding: random values, every midpoint between adjacent codes,
    and the floats just beside each midpoint, against torch's conversion."""
    vals = orc.fp8_decode(np.arange(0, 0x7F, dtype=np.uint8)).astype(np.float64)   # 0 .. 448, ascending
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)                          # exact in fp32
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1000))])
    r = np.random.default_rng(61)
    rnd = (r.uniform(-1, 1, 200000) * np.exp2(r.uniform(-14, 8.8, 200000))).astype(np.float32)
    x = np.concatenate([near, -near, rnd, np.float32([0.0, -0.0, 448.0, -448.0, 2.0 ** -10, 2.0 ** -12])])
    x = np.clip(x, -448, 448)
    assert np.array_equal(orc.fp8_encode(x), _torch_e4m3(x))
    # ties go to the even mantissa: 1 + 1/16 -> 1.0, 1 + 3/16 -> 1.25, 1.5 * 2^-9 -> 2^-8
    assert list(orc.fp8_decode(orc.fp8_encode(np.float32([1.0625, 1.1875, 1.5 * 2 ** -9])))) == [1.0, 1.25, 2 ** -8]
    assert orc.fp8_encode(np.float32([1e6]))[0] == 0x7E                           # saturates (the clamp)


def test_fp8_per_token_invariants(orc):
    """Per row: the absmax element codes to +-448, |x' - dec(q) xs| within half a code
    step (relative 2^-4 for normals), zero rows give scale 0 and code 0, and the codes
    equal an independent recipe (numpy fp32 division + torch's e4m3 conversion)."""
    r = np.random.default_rng(62)
    X = (r.standard_normal((9, 96)) * r.uniform(0.01, 50, (9, 1))).astype(np.float16)
    X[3] = 0
    s = r.uniform(0.2, 5.0, 96).astype(np.float32)
    q, xs = orc.fp8_quantize_per_token(X, s)
    Xs = X.astype(np.float32) / s
    a = np.abs(Xs).max(axis=1)
    assert np.array_equal(xs, (a / np.float32(448)).astype(np.float32))
    assert xs[3] == 0 and not q[3].any()
    live = xs > 0
    v = np.clip(Xs[live] / xs[live, None], -448, 448).astype(np.float32)
    assert np.array_equal(q[live], _torch_e4m3(v))
    dec = orc.fp8_decode(q[live]).astype(np.float64)
    assert np.all(np.abs(dec).max(axis=1) == 448.0)
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6))) - 3), 2.0 ** -9)
    assert np.all(np.abs(v - dec) <= step / 2 * (1 + 1e-12))


def test_fp8_weight_granularity_reductions(orc):
    """Per-channel = per-token on W' = W diag(s) (mode: multiply); per-tensor = one
    flattened row."""
    r = np.random.default_rng(63)
    W = (r.standard_normal((7, 64)) * 0.02).astype(np.float32)
    s = np.exp2(r.integers(-3, 4, 64)).astype(np.float32)      # power-of-two s: W * s exact
    q0, s0 = orc.fp8_quantize_weight(W, s, 0)
    qr, sr = orc.fp8_quantize_per_token(W * s, None)
    assert np.array_equal(q0, qr) and np.array_equal(s0, sr)
    q1, s1 = orc.fp8_quantize_weight(W, s, 1)
    qf, sf = orc.fp8_quantize_per_token((W * s).reshape(1, -1), None)
    assert np.array_equal(q1.ravel(), qf.ravel()) and s1[0] == sf[0]


def test_fp8_gemm_exact(orc):
    """For K = 64 the fp64 product of the decoded operands is exact (spans < 53 bits),
    so the integer-unit GEMM must equal it; for large K, Python integers on a few
    entries.  Transposed operands would fail on the non-square shape."""
    r = np.random.default_rng(64)
    A = r.integers(0, 256, (5, 64), dtype=np.uint16).astype(np.uint8)
    B = r.integers(0, 256, (3, 64), dtype=np.uint16).astype(np.uint8)
    A[A & 0x7F == 0x7F] = 0x11                                  # no NaN codes
    B[B & 0x7F == 0x7F] = 0x22
    acc, ab = orc.gemm_fp8(A, B, with_abs=True)
    da, db = orc.fp8_decode(A).astype(np.float64), orc.fp8_decode(B).astype(np.float64)
    assert np.array_equal(acc, da @ db.T)
    assert np.array_equal(ab, np.abs(da) @ np.abs(db).T)
    K = 40000
    A = r.integers(0, 0x7E, (2, K), dtype=np.uint16).astype(np.uint8) | (r.integers(0, 2, (2, K)) << 7).astype(np.uint8)
    B = r.integers(0, 0x7E, (2, K), dtype=np.uint16).astype(np.uint8)
    acc = orc.gemm_fp8(A, B)
    fa = [Fraction(float(v)) for v in orc.fp8_decode(A[1])]
    fb = [Fraction(float(v)) for v in orc.fp8_decode(B[0])]
    assert Fraction(float(acc[1, 0])) == sum(x * y for x, y in zip(fa, fb))
    rows, cols = np.array([1, 0]), np.array([0, 1])
    sa, _ = orc.gemm_fp8_sampled(A, B, rows, cols)
    assert np.array_equal(sa, acc[rows, cols])


def test_fp8_linear_error_bound(orc):
    """The FP8 W8A8 layer against fp64 X W^T: each code carries at most 2^-4 relative
    error (3 mantissa bits, nearest), so |y - XW^T| <= ((1+2^-4)^2 - 1 + 2^-20) sum|x||w|
    elementwise (normals; subnormal codes add at most 2^-10 xs ws per product)."""
    X, W, _ = workloads.random_layer(65, 32, 256, 48, np.float32, n_outliers=3)
    _, s = orc.smooth_scales(X, W, 0.5)
    Wq, ws = orc.fp8_quantize_weight(W, s, 0)
    y = orc.fp8_linear(X, s, Wq, ws, 0, None, np.float32).astype(np.float64)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    xq, xs = orc.fp8_quantize_per_token(X, s)
    bound = ((1 + 2.0 ** -4) ** 2 - 1 + 2.0 ** -20) * (np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T)
    bound += 2.0 ** -10 * 256 * 2 * (xs[:, None].astype(np.float64) * ws[None, :].astype(np.float64)) * 448
    assert np.all(np.abs(y - ref) <= bound)
    # dequantization with power-of-two scales is exact on an exactly representable acc
    acc = orc.gemm_fp8(xq, Wq)
    rr, cc = np.meshgrid(np.arange(32), np.arange(48), indexing="ij")
    p2x, p2w = np.exp2(np.arange(-2, 30) % 5 - 2).astype(np.float32), np.exp2(np.arange(48) % 3 - 1).astype(np.float32)
    yd = orc.fp8_dequant_sampled(acc.ravel(), p2x, p2w, 0, None, rr.ravel(), cc.ravel()).reshape(32, 48)
    assert np.array_equal(yd, (acc.astype(np.float32) * p2x[:, None]) * p2w[None, :])


def test_results_do_not_depend_on_thread_count(orc):
    """The oracle's OpenMP loops partition rows and columns only; every output must be
    bit-identical on one thread and on all of them (the bench times it both ways)."""
    rng = np.random.default_rng(7)
    X = (rng.standard_normal((37, 1040)) * 3).astype(np.float16)
    W = (rng.standard_normal((129, 1040)) * 0.02).astype(np.float16)
    n0 = orc.num_threads()
    outs = []
    for n in (1, max(2, n0)):
        orc.set_num_threads(n)
        try:
            s = orc.smooth_scales(X, W, 0.5)[1]
            Wq, ws = orc.quantize_weight(W, s, 0)
            outs.append((s, Wq, ws) + tuple(orc.w8a8_linear(X, s, Wq, ws, 0, None, np.float16)))
        finally:
            orc.set_num_threads(n0)
    for a, b in zip(*outs):
        assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8))
    assert orc.num_threads() == n0


# --------------------------------------------------------------------------
# The oracle fixes its own rounding mode: round-half-to-even whatever mode the
# calling thread is in, and the caller's mode comes back afterwards
# --------------------------------------------------------------------------

def test_oracle_runs_nearest_even_under_another_mode(orc):
    import ctypes
    libm = ctypes.CDLL("libm.so.6")
    FE_TONEAREST, FE_UPWARD = 0x000, 0x800          # x86-64 <fenv.h> values
    r = np.random.default_rng(42)
    X = r.uniform(-1.0, 1.0, (64, 64)).astype(np.float32)
    Xq_ref, xs_ref = orc.quantize_per_token(X, None)
    Xq_raw = np.empty_like(Xq_ref)
    xs_raw = np.empty_like(xs_ref)
    raw = orc._load()._raw                           # the C entry point without the mode guard
    assert libm.fegetround() == FE_TONEAREST
    libm.fesetround(FE_UPWARD)
    try:
        raw.orc_quantize_per_token(orc._ptr(X), 0, 64, 64, None, None, orc._ptr(Xq_raw), orc._ptr(xs_raw))
        Xq_got, xs_got = orc.quantize_per_token(X, None)
        mode_after = libm.fegetround()
    finally:
        libm.fesetround(FE_TONEAREST)
    # the mode matters for this input: unguarded, some scale (max/127) rounds differently
    assert not np.array_equal(xs_raw.view(np.uint32), xs_ref.view(np.uint32))
    # the guarded entry point gives the round-to-nearest-even results and restores the mode
    assert np.array_equal(xs_got.view(np.uint32), xs_ref.view(np.uint32))
    assert np.array_equal(Xq_got, Xq_ref)
    assert mode_after == FE_UPWARD


# --------------------------------------------------------------------------
# Asymmetric (zero-point) per-token activations ("量化基础与INT8", 非对称量化)
# --------------------------------------------------------------------------

def test_asym_closed_form_rows(orc):
    """Rows whose scale is a power of two, so every quotient is exact:
    - the ramp 0, 1/8, ..., 255/8: scale 1/8, zero point code 0, codes = the ramp index;
    - its negative: zero point code 255, codes again the index;
    - range [-127c, 128c]: scale c, zero point rne(127) = 127 (odd), and the values
      0.5c, 1.5c round to even before the shift (codes 127, 129; rounding after the
      shift would give 128 and 128);
    - range [-127.5c, 127.5c]: zero point rne(127.5) = 128 (ties to even), -1.5c and 1.5c
      give 126 and 130, 127.5c rounds to 128 and clamps at code 255."""
    ramp = (np.arange(256, dtype=np.float32) / 8).reshape(1, 256)
    for row, zq in ((ramp, -128), (-ramp[:, ::-1], 127)):
        q, xs, xz = orc.quantize_per_token_asym(row)
        assert xs[0] == np.float32(0.125) and xz[0] == zq
        assert np.array_equal(q[0].astype(np.int64), np.arange(256) - 128)
    c = np.float32(0.25)
    row = (np.array([-127.0, 0.5, 1.5, 128.0], np.float32) * c).reshape(1, 4)
    q, xs, xz = orc.quantize_per_token_asym(row)
    assert xs[0] == c and xz[0] == 127 - 128
    assert q[0].tolist() == [0 - 128, 127 - 128, 129 - 128, 255 - 128]
    row = (np.array([-127.5, -1.5, 0.0, 1.5, 127.5], np.float32) * c).reshape(1, 5)
    q, xs, xz = orc.quantize_per_token_asym(row)
    assert xs[0] == c and xz[0] == 0
    assert q[0].tolist() == [0 - 128, 126 - 128, 128 - 128, 130 - 128, 255 - 128]


def test_asym_zero_and_one_sided_rows(orc):
    """The range always contains 0: an all-positive row has zero point code 0, an
    all-negative row 255; an all-zero row has scale 0, zero point 0 and all codes 0."""
    X = np.array([[0.0, 0.0, 0.0, 0.0], [1.0, 2.0, 3.0, 4.0], [-4.0, -3.0, -2.0, -1.0]], np.float32)
    q, xs, xz = orc.quantize_per_token_asym(X)
    assert xs[0] == 0 and xz[0] == -128 and np.all(q[0] == -128)
    assert xz[1] == -128 and xz[2] == 127
    assert xs[1] == np.float32(np.float32(4.0) / np.float32(255.0)) == xs[2]
    assert q[1, 3] == 127 and q[2, 0] == -128       # the extremes reach the ends of the code range


def test_asym_codes_are_nearest_levels(orc):
    """Brute force on small random rows: each code u = q + 128 is the integer nearest to
    v + z over [0, 255], with v = fl32(x / scale) and ties broken by rounding v to even
    before the shift; the zero point is the nearest integer to -lo / scale."""
    rng = np.random.default_rng(31)
    X = (rng.standard_normal((40, 24)) * rng.uniform(0.01, 30, (40, 1)) + rng.uniform(-5, 5, (40, 1))).astype(np.float32)
    X[3] = np.abs(X[3])
    X[5] = -np.abs(X[5])
    q, xs, xz = orc.quantize_per_token_asym(X)
    for m in range(X.shape[0]):
        lo, hi = min(0.0, float(X[m].min())), max(0.0, float(X[m].max()))
        sc = xs[m]
        assert abs(float(sc) * 255 - (hi - lo)) <= 2e-6 * (hi - lo)
        z = int(xz[m]) + 128
        zz = -lo / float(sc)
        assert abs(z - zz) <= 0.5 + 1e-6 and 0 <= z <= 255
        for k in range(X.shape[1]):
            v = float(np.float32(X[m, k]) / np.float32(sc))
            cands = [u for u in range(256) if abs(v + z - u) == min(abs(v + z - w) for w in range(256))]
            if len(cands) == 2:
                cands = [u for u in cands if (u - z) % 2 == 0]
            assert int(q[m, k]) + 128 == cands[0], (m, k)


def test_asym_round_trip_bound_and_invariance(orc):
    """|x - scale (q - zq)| <= scale / 2 inside the range (scale at its two ends, where the
    shifted code can be clamped); scaling a row by a power of two scales its scale and
    keeps its codes and zero point; a power-of-two smoothing vector equals dividing first."""
    rng = np.random.default_rng(32)
    X = (rng.standard_normal((64, 300)) * 3 + rng.uniform(-4, 4, (64, 1))).astype(np.float32)
    q, xs, xz = orc.quantize_per_token_asym(X)
    xhat = xs[:, None].astype(np.float64) * (q.astype(np.float64) - xz[:, None])
    err = np.abs(X - xhat)
    lo = np.minimum(X.min(1), 0)[:, None]
    hi = np.maximum(X.max(1), 0)[:, None]
    inner = (X > lo + xs[:, None]) & (X < hi - xs[:, None])
    assert np.all(err <= xs[:, None] * (1 + 1e-6))
    assert np.all(err[inner] <= (xs[:, None] * np.ones_like(X))[inner] * (0.5 + 1e-6))
    q2, xs2, xz2 = orc.quantize_per_token_asym(X * np.float32(8.0))
    assert np.array_equal(q2, q) and np.array_equal(xz2, xz) and np.array_equal(xs2, xs * np.float32(8.0))
    s = np.exp2(rng.integers(-3, 4, 300)).astype(np.float32)
    q3, xs3, xz3 = orc.quantize_per_token_asym(X, s)
    q4, xs4, xz4 = orc.quantize_per_token_asym(X / s)
    assert np.array_equal(q3, q4) and np.array_equal(xs3, xs4) and np.array_equal(xz3, xz4)


def test_asym_corrected_accumulator_is_dezeroed_integer_product(orc):
    """The corrected accumulator equals sum_k (q - zq) * w, computed here the other way
    round (zero point removed from every code first, then an int64 product), and the
    row sums are numpy's."""
    rng = np.random.default_rng(33)
    X = (rng.standard_normal((37, 200)) + 1.5).astype(np.float32)
    W = (rng.standard_normal((29, 200)) * 0.05).astype(np.float32)
    Wq, ws = orc.quantize_weight(W, None, 0)
    rs = orc.weight_rowsum(Wq)
    assert np.array_equal(rs, Wq.astype(np.int64).sum(1))
    q, xs, xz = orc.quantize_per_token_asym(X)
    acc = orc.gemm_i8(q, Wq)
    y, acc2 = orc.dequant_asym(acc, xs, xz, ws, rs, 0, None)
    ref = (q.astype(np.int64) - xz[:, None]) @ Wq.astype(np.int64).T
    assert np.array_equal(acc2.astype(np.int64), ref)
    # with power-of-two scales the dequantization is exact
    y2, _ = orc.dequant_asym(acc, np.full(37, 0.5, np.float32), xz, np.full(29, 0.25, np.float32), rs, 0, None)
    assert np.array_equal(y2.astype(np.float64), ref * 0.125)


def test_asym_linear_error_bound(orc):
    """The zero-point layer against fp64 X W^T: per element within the sum of the two
    quantization errors (activation at most one scale step, weight half a step) plus
    fp32 rounding."""
    rng = np.random.default_rng(34)
    X = (rng.standard_normal((48, 256)) + 0.7).astype(np.float32)
    W = (rng.standard_normal((40, 256)) * 0.05).astype(np.float32)
    Wq, ws = orc.quantize_weight(W, None, 0)
    Xq, xs, xz, rs, acc2, Y = orc.w8a8_asym_linear(X, None, Wq, ws, 0, None, np.float32)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    what = Wq.astype(np.float64) * ws[:, None]
    bound = xs[:, None] * np.abs(what).sum(1)[None, :] + np.abs(X).astype(np.float64) @ (ws[:, None] / 2 * np.ones_like(W)).T
    assert np.all(np.abs(Y - exact) <= bound * 1.001 + 1e-5 * np.abs(exact) + 1e-6)
