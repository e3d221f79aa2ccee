"""Parity of the zero-point (asymmetric) activation path with the CPU oracle, through
the C ABI: codes, scales, zero points, weight row sums and the corrected int32
accumulators bit-exact; outputs bit-exact too (same fp32 steps in the same order)
and within the stated tolerance.  Every comparison covers the whole output."""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import Guarded, assert_bits_equal, assert_close, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import int8_quantization_amd as sq
    return sq


def gpu_quantize_asym(sq, X, s):
    M, K = X.shape
    Xq = Guarded((M, K), torch.int8)
    xs = Guarded((M,), torch.float32)
    xz = Guarded((M,), torch.int32)
    sq.sq_quantize_per_token_asym(dev(X), None if s is None else dev(s), Xq.t, xs.t, xz.t)
    torch.cuda.synchronize()
    return Xq.np(), xs.np(), xz.np()


def gpu_rowsum(sq, Wq):
    rs = Guarded((Wq.shape[0],), torch.int32)
    sq.sq_weight_rowsum(dev(Wq), rs.t)
    torch.cuda.synchronize()
    return rs.np()


def gpu_gemm_asym(sq, Xq, xs, xz, Wq, ws, gran, rs, bias, out_dt):
    M, N = Xq.shape[0], Wq.shape[0]
    Y = Guarded((M, N), torch.float16 if out_dt == np.float16 else torch.float32)
    acc = Guarded((M, N), torch.int32)
    sq.w8a8_asym_gemm_dequant(dev(Xq), dev(xs), dev(xz), dev(Wq), dev(ws), gran, dev(rs),
                              None if bias is None else dev(bias), Y.t, acc.t)
    torch.cuda.synchronize()
    return acc.np(), Y.np()


def _rows(seed, M, K, dt):
    """Rows not centred on zero: N(0,1) * a + b with per-row a, b, plus special rows."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K), dtype=np.float32) * rng.uniform(0.1, 4, (M, 1)).astype(np.float32)
    X += rng.uniform(-3, 3, (M, 1)).astype(np.float32)
    if M > 4:
        X[1] = np.abs(X[1])            # all positive: zero point code 0
        X[2] = -np.abs(X[2])           # all negative: zero point code 255
        X[3] = 0.0                     # all zero: scale 0
    return X.astype(dt)


# M, K, dtype, smoothing: the register-resident kernel's configurations (one 16-byte chunk per
# thread for few rows or short rows, 2 and 5 chunks, the fp32 ones, more rows than blocks) and
# the two-pass kernel for longer rows
ASYM_CASES = [
    (1, 16, np.float16, False), (7, 48, np.float32, True), (300, 1040, np.float16, True),
    (256, 8192, np.float16, False), (1000, 4096, np.float16, True), (300, 12304, np.float16, True),
    (130, 20480, np.float16, False), (70, 4096, np.float32, False), (90, 12288, np.float32, True),
    (20, 40960, np.float16, True), (9, 20000, np.float32, False),
    (1024, 16, np.float16, True), (1029, 512, np.float16, False), (2048, 1040, np.float16, False),
    (1100, 4096, np.float16, True), (1030, 8192, np.float16, True), (1024, 10240, np.float16, False),
    (1024, 12304, np.float16, True), (1500, 20480, np.float16, False),
]


@pytest.mark.parametrize("M,K,dt,smooth", ASYM_CASES)
def test_quantize_asym(sq, orc, M, K, dt, smooth):
    X = _rows(M * 7 + K, M, K, dt)
    s = np.random.default_rng(K).uniform(0.2, 5.0, K).astype(np.float32) if smooth else None
    q, xs, xz = gpu_quantize_asym(sq, X, s)
    q_r, xs_r, xz_r = orc.quantize_per_token_asym(X, s)
    assert_bits_equal(xs, xs_r, "x_scale")
    assert_bits_equal(xz, xz_r, "x_zero")
    assert_bits_equal(q, q_r, "Xq")


def test_quantize_asym_ties_and_ends(sq, orc):
    """Rows of exact quotients (power-of-two scales): half-even ties before the shift with
    an odd and an even zero point, and the clamp at code 255."""
    c = np.float32(0.25)
    rows = np.zeros((4, 16), np.float32)
    rows[0, :4] = np.array([-127.0, 0.5, 1.5, 128.0], np.float32) * c
    rows[1, :5] = np.array([-127.5, -1.5, 0.0, 1.5, 127.5], np.float32) * c
    rows[2] = np.arange(16, dtype=np.float32) * 17 / 8         # ramp: scale 1/8
    rows[3] = -rows[2]
    q, xs, xz = gpu_quantize_asym(sq, rows, None)
    q_r, xs_r, xz_r = orc.quantize_per_token_asym(rows, None)
    assert_bits_equal(xs, xs_r, "x_scale")
    assert_bits_equal(xz, xz_r, "x_zero")
    assert_bits_equal(q, q_r, "Xq")
    assert q[0, :4].tolist() == [-128, -1, 1, 127]


@pytest.mark.parametrize("N,K", [(1, 16), (300, 4096), (5, 20480), (1000, 144)])
def test_weight_rowsum(sq, orc, N, K):
    Wq = np.random.default_rng(N + K).integers(-128, 128, (N, K)).astype(np.int8)
    Wq[0] = -128
    assert_bits_equal(gpu_rowsum(sq, Wq), orc.weight_rowsum(Wq), "rowsum")


# M <= 16: the decode kernel (its token-group configurations, activations in registers and
# reloaded per chunk); larger M: the tile kernel's 128 x 128, 256 x 192 and 256 x 256 tiles
# and the two-launch column split (each compared over its whole output)
ASYM_GEMM_CASES = [
    (1, 300, 1024), (4, 1000, 4096), (8, 130, 12304), (16, 4100, 8192), (3, 257, 20496), (12, 77, 16384),
    (15, 90, 20496),
    (300, 520, 1040), (2047, 6143, 144), (3000, 5000, 272), (4096, 10240, 144),
]


@pytest.mark.parametrize("M,N,K", ASYM_GEMM_CASES)
@pytest.mark.parametrize("gran,use_bias,out_dt", [(0, False, np.float16), (1, True, np.float32)])
def test_gemm_asym(sq, orc, M, N, K, gran, use_bias, out_dt):
    rng = np.random.default_rng(M * 13 + N + K)
    X = _rows(M + N, M, K, np.float16)
    Xq, xs, xz = orc.quantize_per_token_asym(X, None)
    Wq = rng.integers(-128, 128, (N, K)).astype(np.int8)
    Wq[N - 1] = -128                    # extreme row sum
    ws = rng.uniform(1e-4, 1e-2, N if gran == 0 else 1).astype(np.float32)
    bias = rng.standard_normal(N).astype(np.float32) if use_bias else None
    rs = orc.weight_rowsum(Wq)
    acc, Y = gpu_gemm_asym(sq, Xq, xs, xz, Wq, ws, gran, rs, bias, out_dt)
    y, acc_r = orc.dequant_asym(orc.gemm_i8(Xq, Wq), xs, xz, ws, rs, gran, bias)
    assert_bits_equal(acc, acc_r, "corrected acc")
    ref = y if out_dt == np.float32 else orc.float_to_half(y)
    assert_close(Y, ref, 1e-3 if out_dt == np.float32 else 1e-2)
    assert_bits_equal(Y, ref, "Y")


@pytest.mark.slow
def test_full_ffn_down_7b_asym(sq, orc):
    """The 7B FFN-down projection on SiLU activations at full size (2048 x 11008 -> 4096),
    the workload bench.py times: every code, scale, zero point, row sum, corrected
    accumulator and output."""
    wl = workloads.ffn_down_7b_post_activation()
    X, W = wl.X, wl.weights["down"]
    print(f"full-size zero-point layer: {wl.name}", flush=True)
    N, K = W.shape
    Wq_g, ws_g = Guarded((N, K), torch.int8), Guarded((N,), torch.float32)
    wsp = torch.empty(sq.sq_workspace_size(sq.SQ_OP_QUANT_WEIGHT, 0, N, K), dtype=torch.uint8, device="cuda")
    sq.sq_quantize_weight(dev(W), None, 0, Wq_g.t, ws_g.t, wsp)
    torch.cuda.synchronize()
    Wq, ws = Wq_g.np(), ws_g.np()
    Wq_r, ws_r = orc.quantize_weight(W, None, 0)
    assert_bits_equal(Wq, Wq_r, "Wq")
    assert_bits_equal(ws, ws_r, "w_scale")
    rs = gpu_rowsum(sq, Wq)
    rs_r = orc.weight_rowsum(Wq_r)
    assert_bits_equal(rs, rs_r, "rowsum")
    q, xs, xz = gpu_quantize_asym(sq, X, None)
    Xq_r, xs_r, xz_r, _, acc_r, Y_r = orc.w8a8_asym_linear(X, None, Wq_r, ws_r, 0, None, np.float16)
    assert_bits_equal(xs, xs_r, "x_scale")
    assert_bits_equal(xz, xz_r, "x_zero")
    assert_bits_equal(q, Xq_r, "Xq")
    acc, Y = gpu_gemm_asym(sq, q, xs, xz, Wq, ws, 0, rs, None, np.float16)
    assert_bits_equal(acc, acc_r, "corrected acc")
    assert_close(Y, Y_r, 1e-2)
    assert_bits_equal(Y, Y_r, "Y")
