"""CPU oracle for the quantized INT8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
Python binding) never imports it and shares no code with it.

The arithmetic lives in ``sq_oracle.c`` (plain C, gcc, exact int64
accumulation, IEEE binary32 steps with round-half-to-even); this module only
marshals numpy arrays.  The composite functions at the bottom chain those steps
in the order the pages give: smooth -> per-token quantize -> int8 GEMM ->
dequantize ("量化基础与INT8", section "INT8推理流程"; "SmoothQuant量化实战",
section 3.4), and the LLM.int8() split ("LLM.int8()技术解析", section 3.1).
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_F32, _F16 = 0, 1
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("SQ_ORACLE_LIB")       # another build of the same source (sanitizer runs)
    if path is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
    lib = C.CDLL(path)
    P, I64, F, D, I = C.c_void_p, C.c_int64, C.c_float, C.c_double, C.c_int
    sig = {
        "orc_half_to_float_array": (None, [P, P, I64]),
        "orc_float_to_half_array": (None, [P, P, I64]),
        "orc_num_threads": (I, []),
        "orc_set_num_threads": (None, [I]),
        "orc_col_absmax": (None, [P, I, I64, I64, P]),
        "orc_smooth_from_maxima": (None, [P, P, I64, F, P]),
        "orc_smooth_scales": (None, [P, I, I64, P, I, I64, I64, F, P, P]),
        "orc_quantize_weight": (None, [P, I, I64, I64, P, I, P, P]),
        "orc_quantize_per_token": (None, [P, I, I64, I64, P, P, P, P]),
        "orc_gemm_i8": (I64, [P, P, I64, I64, I64, P]),
        "orc_gemm_i8_sampled": (I64, [P, P, I64, P, P, I64, P]),
        "orc_dequant": (None, [P, P, P, I, P, I64, I64, P]),
        "orc_dequant_sampled": (None, [P, P, P, I, P, P, P, I64, P]),
        "orc_outlier_columns": (I64, [P, I64, I64, F, P, P]),
        "orc_side_product_sampled": (None, [P, P, I64, P, I64, P, P, I64, P]),
        "orc_combine_to_half": (None, [P, P, I64, P]),
        "orc_layernorm_stats": (None, [P, I64, I64, F, P, P, P, P]),
        "orc_layernorm": (None, [P, I64, I64, P, P, F, P]),
        "orc_layernorm_quantize": (None, [P, I64, I64, P, P, F, P, P]),
        "orc_fold_layernorm": (None, [P, P, P, I64, P, P]),
        "orc_percentile_rank": (I64, [I64, D]),
        "orc_abs_percentile": (F, [P, I, I64, I64, P, D]),
        "orc_static_scale": (F, [P, I, I64, I64, P, D]),
        "orc_quantize_static": (None, [P, I, I64, I64, P, F, P]),
        "orc_quantize_per_token_asym": (None, [P, I, I64, I64, P, P, P, P]),
        "orc_weight_rowsum": (None, [P, I64, I64, P]),
        "orc_dequant_asym": (I64, [P, P, P, P, I, P, P, I64, I64, P, P]),
        "orc_kv_calibrate_per_head": (None, [P, I, I64, I64, I64, F, P]),
        "orc_kv_quantize_per_head": (None, [P, I, I64, I64, I64, P, P]),
        "orc_dequantize": (None, [P, I64, I64, P, I64, I64, P]),
        "orc_fp8_encode_array": (None, [P, P, I64]),
        "orc_fp8_decode_array": (None, [P, P, I64]),
        "orc_fp8_quantize_rows": (None, [P, I, I64, I64, P, I, P, P]),
        "orc_fp8_quantize_tensor": (None, [P, I, I64, I64, P, P, P]),
        "orc_gemm_fp8": (None, [P, P, I64, I64, I64, P, P]),
        "orc_gemm_fp8_sampled": (None, [P, P, I64, P, P, I64, P, P]),
        "orc_fp8_dequant": (None, [P, P, P, I, P, P, P, I64, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    lib.orc_rounding_enter.restype = I
    lib.orc_rounding_enter.argtypes = []
    lib.orc_rounding_leave.restype = None
    lib.orc_rounding_leave.argtypes = [I]
    _lib = _NearestEven(lib, sig)
    return _lib


class _NearestEven:
    """The oracle library with every entry point run under round-to-nearest-even (the
    caller's rounding mode is restored afterwards)."""

    def __init__(self, lib, names):
        self._raw = lib
        for name in names:
            setattr(self, name, self._wrap(getattr(lib, name)))

    def _wrap(self, fn):
        raw = self._raw

        def call(*args):
            prev = raw.orc_rounding_enter()
            try:
                return fn(*args)
            finally:
                raw.orc_rounding_leave(prev)
        return call


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _as(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _fp(a):
    """(contiguous array, dtype code) for a float16 or float32 input."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        return a, _F16
    if a.dtype == np.float32:
        return a, _F32
    raise TypeError(f"oracle takes float16 or float32, got {a.dtype}")


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's OpenMP loops (timing only; results do not depend on it)."""
    _load().orc_set_num_threads(int(n))


def half_to_float(h):
    h = _as(h, np.float16)
    out = np.empty(h.shape, np.float32)
    _load().orc_half_to_float_array(_ptr(h), _ptr(out), h.size)
    return out


def float_to_half(f):
    f = _as(f, np.float32)
    out = np.empty(f.shape, np.float16)
    _load().orc_float_to_half_array(_ptr(f), _ptr(out), f.size)
    return out


def col_absmax(X, amax=None):
    """Running per-column absolute maximum (calibration statistic)."""
    X, dt = _fp(X)
    M, K = X.shape
    amax = np.zeros(K, np.float32) if amax is None else _as(amax, np.float32).copy()
    _load().orc_col_absmax(_ptr(X), dt, M, K, _ptr(amax))
    return amax


def smooth_from_maxima(act_max, w_max, alpha):
    act_max, w_max = _as(act_max, np.float32), _as(w_max, np.float32)
    s = np.empty(act_max.shape[0], np.float32)
    _load().orc_smooth_from_maxima(_ptr(act_max), _ptr(w_max), act_max.shape[0], float(alpha), _ptr(s))
    return s


def smooth_scales(X_cal, W, alpha, act_max=None):
    """Returns (updated act_max, s)."""
    W, wdt = _fp(W)
    N, K = W.shape
    amax = np.zeros(K, np.float32) if act_max is None else _as(act_max, np.float32).copy()
    if X_cal is None:
        xp, xdt, Mc = None, _F32, 0
    else:
        X_cal, xdt = _fp(X_cal)
        xp, Mc = _ptr(X_cal), X_cal.shape[0]
    s = np.empty(K, np.float32)
    _load().orc_smooth_scales(xp, xdt, Mc, _ptr(W), wdt, N, K, float(alpha), _ptr(amax), _ptr(s))
    return amax, s


def quantize_weight(W, s=None, gran=0):
    """gran 0: per output channel; 1: per tensor.  Returns (Wq int8 [N,K], w_scale)."""
    W, dt = _fp(W)
    N, K = W.shape
    s = None if s is None else _as(s, np.float32)
    Wq = np.empty((N, K), np.int8)
    ws = np.empty(N if gran == 0 else 1, np.float32)
    _load().orc_quantize_weight(_ptr(W), dt, N, K, _ptr(s), int(gran), _ptr(Wq), _ptr(ws))
    return Wq, ws


def quantize_per_token(X, s=None, skip=None):
    """Returns (Xq int8 [M,K], x_scale [M]).  skip: bool/uint8 [K] columns to leave out."""
    X, dt = _fp(X)
    M, K = X.shape
    s = None if s is None else _as(s, np.float32)
    skip = None if skip is None else _as(skip, np.uint8)
    Xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    _load().orc_quantize_per_token(_ptr(X), dt, M, K, _ptr(s), _ptr(skip), _ptr(Xq), _ptr(xs))
    return Xq, xs


def gemm_i8(A, B):
    A, B = _as(A, np.int8), _as(B, np.int8)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    acc = np.empty((M, N), np.int32)
    bad = _load().orc_gemm_i8(_ptr(A), _ptr(B), M, N, K, _ptr(acc))
    if bad:
        raise OverflowError(f"{bad} accumulators exceed int32")
    return acc


def gemm_i8_sampled(A, B, rows, cols):
    A, B = _as(A, np.int8), _as(B, np.int8)
    rows, cols = _as(rows, np.int64), _as(cols, np.int64)
    out = np.empty(rows.shape[0], np.int32)
    bad = _load().orc_gemm_i8_sampled(_ptr(A), _ptr(B), A.shape[1], _ptr(rows), _ptr(cols),
                                      rows.shape[0], _ptr(out))
    if bad:
        raise OverflowError(f"{bad} accumulators exceed int32")
    return out


def dequant(acc, x_scale, w_scale, gran=0, bias=None):
    acc = _as(acc, np.int32)
    M, N = acc.shape
    xs, ws = _as(x_scale, np.float32), _as(w_scale, np.float32)
    bias = None if bias is None else _as(bias, np.float32)
    y = np.empty((M, N), np.float32)
    _load().orc_dequant(_ptr(acc), _ptr(xs), _ptr(ws), int(gran), _ptr(bias), M, N, _ptr(y))
    return y


def dequant_sampled(acc, x_scale, w_scale, gran, bias, rows, cols):
    acc = _as(acc, np.int32)
    xs, ws = _as(x_scale, np.float32), _as(w_scale, np.float32)
    bias = None if bias is None else _as(bias, np.float32)
    rows, cols = _as(rows, np.int64), _as(cols, np.int64)
    y = np.empty(rows.shape[0], np.float32)
    _load().orc_dequant_sampled(_ptr(acc), _ptr(xs), _ptr(ws), int(gran), _ptr(bias), _ptr(rows),
                                _ptr(cols), rows.shape[0], _ptr(y))
    return y


def outlier_columns(X16, threshold):
    """Returns (mask uint8 [K], ascending idx int32 [count])."""
    X16 = _as(X16, np.float16)
    M, K = X16.shape
    mask = np.empty(K, np.uint8)
    idx = np.empty(K, np.int32)
    count = _load().orc_outlier_columns(_ptr(X16), M, K, float(threshold), _ptr(mask), _ptr(idx))
    return mask, idx[:count].copy()


def side_product_sampled(X16, W16, idx, rows, cols):
    X16, W16 = _as(X16, np.float16), _as(W16, np.float16)
    idx = _as(idx, np.int32)
    rows, cols = _as(rows, np.int64), _as(cols, np.int64)
    side = np.empty(rows.shape[0], np.float64)
    _load().orc_side_product_sampled(_ptr(X16), _ptr(W16), X16.shape[1], _ptr(idx), idx.shape[0],
                                     _ptr(rows), _ptr(cols), rows.shape[0], _ptr(side))
    return side


def combine_to_half(y_int8, side):
    y, side = _as(y_int8, np.float32), _as(side, np.float64)
    out = np.empty(y.shape, np.float16)
    _load().orc_combine_to_half(_ptr(y), _ptr(side), y.size, _ptr(out))
    return out


# ---------------------------------------------------------------------------
# Composite paths (steps chained in the pages' order; no extra arithmetic).
# ---------------------------------------------------------------------------

def _store(y, out_dtype):
    return y if out_dtype == np.float32 else float_to_half(y)


def w8a8_linear(X, s, Wq, w_scale, gran=0, bias=None, out_dtype=np.float16, rows=None):
    """X [M,K] -> (Xq, xs, acc, Y) for the rows given (all rows when None).

    Per-token quantization of X diag(s)^-1, int8 GEMM against the prepared
    Wq, dequantization, output stored as out_dtype."""
    Xr = X if rows is None else X[rows]
    Xq, xs = quantize_per_token(Xr, s)
    acc = gemm_i8(Xq, Wq)
    y = dequant(acc, xs, w_scale, gran, bias)
    return Xq, xs, acc, _store(y, out_dtype)


# ---------------------------------------------------------------------------
# Asymmetric (zero-point) per-token activations ("量化基础与INT8", 非对称量化):
# x' ~ scale * (q - zq), the GEMM corrected by zq * rowsum(Wq).
# ---------------------------------------------------------------------------
def quantize_per_token_asym(X, s=None):
    """Returns (Xq int8 [M,K], x_scale [M] float32, x_zero [M] int32)."""
    X, dt = _fp(X)
    M, K = X.shape
    s = None if s is None else _as(s, np.float32)
    Xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    xz = np.empty(M, np.int32)
    _load().orc_quantize_per_token_asym(_ptr(X), dt, M, K, _ptr(s), _ptr(Xq), _ptr(xs), _ptr(xz))
    return Xq, xs, xz


def weight_rowsum(Wq):
    Wq = _as(Wq, np.int8)
    N, K = Wq.shape
    rs = np.empty(N, np.int32)
    _load().orc_weight_rowsum(_ptr(Wq), N, K, _ptr(rs))
    return rs


def dequant_asym(acc, x_scale, x_zero, w_scale, rowsum, gran=0, bias=None):
    """Returns (y float32 [M,N], corrected accumulators int32 [M,N])."""
    acc = _as(acc, np.int32)
    M, N = acc.shape
    xs, xz = _as(x_scale, np.float32), _as(x_zero, np.int32)
    ws, rs = _as(w_scale, np.float32), _as(rowsum, np.int32)
    bias = None if bias is None else _as(bias, np.float32)
    y = np.empty((M, N), np.float32)
    acc2 = np.empty((M, N), np.int32)
    bad = _load().orc_dequant_asym(_ptr(acc), _ptr(xs), _ptr(xz), _ptr(ws), int(gran), _ptr(rs), _ptr(bias), M, N,
                                   _ptr(y), _ptr(acc2))
    if bad:
        raise OverflowError(f"{bad} corrected accumulators exceed int32")
    return y, acc2


def w8a8_asym_linear(X, s, Wq, w_scale, gran=0, bias=None, out_dtype=np.float16):
    """Zero-point activations: (Xq, xs, xz, rowsum, corrected acc, Y) in the pages' order:
    quantize, int8 GEMM, correction, dequantize."""
    Xq, xs, xz = quantize_per_token_asym(X, s)
    rs = weight_rowsum(Wq)
    acc = gemm_i8(Xq, Wq)
    y, acc2 = dequant_asym(acc, xs, xz, w_scale, rs, gran, bias)
    return Xq, xs, xz, rs, acc2, _store(y, out_dtype)


def llm_int8_linear(X16, W16, Wq, w_scale, threshold, bias=None, rows=None):
    """LLM.int8(): returns (mask, idx, Xq, xs, acc, Y fp16) for the rows given."""
    mask, idx = outlier_columns(X16, threshold)          # columns decided over all rows
    Xr = X16 if rows is None else X16[rows]
    Xq, xs = quantize_per_token(Xr, None, skip=mask)
    acc = gemm_i8(Xq, Wq)
    y = dequant(acc, xs, w_scale, 0, bias)
    M, N = y.shape
    rr = np.repeat(np.arange(M, dtype=np.int64), N)
    cc = np.tile(np.arange(N, dtype=np.int64), M)
    side = side_product_sampled(Xr, W16, idx, rr, cc).reshape(M, N)
    return mask, idx, Xq, xs, acc, combine_to_half(y, side)


# ---------------------------------------------------------------------------
# LayerNorm with the smoothing folded in, fused with per-token quantization
# ("SmoothQuant量化实战", sections 2.3, 4.2, 4.5).  Binary16 inputs; exact
# integer row statistics (see sq_oracle.c for the reading).
# ---------------------------------------------------------------------------
def _half_bits(X16):
    X16 = np.ascontiguousarray(X16, dtype=np.float16)
    return X16.view(np.uint16)


def fold_layernorm(gamma, beta, s):
    """gamma' = fl32(gamma / s), beta' = fl32(beta / s) (beta may be None)."""
    g = _as(gamma, np.float32)
    b = None if beta is None else _as(beta, np.float32)
    sv = _as(s, np.float32)
    K = g.size
    go = np.empty(K, np.float32)
    bo = None if b is None else np.empty(K, np.float32)
    _load().orc_fold_layernorm(_ptr(g), _ptr(b), _ptr(sv), K, _ptr(go), _ptr(bo))
    return go, bo


def layernorm_stats(X16, eps):
    """(mu32, rstd32, mu64, var64) per row."""
    h = _half_bits(X16)
    M, K = h.shape
    mu32, r32 = np.empty(M, np.float32), np.empty(M, np.float32)
    mu64, var64 = np.empty(M, np.float64), np.empty(M, np.float64)
    _load().orc_layernorm_stats(_ptr(h), M, K, float(eps), _ptr(mu32), _ptr(r32), _ptr(mu64), _ptr(var64))
    return mu32, r32, mu64, var64


def layernorm(X16, gamma, beta, eps):
    """LayerNorm output y (fp32 [M, K]) with the (folded) weights."""
    h = _half_bits(X16)
    M, K = h.shape
    g = _as(gamma, np.float32)
    b = None if beta is None else _as(beta, np.float32)
    Y = np.empty((M, K), np.float32)
    _load().orc_layernorm(_ptr(h), M, K, _ptr(g), _ptr(b), float(eps), _ptr(Y))
    return Y


def layernorm_quantize(X16, gamma, beta, eps):
    """The fused forward step: (Xq int8 [M, K], x_scale fp32 [M])."""
    h = _half_bits(X16)
    M, K = h.shape
    g = _as(gamma, np.float32)
    b = None if beta is None else _as(beta, np.float32)
    Xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    _load().orc_layernorm_quantize(_ptr(h), M, K, _ptr(g), _ptr(b), float(eps), _ptr(Xq), _ptr(xs))
    return Xq, xs


# ---------------------------------------------------------------------------
# Static per-tensor activation scale (basics notes, 静态量化; the percentile
# calibrator of the deployment page): nearest-rank percentile of |x'| over the
# calibration batch, scale = fl32(T / 127), then quantization with that scale.
# ---------------------------------------------------------------------------
def percentile_rank(n, p):
    return int(_load().orc_percentile_rank(int(n), float(p)))


def abs_percentile(X, s, p):
    Xc, dt = _fp(X)
    M, K = Xc.shape
    sv = None if s is None else _as(s, np.float32)
    return np.float32(_load().orc_abs_percentile(_ptr(Xc), dt, M, K, _ptr(sv), float(p)))


def static_scale(X, s, p):
    Xc, dt = _fp(X)
    M, K = Xc.shape
    sv = None if s is None else _as(s, np.float32)
    return np.float32(_load().orc_static_scale(_ptr(Xc), dt, M, K, _ptr(sv), float(p)))


def quantize_static(X, s, xs):
    Xc, dt = _fp(X)
    M, K = Xc.shape
    sv = None if s is None else _as(s, np.float32)
    Xq = np.empty((M, K), np.int8)
    _load().orc_quantize_static(_ptr(Xc), dt, M, K, _ptr(sv), float(np.float32(xs)), _ptr(Xq))
    return Xq


# ---------------------------------------------------------------------------
# INT8 KV cache with per-head scales ("SmoothQuant量化实战", section 5.2).
# KV layout [T, H, D] (tokens, heads, head dim).
# ---------------------------------------------------------------------------
def kv_calibrate_per_head(KV, margin=1.0):
    KVc, dt = _fp(KV)
    T, H, D = KVc.shape
    sc = np.empty(H, np.float32)
    _load().orc_kv_calibrate_per_head(_ptr(KVc), dt, T, H, D, float(margin), _ptr(sc))
    return sc


def kv_quantize_per_head(KV, scale):
    KVc, dt = _fp(KV)
    T, H, D = KVc.shape
    sc = _as(scale, np.float32)
    q = np.empty((T, H, D), np.int8)
    _load().orc_kv_quantize_per_head(_ptr(KVc), dt, T, H, D, _ptr(sc), _ptr(q))
    return q


def dequantize(q, scale, row_stride, group):
    """y[m, j] = fl32(q[m, j] * scale[m * row_stride + j // group]) (fp32)."""
    qc = np.ascontiguousarray(q, np.int8)
    M, K = qc.shape
    sc = _as(scale, np.float32)
    y = np.empty((M, K), np.float32)
    _load().orc_dequantize(_ptr(qc), M, K, _ptr(sc), int(row_stride), int(group), _ptr(y))
    return y


# ---------------------------------------------------------------------------
# FP8 (E4M3, OCP e4m3fn) W8A8 variant (SmoothQuant page, section 6.1)
# ---------------------------------------------------------------------------
def fp8_encode(v):
    """float32 -> e4m3fn code bytes (uint8), nearest-even, saturating at 448."""
    v = _as(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().orc_fp8_encode_array(_ptr(v), _ptr(out), v.size)
    return out


def fp8_decode(c):
    c = _as(c, np.uint8)
    out = np.empty(c.shape, np.float32)
    _load().orc_fp8_decode_array(_ptr(c), _ptr(out), c.size)
    return out


def fp8_quantize_per_token(X, s=None):
    """Per-row FP8 codes of X' = X / s (or X): (codes uint8 [M,K], scale fp32 [M])."""
    X, dt = _fp(X)
    M, K = X.shape
    q = np.empty((M, K), np.uint8)
    sc = np.empty(M, np.float32)
    sv = None if s is None else _as(s, np.float32)
    _load().orc_fp8_quantize_rows(_ptr(X), dt, M, K, _ptr(sv), 0 if s is None else 1, _ptr(q), _ptr(sc))
    return q, sc


def fp8_quantize_weight(W, s, gran):
    """FP8 codes of W' = W diag(s) (or W): per output row (gran 0) or per tensor (gran 1)."""
    W, dt = _fp(W)
    N, K = W.shape
    q = np.empty((N, K), np.uint8)
    sv = None if s is None else _as(s, np.float32)
    if gran == 0:
        sc = np.empty(N, np.float32)
        _load().orc_fp8_quantize_rows(_ptr(W), dt, N, K, _ptr(sv), 0 if s is None else 2, _ptr(q), _ptr(sc))
    else:
        sc = np.empty(1, np.float32)
        _load().orc_fp8_quantize_tensor(_ptr(W), dt, N, K, _ptr(sv), _ptr(q), _ptr(sc))
    return q, sc


def gemm_fp8(A, B, with_abs=False):
    """Exact sum_k dec(A[m,k]) dec(B[n,k]) in fp64 (and sum_k |...| when with_abs)."""
    A = _as(A, np.uint8)
    B = _as(B, np.uint8)
    M, K = A.shape
    N = B.shape[0]
    acc = np.empty((M, N), np.float64)
    ab = np.empty((M, N), np.float64) if with_abs else None
    _load().orc_gemm_fp8(_ptr(A), _ptr(B), M, N, K, _ptr(acc), _ptr(ab))
    return (acc, ab) if with_abs else acc


def gemm_fp8_sampled(A, B, rows, cols):
    """(exact acc, sum |products|) at the given positions."""
    A = _as(A, np.uint8)
    B = _as(B, np.uint8)
    K = A.shape[1]
    rows = _as(rows, np.int64)
    cols = _as(cols, np.int64)
    acc = np.empty(rows.size, np.float64)
    ab = np.empty(rows.size, np.float64)
    _load().orc_gemm_fp8_sampled(_ptr(A), _ptr(B), K, _ptr(rows), _ptr(cols), rows.size, _ptr(acc), _ptr(ab))
    return acc, ab


def fp8_dequant_sampled(acc, x_scale, w_scale, wgran, bias, rows, cols):
    """y = ((float)acc * xs[m]) * ws[n or 0] (+ bias[n]) at the given positions (fp32)."""
    acc = _as(acc, np.float64)
    rows = _as(rows, np.int64)
    cols = _as(cols, np.int64)
    y = np.empty(rows.size, np.float32)
    _load().orc_fp8_dequant(_ptr(acc), _ptr(_as(x_scale, np.float32)), _ptr(_as(w_scale, np.float32)), int(wgran),
                            _ptr(None if bias is None else _as(bias, np.float32)), _ptr(rows), _ptr(cols), rows.size,
                            _ptr(y))
    return y


def fp8_linear(X, s, Wq, ws, wgran, bias, out_dtype):
    """FP8 W8A8 forward for small shapes: per-token FP8 codes, exact GEMM, dequant."""
    Xq, xs = fp8_quantize_per_token(X, s)
    M, N = X.shape[0], Wq.shape[0]
    acc = gemm_fp8(Xq, Wq)
    rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    y = fp8_dequant_sampled(acc.ravel(), xs, ws, wgran, bias, rr.ravel(), cc.ravel()).reshape(M, N)
    return float_to_half(y) if out_dtype == np.float16 else y
