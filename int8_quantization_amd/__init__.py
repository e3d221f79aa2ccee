"""MI355X (gfx950) quantized INT8 linear layer -- Python binding of libsq.so.

Every function here marshals torch tensors (device memory, the current HIP
stream) into the C ABI declared in include/sq.h and raises SqError on a
non-zero status.  All computation happens in the HIP kernels of libsq.so; if
the library is missing, importing the binding fails loudly -- there is no
fallback.

Names match the C entry points:
  sq_smooth_scales, sq_quantize_per_token, sq_quantize_weight,
  w8a8_gemm_dequant, int8_outlier_matmul, sq_workspace_size, sq_status_string.
"""
import ctypes as C
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsq.so")

SQ_F32, SQ_F16 = 0, 1
SQ_PER_CHANNEL, SQ_PER_TENSOR = 0, 1
SQ_OP_QUANT_WEIGHT, SQ_OP_OUTLIER, SQ_OP_CALIB_STATIC, SQ_OP_LINEAR = 0, 1, 2, 3


class SqError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn}: {sq_status_string(code)} (status {code})")
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950)")
    lib = C.CDLL(LIB_PATH)
    P, I64, F, I, SZ = C.c_void_p, C.c_int64, C.c_float, C.c_int, C.c_size_t
    sigs = {
        "sq_status_string": (C.c_char_p, [I]),
        "sq_workspace_size": (SZ, [I, I64, I64, I64]),
        "sq_smooth_scales": (I, [P, I, I64, P, I, I64, I64, F, P, P, P]),
        "sq_quantize_per_token": (I, [P, I, I64, I64, P, P, P, P]),
        "sq_quantize_weight": (I, [P, I, I64, I64, P, I, P, P, P, SZ, P]),
        "w8a8_gemm_dequant": (I, [P, P, P, P, I, P, I64, I64, I64, P, I, P, P]),
        "int8_outlier_matmul": (I, [P, P, P, P, P, I64, I64, I64, F, P, P, SZ, P, P, P, P]),
        "sq_fold_smoothing_layernorm": (I, [P, P, P, I64, P, P, P]),
        "sq_layernorm_quantize_per_token": (I, [P, I, I64, I64, P, P, F, P, P, P]),
        "sq_calibrate_static_scale": (I, [P, I, I64, I64, P, C.c_double, P, P, SZ, P]),
        "sq_quantize_static": (I, [P, I, I64, I64, P, P, P, P, P]),
        "sq_w8a8_linear": (I, [P, I, I64, I64, P, P, P, I, P, I64, P, I, P, P, SZ, P]),
        "sq_quantize_per_token_fp8": (I, [P, I, I64, I64, P, P, P, P]),
        "sq_quantize_weight_fp8": (I, [P, I, I64, I64, P, I, P, P, P, SZ, P]),
        "fp8_gemm_dequant": (I, [P, P, P, P, I, P, I64, I64, I64, P, I, P, P]),
        "sq_kv_calibrate_per_head": (I, [P, I, I64, I64, I64, F, P, P]),
        "sq_kv_quantize_per_head": (I, [P, I, I64, I64, I64, P, P, P]),
        "sq_dequantize": (I, [P, I64, I64, P, I64, I64, P, I, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()

EXPORTS = ("sq_status_string", "sq_workspace_size", "sq_smooth_scales", "sq_quantize_per_token",
           "sq_quantize_weight", "w8a8_gemm_dequant", "int8_outlier_matmul", "sq_fold_smoothing_layernorm",
           "sq_layernorm_quantize_per_token", "sq_calibrate_static_scale", "sq_quantize_static",
           "sq_kv_calibrate_per_head", "sq_kv_quantize_per_head", "sq_dequantize", "sq_quantize_per_token_fp8",
           "sq_quantize_weight_fp8", "fp8_gemm_dequant", "sq_w8a8_linear")


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _dt(t):
    if t.dtype == torch.float16:
        return SQ_F16
    if t.dtype == torch.float32:
        return SQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dense(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _check(fn, code):
    if code != 0:
        raise SqError(fn, code)


def sq_status_string(code: int) -> str:
    return _lib.sq_status_string(int(code)).decode()


def sq_workspace_size(op: int, M: int, N: int, K: int) -> int:
    return int(_lib.sq_workspace_size(int(op), int(M), int(N), int(K)))


def sq_smooth_scales(X_cal, W, alpha, act_max, s):
    """act_max [K] fp32 (running max, in/out); s [K] fp32 out. X_cal or W may be None."""
    _dense(X_cal, W, act_max, s)
    K = act_max.shape[0]
    Mc = 0 if X_cal is None else X_cal.shape[0]
    N = 0 if W is None else W.shape[0]
    _check("sq_smooth_scales", _lib.sq_smooth_scales(
        _p(X_cal), SQ_F32 if X_cal is None else _dt(X_cal), Mc, _p(W), SQ_F32 if W is None else _dt(W),
        N, K, float(alpha), _p(act_max), _p(s), _stream()))


def sq_quantize_per_token(X, s, Xq, x_scale):
    _dense(X, s, Xq, x_scale)
    M, K = X.shape
    _check("sq_quantize_per_token", _lib.sq_quantize_per_token(
        _p(X), _dt(X), M, K, _p(s), _p(Xq), _p(x_scale), _stream()))


def sq_quantize_weight(W, s, gran, Wq, w_scale, ws=None):
    _dense(W, s, Wq, w_scale, ws)
    N, K = W.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("sq_quantize_weight", _lib.sq_quantize_weight(
        _p(W), _dt(W), N, K, _p(s), int(gran), _p(Wq), _p(w_scale), _p(ws), nbytes, _stream()))


def w8a8_gemm_dequant(Xq, x_scale, Wq, w_scale, gran, bias, Y, acc_out=None):
    _dense(Xq, x_scale, Wq, w_scale, bias, Y, acc_out)
    M, K = Xq.shape
    N = Wq.shape[0]
    _check("w8a8_gemm_dequant", _lib.w8a8_gemm_dequant(
        _p(Xq), _p(x_scale), _p(Wq), _p(w_scale), int(gran), _p(bias), M, N, K, _p(Y), _dt(Y),
        _p(acc_out), _stream()))


def int8_outlier_matmul(X, W16, Wq, w_scale, bias, threshold, Y, ws, n_outliers=None,
                        outlier_idx=None, acc_out=None):
    _dense(X, W16, Wq, w_scale, bias, Y, ws, n_outliers, outlier_idx, acc_out)
    M, K = X.shape
    N = W16.shape[0]
    nbytes = ws.numel() * ws.element_size()
    _check("int8_outlier_matmul", _lib.int8_outlier_matmul(
        _p(X), _p(W16), _p(Wq), _p(w_scale), _p(bias), M, N, K, float(threshold), _p(Y), _p(ws),
        nbytes, _p(n_outliers), _p(outlier_idx), _p(acc_out), _stream()))


def sq_fold_smoothing_layernorm(gamma, beta, s, gamma_out, beta_out=None):
    _dense(gamma, beta, s, gamma_out, beta_out)
    K = gamma.numel()
    _check("sq_fold_smoothing_layernorm", _lib.sq_fold_smoothing_layernorm(
        _p(gamma), _p(beta), _p(s), K, _p(gamma_out), _p(beta_out), _stream()))


def sq_layernorm_quantize_per_token(X, gamma, beta, eps, Xq, x_scale):
    _dense(X, gamma, beta, Xq, x_scale)
    M, K = X.shape
    _check("sq_layernorm_quantize_per_token", _lib.sq_layernorm_quantize_per_token(
        _p(X), _dt(X), M, K, _p(gamma), _p(beta), float(eps), _p(Xq), _p(x_scale), _stream()))


def sq_calibrate_static_scale(X_cal, s, percentile, x_scale, ws):
    _dense(X_cal, s, x_scale, ws)
    M, K = X_cal.shape
    nbytes = ws.numel() * ws.element_size()
    _check("sq_calibrate_static_scale", _lib.sq_calibrate_static_scale(
        _p(X_cal), _dt(X_cal), M, K, _p(s), float(percentile), _p(x_scale), _p(ws), nbytes, _stream()))


def sq_quantize_static(X, s, x_scale, Xq, x_scale_rows=None):
    _dense(X, s, x_scale, Xq, x_scale_rows)
    M, K = X.shape
    _check("sq_quantize_static", _lib.sq_quantize_static(
        _p(X), _dt(X), M, K, _p(s), _p(x_scale), _p(Xq), _p(x_scale_rows), _stream()))


def sq_kv_calibrate_per_head(KV, margin, scale):
    """KV [T, H, D] fp16/fp32; scale [H] fp32 out."""
    _dense(KV, scale)
    T, H, D = KV.shape
    _check("sq_kv_calibrate_per_head", _lib.sq_kv_calibrate_per_head(
        _p(KV), _dt(KV), T, H, D, float(margin), _p(scale), _stream()))


def sq_kv_quantize_per_head(KV, scale, q):
    """KV [T, H, D] fp16/fp32; scale [H] fp32; q [T, H, D] int8 out."""
    _dense(KV, scale, q)
    T, H, D = KV.shape
    _check("sq_kv_quantize_per_head", _lib.sq_kv_quantize_per_head(
        _p(KV), _dt(KV), T, H, D, _p(scale), _p(q), _stream()))


def sq_dequantize(q, scale, scale_row_stride, group, Y):
    """q [M, K] int8 (or any shape whose last dimension is K); Y the same shape, fp16/fp32 out."""
    _dense(q, Y)
    K = q.shape[-1]
    M = q.numel() // K
    _check("sq_dequantize", _lib.sq_dequantize(
        _p(q), M, K, _p(scale), int(scale_row_stride), int(group), _p(Y), _dt(Y), _stream()))


def sq_quantize_per_token_fp8(X, s, Xq, x_scale):
    """Xq: uint8 [M, K] (FP8 E4M3 code bytes) out; x_scale fp32 [M] out."""
    _dense(X, s, Xq, x_scale)
    M, K = X.shape
    _check("sq_quantize_per_token_fp8", _lib.sq_quantize_per_token_fp8(
        _p(X), _dt(X), M, K, _p(s), _p(Xq), _p(x_scale), _stream()))


def sq_quantize_weight_fp8(W, s, gran, Wq, w_scale, ws=None):
    _dense(W, s, Wq, w_scale, ws)
    N, K = W.shape
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check("sq_quantize_weight_fp8", _lib.sq_quantize_weight_fp8(
        _p(W), _dt(W), N, K, _p(s), int(gran), _p(Wq), _p(w_scale), _p(ws), nbytes, _stream()))


def fp8_gemm_dequant(Xq, x_scale, Wq, w_scale, gran, bias, Y, acc_out=None):
    """Xq uint8 [M, K], Wq uint8 [N, K] (FP8 E4M3 codes); Y fp16/fp32 [M, N]; acc_out fp32 [M, N]."""
    _dense(Xq, x_scale, Wq, w_scale, bias, Y, acc_out)
    M, K = Xq.shape
    N = Wq.shape[0]
    _check("fp8_gemm_dequant", _lib.fp8_gemm_dequant(
        _p(Xq), _p(x_scale), _p(Wq), _p(w_scale), int(gran), _p(bias), M, N, K, _p(Y), _dt(Y),
        _p(acc_out), _stream()))


def sq_w8a8_linear(X, s, Wq, w_scale, gran, bias, Y, ws, x_scale=None):
    """Per-token quantization of X (with smoothing s) and the W8A8 GEMM + dequant in one call."""
    _dense(X, s, Wq, w_scale, bias, Y, ws, x_scale)
    M, K = X.shape
    N = Wq.shape[0]
    nbytes = ws.numel() * ws.element_size()
    _check("sq_w8a8_linear", _lib.sq_w8a8_linear(
        _p(X), _dt(X), M, K, _p(s), _p(Wq), _p(w_scale), int(gran), _p(bias), N, _p(Y), _dt(Y), _p(x_scale),
        _p(ws), nbytes, _stream()))
