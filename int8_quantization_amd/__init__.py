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
        "sq_w8a8_linear_noalloc": (I, [P, I, I64, I64, P, P, P, I, P, I64, P, I, P, P]),
        "sq_quantize_per_token_fp8": (I, [P, I, I64, I64, P, P, P, P]),
        "sq_quantize_weight_fp8": (I, [P, I, I64, I64, P, I, P, P, P, SZ, P]),
        "fp8_gemm_dequant": (I, [P, P, P, P, I, P, I64, I64, I64, P, I, P, P]),
        "sq_quantize_per_token_asym": (I, [P, I, I64, I64, P, P, P, P, P]),
        "sq_weight_rowsum": (I, [P, I64, I64, P, P]),
        "w8a8_asym_gemm_dequant": (I, [P, P, P, P, P, I, P, P, I64, I64, I64, P, I, P, P]),
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
           "sq_quantize_weight_fp8", "fp8_gemm_dequant", "sq_w8a8_linear", "sq_w8a8_linear_noalloc",
           "sq_quantize_per_token_asym", "sq_weight_rowsum", "w8a8_asym_gemm_dequant")


def _p(t):
    return None if t is None else t.data_ptr()


def _dt(t):
    if t.dtype == torch.float16:
        return SQ_F16
    if t.dtype == torch.float32:
        return SQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


# The current stream's raw handle without building a torch.cuda.Stream object (a few
# microseconds per call, which small kernels would otherwise wait for on the host).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream():
    if _raw_stream is not None:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _on_gpu(t):
    """True when t lives on the current GPU (the device the library launches on)."""
    return t.is_cuda and t.get_device() == torch.cuda.current_device()


F16, F32, I8, U8, I32 = torch.float16, torch.float32, torch.int8, torch.uint8, torch.int32
FLOAT = (F16, F32)


def _need(fn, name, t, dtypes, shape=None, numel=None, min_numel=None, ndim=None, optional=False):
    """Checks one tensor argument before anything reaches the library: present (unless
    optional), on the current GPU, contiguous, of an accepted dtype, and of the shape or
    element count the call implies.  Raises ValueError (TypeError for a non-tensor)."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{fn}: {name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{fn}: {name} must be a torch.Tensor, got {type(t).__name__}")
    if not _on_gpu(t):
        raise ValueError(f"{fn}: {name} must be on the current GPU, got device {t.device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{fn}: {name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{fn}: {name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{fn}: {name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{fn}: {name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{fn}: {name} must hold {numel} elements, got {t.numel()}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{fn}: {name} must hold at least {min_numel} elements, got {t.numel()}")


def _workspace(fn, ws):
    """A workspace is any contiguous tensor on the current GPU; its byte size goes to the
    library, which rejects one that is too small."""
    if ws is None:
        raise ValueError(f"{fn}: workspace is required")
    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"{fn}: workspace must be a torch.Tensor")
    if not _on_gpu(ws):
        raise ValueError(f"{fn}: workspace must be on the current GPU, got device {ws.device}")
    if not ws.is_contiguous():
        raise ValueError(f"{fn}: workspace must be contiguous")
    return ws.numel() * ws.element_size()


def _gran(fn, gran, N):
    if int(gran) not in (SQ_PER_CHANNEL, SQ_PER_TENSOR):
        raise ValueError(f"{fn}: gran must be 0 (per channel) or 1 (per tensor), got {gran}")
    return N if int(gran) == SQ_PER_CHANNEL else 1


def _check(fn, code):
    if code != 0:
        raise SqError(fn, code)


def sq_status_string(code: int) -> str:
    return _lib.sq_status_string(int(code)).decode()


def sq_workspace_size(op: int, M: int, N: int, K: int) -> int:
    return int(_lib.sq_workspace_size(int(op), int(M), int(N), int(K)))


def sq_smooth_scales(X_cal, W, alpha, act_max, s):
    """act_max [K] fp32 (running max, in/out); s [K] fp32 out. X_cal or W may be None."""
    fn = "sq_smooth_scales"
    _need(fn, "act_max", act_max, (F32,), ndim=1)
    K = act_max.shape[0]
    _need(fn, "X_cal", X_cal, FLOAT, ndim=2, optional=True)
    if X_cal is not None and X_cal.shape[1] != K:
        raise ValueError(f"{fn}: X_cal has {X_cal.shape[1]} columns, act_max {K}")
    _need(fn, "W", W, FLOAT, ndim=2, optional=True)
    if W is not None and W.shape[1] != K:
        raise ValueError(f"{fn}: W has {W.shape[1]} columns, act_max {K}")
    _need(fn, "s", s, (F32,), numel=K, optional=W is None)
    Mc = 0 if X_cal is None else X_cal.shape[0]
    N = 0 if W is None else W.shape[0]
    _check(fn, _lib.sq_smooth_scales(
        _p(X_cal), SQ_F32 if X_cal is None else _dt(X_cal), Mc, _p(W), SQ_F32 if W is None else _dt(W),
        N, K, float(alpha), _p(act_max), _p(s), _stream()))


def _rows_in(fn, X, s, dtypes=FLOAT):
    """[M, K] activation (or weight) rows and the optional smoothing vector s [K]."""
    _need(fn, "X", X, dtypes, ndim=2)
    M, K = X.shape
    _need(fn, "s", s, (F32,), numel=K, optional=True)
    return M, K


def sq_quantize_per_token(X, s, Xq, x_scale):
    fn = "sq_quantize_per_token"
    M, K = _rows_in(fn, X, s)
    _need(fn, "Xq", Xq, (I8,), shape=(M, K))
    _need(fn, "x_scale", x_scale, (F32,), numel=M)
    _check(fn, _lib.sq_quantize_per_token(_p(X), _dt(X), M, K, _p(s), _p(Xq), _p(x_scale), _stream()))


def sq_quantize_weight(W, s, gran, Wq, w_scale, ws=None):
    fn = "sq_quantize_weight"
    N, K = _rows_in(fn, W, s)
    _need(fn, "Wq", Wq, (I8,), shape=(N, K))
    _need(fn, "w_scale", w_scale, (F32,), numel=_gran(fn, gran, N))
    nbytes = 0 if ws is None else _workspace(fn, ws)
    _check(fn, _lib.sq_quantize_weight(
        _p(W), _dt(W), N, K, _p(s), int(gran), _p(Wq), _p(w_scale), _p(ws), nbytes, _stream()))


def _gemm_args(fn, Xq, x_scale, Wq, w_scale, gran, bias, Y, acc_out, code_dtype, acc_dtype):
    _need(fn, "Xq", Xq, (code_dtype,), ndim=2)
    M, K = Xq.shape
    _need(fn, "Wq", Wq, (code_dtype,), ndim=2)
    N = Wq.shape[0]
    if Wq.shape[1] != K:
        raise ValueError(f"{fn}: Wq has {Wq.shape[1]} columns, Xq {K}")
    _need(fn, "x_scale", x_scale, (F32,), numel=M)
    _need(fn, "w_scale", w_scale, (F32,), numel=_gran(fn, gran, N))
    _need(fn, "bias", bias, (F32,), numel=N, optional=True)
    _need(fn, "Y", Y, FLOAT, shape=(M, N))
    _need(fn, "acc_out", acc_out, (acc_dtype,), shape=(M, N), optional=True)
    return M, N, K


def w8a8_gemm_dequant(Xq, x_scale, Wq, w_scale, gran, bias, Y, acc_out=None):
    fn = "w8a8_gemm_dequant"
    M, N, K = _gemm_args(fn, Xq, x_scale, Wq, w_scale, gran, bias, Y, acc_out, I8, I32)
    _check(fn, _lib.w8a8_gemm_dequant(
        _p(Xq), _p(x_scale), _p(Wq), _p(w_scale), int(gran), _p(bias), M, N, K, _p(Y), _dt(Y),
        _p(acc_out), _stream()))


def int8_outlier_matmul(X, W16, Wq, w_scale, bias, threshold, Y, ws, n_outliers=None,
                        outlier_idx=None, acc_out=None):
    fn = "int8_outlier_matmul"
    _need(fn, "X", X, (F16,), ndim=2)
    M, K = X.shape
    _need(fn, "W16", W16, (F16,), ndim=2)
    N = W16.shape[0]
    if W16.shape[1] != K:
        raise ValueError(f"{fn}: W16 has {W16.shape[1]} columns, X {K}")
    _need(fn, "Wq", Wq, (I8,), shape=(N, K))
    _need(fn, "w_scale", w_scale, (F32,), numel=N)
    _need(fn, "bias", bias, (F32,), numel=N, optional=True)
    _need(fn, "Y", Y, (F16,), shape=(M, N))
    _need(fn, "n_outliers", n_outliers, (I32,), min_numel=1, optional=True)
    _need(fn, "outlier_idx", outlier_idx, (I32,), min_numel=K, optional=True)
    _need(fn, "acc_out", acc_out, (I32,), shape=(M, N), optional=True)
    nbytes = _workspace(fn, ws)
    _check(fn, _lib.int8_outlier_matmul(
        _p(X), _p(W16), _p(Wq), _p(w_scale), _p(bias), M, N, K, float(threshold), _p(Y), _p(ws),
        nbytes, _p(n_outliers), _p(outlier_idx), _p(acc_out), _stream()))


def sq_fold_smoothing_layernorm(gamma, beta, s, gamma_out, beta_out=None):
    fn = "sq_fold_smoothing_layernorm"
    _need(fn, "gamma", gamma, (F32,), ndim=1)
    K = gamma.numel()
    _need(fn, "s", s, (F32,), numel=K)
    _need(fn, "gamma_out", gamma_out, (F32,), numel=K)
    _need(fn, "beta", beta, (F32,), numel=K, optional=True)
    _need(fn, "beta_out", beta_out, (F32,), numel=K, optional=beta is None)
    if beta is None and beta_out is not None:
        raise ValueError(f"{fn}: beta_out given without beta")
    _check(fn, _lib.sq_fold_smoothing_layernorm(
        _p(gamma), _p(beta), _p(s), K, _p(gamma_out), _p(beta_out), _stream()))


def sq_layernorm_quantize_per_token(X, gamma, beta, eps, Xq, x_scale):
    fn = "sq_layernorm_quantize_per_token"
    _need(fn, "X", X, (F16,), ndim=2)
    M, K = X.shape
    _need(fn, "gamma", gamma, (F32,), numel=K)
    _need(fn, "beta", beta, (F32,), numel=K, optional=True)
    _need(fn, "Xq", Xq, (I8,), shape=(M, K))
    _need(fn, "x_scale", x_scale, (F32,), numel=M)
    _check(fn, _lib.sq_layernorm_quantize_per_token(
        _p(X), _dt(X), M, K, _p(gamma), _p(beta), float(eps), _p(Xq), _p(x_scale), _stream()))


def sq_calibrate_static_scale(X_cal, s, percentile, x_scale, ws):
    fn = "sq_calibrate_static_scale"
    M, K = _rows_in(fn, X_cal, s)
    _need(fn, "x_scale", x_scale, (F32,), min_numel=1)
    nbytes = _workspace(fn, ws)
    _check(fn, _lib.sq_calibrate_static_scale(
        _p(X_cal), _dt(X_cal), M, K, _p(s), float(percentile), _p(x_scale), _p(ws), nbytes, _stream()))


def sq_quantize_static(X, s, x_scale, Xq, x_scale_rows=None):
    fn = "sq_quantize_static"
    M, K = _rows_in(fn, X, s)
    _need(fn, "x_scale", x_scale, (F32,), min_numel=1)
    _need(fn, "Xq", Xq, (I8,), shape=(M, K))
    _need(fn, "x_scale_rows", x_scale_rows, (F32,), numel=M, optional=True)
    _check(fn, _lib.sq_quantize_static(
        _p(X), _dt(X), M, K, _p(s), _p(x_scale), _p(Xq), _p(x_scale_rows), _stream()))


def sq_kv_calibrate_per_head(KV, margin, scale):
    """KV [T, H, D] fp16/fp32; scale [H] fp32 out."""
    fn = "sq_kv_calibrate_per_head"
    _need(fn, "KV", KV, FLOAT, ndim=3)
    T, H, D = KV.shape
    _need(fn, "scale", scale, (F32,), numel=H)
    _check(fn, _lib.sq_kv_calibrate_per_head(
        _p(KV), _dt(KV), T, H, D, float(margin), _p(scale), _stream()))


def sq_kv_quantize_per_head(KV, scale, q):
    """KV [T, H, D] fp16/fp32; scale [H] fp32; q [T, H, D] int8 out."""
    fn = "sq_kv_quantize_per_head"
    _need(fn, "KV", KV, FLOAT, ndim=3)
    T, H, D = KV.shape
    _need(fn, "scale", scale, (F32,), numel=H)
    _need(fn, "q", q, (I8,), shape=(T, H, D))
    _check(fn, _lib.sq_kv_quantize_per_head(
        _p(KV), _dt(KV), T, H, D, _p(scale), _p(q), _stream()))


def sq_dequantize(q, scale, scale_row_stride, group, Y):
    """q [M, K] int8 (or any shape whose last dimension is K); Y fp16/fp32 out with as many
    elements, in the same row-major order."""
    fn = "sq_dequantize"
    _need(fn, "q", q, (I8,))
    if q.dim() < 1 or q.numel() == 0:
        raise ValueError(f"{fn}: q must be non-empty")
    K = q.shape[-1]
    M = q.numel() // K
    _need(fn, "Y", Y, FLOAT, numel=q.numel())
    group, stride = int(group), int(scale_row_stride)
    if group <= 0 or K % group != 0 or stride < 0:
        raise ValueError(f"{fn}: group must divide K = {K} and the row stride be >= 0")
    _need(fn, "scale", scale, (F32,), min_numel=(M - 1) * stride + K // group)
    _check(fn, _lib.sq_dequantize(
        _p(q), M, K, _p(scale), stride, group, _p(Y), _dt(Y), _stream()))


def sq_quantize_per_token_fp8(X, s, Xq, x_scale):
    """Xq: uint8 [M, K] (FP8 E4M3 code bytes) out; x_scale fp32 [M] out."""
    fn = "sq_quantize_per_token_fp8"
    M, K = _rows_in(fn, X, s)
    _need(fn, "Xq", Xq, (U8,), shape=(M, K))
    _need(fn, "x_scale", x_scale, (F32,), numel=M)
    _check(fn, _lib.sq_quantize_per_token_fp8(
        _p(X), _dt(X), M, K, _p(s), _p(Xq), _p(x_scale), _stream()))


def sq_quantize_weight_fp8(W, s, gran, Wq, w_scale, ws=None):
    fn = "sq_quantize_weight_fp8"
    N, K = _rows_in(fn, W, s)
    _need(fn, "Wq", Wq, (U8,), shape=(N, K))
    _need(fn, "w_scale", w_scale, (F32,), numel=_gran(fn, gran, N))
    nbytes = 0 if ws is None else _workspace(fn, ws)
    _check(fn, _lib.sq_quantize_weight_fp8(
        _p(W), _dt(W), N, K, _p(s), int(gran), _p(Wq), _p(w_scale), _p(ws), nbytes, _stream()))


def fp8_gemm_dequant(Xq, x_scale, Wq, w_scale, gran, bias, Y, acc_out=None):
    """Xq uint8 [M, K], Wq uint8 [N, K] (FP8 E4M3 codes); Y fp16/fp32 [M, N]; acc_out fp32 [M, N]."""
    fn = "fp8_gemm_dequant"
    M, N, K = _gemm_args(fn, Xq, x_scale, Wq, w_scale, gran, bias, Y, acc_out, U8, F32)
    _check(fn, _lib.fp8_gemm_dequant(
        _p(Xq), _p(x_scale), _p(Wq), _p(w_scale), int(gran), _p(bias), M, N, K, _p(Y), _dt(Y),
        _p(acc_out), _stream()))


def sq_quantize_per_token_asym(X, s, Xq, x_scale, x_zero):
    """Zero-point per-token codes: Xq int8 [M, K], x_scale fp32 [M], x_zero int32 [M] out."""
    fn = "sq_quantize_per_token_asym"
    M, K = _rows_in(fn, X, s)
    _need(fn, "Xq", Xq, (I8,), shape=(M, K))
    _need(fn, "x_scale", x_scale, (F32,), numel=M)
    _need(fn, "x_zero", x_zero, (I32,), numel=M)
    _check(fn, _lib.sq_quantize_per_token_asym(
        _p(X), _dt(X), M, K, _p(s), _p(Xq), _p(x_scale), _p(x_zero), _stream()))


def sq_weight_rowsum(Wq, rowsum):
    """rowsum int32 [N] out: the sum of each row of Wq int8 [N, K]."""
    fn = "sq_weight_rowsum"
    _need(fn, "Wq", Wq, (I8,), ndim=2)
    N, K = Wq.shape
    _need(fn, "rowsum", rowsum, (I32,), numel=N)
    _check(fn, _lib.sq_weight_rowsum(_p(Wq), N, K, _p(rowsum), _stream()))


def w8a8_asym_gemm_dequant(Xq, x_scale, x_zero, Wq, w_scale, gran, w_rowsum, bias, Y, acc_out=None):
    """The int8 GEMM with zero-point activations; acc_out int32 [M, N] receives the corrected accumulators."""
    fn = "w8a8_asym_gemm_dequant"
    M, N, K = _gemm_args(fn, Xq, x_scale, Wq, w_scale, gran, bias, Y, acc_out, I8, I32)
    _need(fn, "x_zero", x_zero, (I32,), numel=M)
    _need(fn, "w_rowsum", w_rowsum, (I32,), numel=N)
    _check(fn, _lib.w8a8_asym_gemm_dequant(
        _p(Xq), _p(x_scale), _p(x_zero), _p(Wq), _p(w_scale), int(gran), _p(w_rowsum), _p(bias), M, N, K, _p(Y),
        _dt(Y), _p(acc_out), _stream()))


def sq_w8a8_linear(X, s, Wq, w_scale, gran, bias, Y, ws, x_scale=None):
    """Per-token quantization of X (with smoothing s) and the W8A8 GEMM + dequant in one call."""
    fn = "sq_w8a8_linear"
    M, K = _rows_in(fn, X, s)
    _need(fn, "Wq", Wq, (I8,), ndim=2)
    N = Wq.shape[0]
    if Wq.shape[1] != K:
        raise ValueError(f"{fn}: Wq has {Wq.shape[1]} columns, X {K}")
    _need(fn, "w_scale", w_scale, (F32,), numel=_gran(fn, gran, N))
    _need(fn, "bias", bias, (F32,), numel=N, optional=True)
    _need(fn, "Y", Y, FLOAT, shape=(M, N))
    _need(fn, "x_scale", x_scale, (F32,), numel=M, optional=True)
    nbytes = _workspace(fn, ws)
    _check(fn, _lib.sq_w8a8_linear(
        _p(X), _dt(X), M, K, _p(s), _p(Wq), _p(w_scale), int(gran), _p(bias), N, _p(Y), _dt(Y), _p(x_scale),
        _p(ws), nbytes, _stream()))


SQ_NOALLOC_XQ_BYTES = 16 << 20
SQ_NOALLOC_MAX_M = 16384


def sq_w8a8_linear_noalloc(X, s, Wq, w_scale, gran, bias, Y, x_scale=None):
    """sq_w8a8_linear without a workspace: the library's own fixed device scratch holds Xq
    (M * K <= 16 MiB; M <= 16384 when x_scale is None).  Calls that can overlap on one GPU
    share that scratch and must be ordered by the caller."""
    fn = "sq_w8a8_linear_noalloc"
    M, K = _rows_in(fn, X, s)
    _need(fn, "Wq", Wq, (I8,), ndim=2)
    N = Wq.shape[0]
    if Wq.shape[1] != K:
        raise ValueError(f"{fn}: Wq has {Wq.shape[1]} columns, X {K}")
    _need(fn, "w_scale", w_scale, (F32,), numel=_gran(fn, gran, N))
    _need(fn, "bias", bias, (F32,), numel=N, optional=True)
    _need(fn, "Y", Y, FLOAT, shape=(M, N))
    _need(fn, "x_scale", x_scale, (F32,), numel=M, optional=True)
    _check(fn, _lib.sq_w8a8_linear_noalloc(
        _p(X), _dt(X), M, K, _p(s), _p(Wq), _p(w_scale), int(gran), _p(bias), N, _p(Y), _dt(Y), _p(x_scale),
        _stream()))
