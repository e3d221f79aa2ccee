"""The Python binding's argument checks, on the CPU: every wrapper rejects a
tensor of the wrong device, dtype, shape or element count before anything
reaches the C library (no pointer of a bad tensor is ever passed to a kernel).

The library is replaced by a recorder and the device test by "always on the
GPU", so the checks run on CPU tensors; a valid call must reach the recorder
exactly once, every invalid one must raise without reaching it."""
import pytest
import torch

import int8_quantization_amd as sq

F16, F32, I8, U8, I32 = torch.float16, torch.float32, torch.int8, torch.uint8, torch.int32


class Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(sq, "_lib", r)
    monkeypatch.setattr(sq, "_on_gpu", lambda t: True)
    monkeypatch.setattr(sq, "_stream", lambda: None)
    return r


def t(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


M, N, K = 4, 6, 32


def _valid():
    """Valid arguments for every wrapper, as (function name, kwargs)."""
    ws = t(4096, U8)
    return {
        "sq_smooth_scales": dict(X_cal=t((M, K), F16), W=t((N, K), F32), alpha=0.5, act_max=t(K, F32), s=t(K, F32)),
        "sq_quantize_per_token": dict(X=t((M, K), F16), s=t(K, F32), Xq=t((M, K), I8), x_scale=t(M, F32)),
        "sq_quantize_weight": dict(W=t((N, K), F16), s=None, gran=0, Wq=t((N, K), I8), w_scale=t(N, F32), ws=ws),
        "w8a8_gemm_dequant": dict(Xq=t((M, K), I8), x_scale=t(M, F32), Wq=t((N, K), I8), w_scale=t(1, F32), gran=1,
                                  bias=t(N, F32), Y=t((M, N), F16), acc_out=t((M, N), I32)),
        "int8_outlier_matmul": dict(X=t((M, K), F16), W16=t((N, K), F16), Wq=t((N, K), I8), w_scale=t(N, F32),
                                    bias=None, threshold=6.0, Y=t((M, N), F16), ws=ws, n_outliers=t(1, I32),
                                    outlier_idx=t(K, I32), acc_out=t((M, N), I32)),
        "sq_fold_smoothing_layernorm": dict(gamma=t(K, F32), beta=t(K, F32), s=t(K, F32), gamma_out=t(K, F32),
                                            beta_out=t(K, F32)),
        "sq_layernorm_quantize_per_token": dict(X=t((M, K), F16), gamma=t(K, F32), beta=None, eps=1e-5,
                                                Xq=t((M, K), I8), x_scale=t(M, F32)),
        "sq_calibrate_static_scale": dict(X_cal=t((M, K), F32), s=t(K, F32), percentile=99.9, x_scale=t(1, F32),
                                          ws=ws),
        "sq_quantize_static": dict(X=t((M, K), F16), s=None, x_scale=t(1, F32), Xq=t((M, K), I8),
                                   x_scale_rows=t(M, F32)),
        "sq_kv_calibrate_per_head": dict(KV=t((M, 2, 16), F16), margin=1.2, scale=t(2, F32)),
        "sq_kv_quantize_per_head": dict(KV=t((M, 2, 16), F16), scale=t(2, F32), q=t((M, 2, 16), I8)),
        "sq_dequantize": dict(q=t((M, K), I8), scale=t(M * 2, F32), scale_row_stride=2, group=16, Y=t((M, K), F32)),
        "sq_quantize_per_token_fp8": dict(X=t((M, K), F32), s=None, Xq=t((M, K), U8), x_scale=t(M, F32)),
        "sq_quantize_weight_fp8": dict(W=t((N, K), F16), s=t(K, F32), gran=1, Wq=t((N, K), U8), w_scale=t(1, F32),
                                       ws=ws),
        "fp8_gemm_dequant": dict(Xq=t((M, K), U8), x_scale=t(M, F32), Wq=t((N, K), U8), w_scale=t(N, F32), gran=0,
                                 bias=None, Y=t((M, N), F32), acc_out=t((M, N), F32)),
        "sq_w8a8_linear": dict(X=t((M, K), F16), s=t(K, F32), Wq=t((N, K), I8), w_scale=t(N, F32), gran=0,
                               bias=t(N, F32), Y=t((M, N), F16), ws=ws, x_scale=t(M, F32)),
        "sq_w8a8_linear_noalloc": dict(X=t((M, K), F32), s=None, Wq=t((N, K), I8), w_scale=t(1, F32), gran=1,
                                       bias=None, Y=t((M, N), F32), x_scale=None),
        "sq_quantize_per_token_asym": dict(X=t((M, K), F16), s=t(K, F32), Xq=t((M, K), I8), x_scale=t(M, F32),
                                           x_zero=t(M, I32)),
        "sq_weight_rowsum": dict(Wq=t((N, K), I8), rowsum=t(N, I32)),
        "w8a8_asym_gemm_dequant": dict(Xq=t((M, K), I8), x_scale=t(M, F32), x_zero=t(M, I32), Wq=t((N, K), I8),
                                       w_scale=t(N, F32), gran=0, w_rowsum=t(N, I32), bias=None, Y=t((M, N), F16),
                                       acc_out=t((M, N), I32)),
    }


# (function, argument, bad value) -- each must raise before the library is called
BAD = [
    ("sq_smooth_scales", "act_max", t(K, F16)),
    ("sq_smooth_scales", "X_cal", t((M, K + 16), F16)),
    ("sq_smooth_scales", "W", t((N, K - 16), F32)),
    ("sq_smooth_scales", "s", t(K - 1, F32)),
    ("sq_smooth_scales", "s", None),
    ("sq_smooth_scales", "X_cal", t((M, K), I8)),
    ("sq_quantize_per_token", "X", t((M, K), I8)),
    ("sq_quantize_per_token", "X", t((M * K,), F16)),
    ("sq_quantize_per_token", "Xq", t((M, K), U8)),
    ("sq_quantize_per_token", "Xq", t((M, K + 16), I8)),
    ("sq_quantize_per_token", "x_scale", t(M - 1, F32)),
    ("sq_quantize_per_token", "x_scale", t(M, F16)),
    ("sq_quantize_per_token", "s", t(K + 1, F32)),
    ("sq_quantize_per_token", "X", t((K, M), F16).t()),              # not contiguous
    ("sq_quantize_weight", "w_scale", t(1, F32)),                      # per-channel needs N scales
    ("sq_quantize_weight", "gran", 2),
    ("sq_quantize_weight", "Wq", t((N, K), I32)),
    ("sq_quantize_weight", "ws", [0]),
    ("w8a8_gemm_dequant", "Wq", t((N, K + 16), I8)),                   # K differs from Xq's
    ("w8a8_gemm_dequant", "x_scale", t(M + 1, F32)),
    ("w8a8_gemm_dequant", "w_scale", t(N, F32)),                       # per-tensor needs one scale
    ("w8a8_gemm_dequant", "bias", t(N - 1, F32)),
    ("w8a8_gemm_dequant", "Y", t((M, N + 1), F16)),
    ("w8a8_gemm_dequant", "Y", t((M, N), I32)),
    ("w8a8_gemm_dequant", "acc_out", t((M, N), F32)),
    ("w8a8_gemm_dequant", "acc_out", t((M, N - 1), I32)),
    ("w8a8_gemm_dequant", "Xq", t((M, K), U8)),
    ("int8_outlier_matmul", "X", t((M, K), F32)),                      # the side product reads fp16
    ("int8_outlier_matmul", "W16", t((N, K), F32)),
    ("int8_outlier_matmul", "W16", t((N, K + 16), F16)),
    ("int8_outlier_matmul", "Wq", t((N - 1, K), I8)),
    ("int8_outlier_matmul", "w_scale", t(1, F32)),
    ("int8_outlier_matmul", "Y", t((M, N), F32)),
    ("int8_outlier_matmul", "ws", None),
    ("int8_outlier_matmul", "outlier_idx", t(K - 1, I32)),
    ("int8_outlier_matmul", "n_outliers", t(1, F32)),
    ("int8_outlier_matmul", "acc_out", t((M, N + 1), I32)),
    ("sq_fold_smoothing_layernorm", "s", t(K - 1, F32)),
    ("sq_fold_smoothing_layernorm", "beta_out", None),
    ("sq_fold_smoothing_layernorm", "gamma_out", t(K, F16)),
    ("sq_layernorm_quantize_per_token", "X", t((M, K), F32)),
    ("sq_layernorm_quantize_per_token", "gamma", t(K + 1, F32)),
    ("sq_layernorm_quantize_per_token", "Xq", t((M, K), U8)),
    ("sq_calibrate_static_scale", "x_scale", t(0, F32)),
    ("sq_calibrate_static_scale", "ws", None),
    ("sq_quantize_static", "x_scale_rows", t(M - 1, F32)),
    ("sq_quantize_static", "Xq", t((M, K - 16), I8)),
    ("sq_kv_calibrate_per_head", "scale", t(3, F32)),
    ("sq_kv_calibrate_per_head", "KV", t((M, 32), F16)),
    ("sq_kv_quantize_per_head", "q", t((M, 2, 32), I8)),
    ("sq_dequantize", "scale", t(M * 2 - 1, F32)),                     # too few scales for the stride
    ("sq_dequantize", "Y", t((M, K - 16), F16)),
    ("sq_dequantize", "q", t((M, K), U8)),
    ("sq_dequantize", "group", 5),
    ("sq_quantize_per_token_fp8", "Xq", t((M, K), I8)),
    ("sq_quantize_weight_fp8", "w_scale", t(N, F32)),
    ("fp8_gemm_dequant", "Xq", t((M, K), I8)),
    ("fp8_gemm_dequant", "acc_out", t((M, N), I32)),
    ("sq_quantize_per_token_asym", "x_zero", t(M, F32)),
    ("sq_quantize_per_token_asym", "x_zero", t(M - 1, I32)),
    ("sq_quantize_per_token_asym", "Xq", t((M, K), U8)),
    ("sq_weight_rowsum", "rowsum", t(N + 1, I32)),
    ("sq_weight_rowsum", "Wq", t((N, K), U8)),
    ("w8a8_asym_gemm_dequant", "x_zero", None),
    ("w8a8_asym_gemm_dequant", "w_rowsum", t(N - 1, I32)),
    ("w8a8_asym_gemm_dequant", "w_rowsum", t(N, F32)),
    ("w8a8_asym_gemm_dequant", "Wq", t((N, K + 16), I8)),
    ("sq_w8a8_linear", "Wq", t((N, K + 16), I8)),
    ("sq_w8a8_linear", "x_scale", t(M + 1, F32)),
    ("sq_w8a8_linear", "Y", t((M + 1, N), F16)),
    ("sq_w8a8_linear", "ws", None),
    ("sq_w8a8_linear", "w_scale", t(N, F16)),
    ("sq_w8a8_linear_noalloc", "Wq", t((N, K - 16), I8)),
    ("sq_w8a8_linear_noalloc", "Y", t((M, N), I8)),
    ("sq_w8a8_linear_noalloc", "x_scale", t(M - 1, F32)),
    ("sq_w8a8_linear_noalloc", "w_scale", t(N, F32)),
]


@pytest.mark.parametrize("fn", sorted(_valid()))
def test_valid_call_reaches_the_library(rec, fn):
    getattr(sq, fn)(**_valid()[fn])
    assert rec.calls == [fn]


@pytest.mark.parametrize("fn,arg,bad", BAD, ids=[f"{f}-{a}-{i}" for i, (f, a, _) in enumerate(BAD)])
def test_bad_argument_raises_before_the_library(rec, fn, arg, bad):
    kwargs = _valid()[fn]
    kwargs[arg] = bad
    with pytest.raises((ValueError, TypeError)):
        getattr(sq, fn)(**kwargs)
    assert rec.calls == []


def test_every_wrapper_is_covered():
    assert set(_valid()) == set(sq.EXPORTS) - {"sq_status_string", "sq_workspace_size"}
    assert {f for f, _, _ in BAD} == set(_valid())


def test_host_tensor_is_refused(monkeypatch):
    """With the real device test: a host tensor never reaches the library (its address
    would be a host pointer handed to a kernel)."""
    r = Recorder()
    monkeypatch.setattr(sq, "_lib", r)
    with pytest.raises(ValueError, match="current GPU"):
        sq.sq_quantize_per_token(t((M, K), F16), None, t((M, K), I8), t(M, F32))
    assert r.calls == []
