// C ABI of libsq: argument validation on the host, then kernel launches on the
// caller's stream.  No allocation, no host synchronization, no device-to-host copy.
#include <math.h>

#include <mutex>

#include "sq_internal.h"

using namespace sq;

// Scratch of sq_w8a8_linear_noalloc: the int8 codes of the activation rows, then their
// per-token scales.  Each GPU the library runs on holds its own copy from the code
// object's load until the process ends.  In host code this name is a host-side stand-in:
// kernels get the device address that scratch_base() looks up.
static __device__ __align__(256) int8_t scratch[SQ_NOALLOC_XQ_BYTES + 4 * SQ_NOALLOC_MAX_M];

namespace {

constexpr int64_t kMaxK = 131056;   // 127^2 * K < 2^31, K % 16 == 0
constexpr int64_t kMaxMN = (int64_t)1 << 30;

bool bad_shape(int64_t M, int64_t N, int64_t K) {
    return M < 1 || N < 1 || K < 16 || K > kMaxK || (K % 16) != 0 || M > kMaxMN || N > kMaxMN;
}
bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }
bool bad_dtype(int d) { return d != SQ_F32 && d != SQ_F16; }

sq_status hip_status(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_ERR_HIP; }

#define SQ_TRY(call)                                  \
    do {                                              \
        hipError_t e_ = (call);                       \
        if (e_ != hipSuccess) return SQ_ERR_HIP;      \
    } while (0)

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// LLM.int8() workspace layout (byte offsets), sized for K outlier columns.
struct OutlierLayout {
    size_t cmax, pos, idx, count, xs, xq, xo, total;
};
OutlierLayout outlier_layout(int64_t M, int64_t N, int64_t K) {
    OutlierLayout L;
    size_t o = 0;
    L.cmax = o;  o = align256(o + 4 * (size_t)K);
    L.pos = o;   o = align256(o + 4 * (size_t)K);
    L.idx = o;   o = align256(o + 4 * (size_t)K);
    L.count = o; o = align256(o + 16);
    L.xs = o;    o = align256(o + 4 * (size_t)M);
    L.xq = o;    o = align256(o + (size_t)M * (size_t)K);
    L.xo = o;    o = align256(o + 2 * (size_t)M * (size_t)K);
    L.total = o;
    (void)N;
    return L;
}

// Device address of `scratch` on the current device, looked up once per device (with
// that device current) by hipGetSymbolAddress; nullptr when the lookup failed.
int8_t* scratch_base() {
    constexpr int kMaxDevices = 64;
    static int8_t* base[kMaxDevices];
    static std::once_flag once[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::call_once(once[dev], [dev]() {
        void* p = nullptr;
        base[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess ? static_cast<int8_t*>(p) : nullptr;
    });
    return base[dev];
}

// The layer after validation: the fused decode kernel when it applies, else the
// quantizer into xq / xs and the GEMM (decode kernel for M <= 16).
sq_status linear_body(const void* X, int xdt, int64_t M, int64_t K, const float* s, const int8_t* Wq,
                      const float* w_scale, int g, const float* bias, int64_t N, void* Y, int ydt, float* x_scale,
                      int8_t* xq, float* xs, hipStream_t stream) {
    const int stride = g == SQ_PER_CHANNEL ? 1 : 0;
    SQ_TRY(launch_quant_rows(X, xdt, M, K, s, s ? 1 : 0, xq, xs, nullptr, nullptr, stream));
    if (M <= 16)
        return hip_status(launch_gemv(xq, xs, Wq, w_scale, stride, bias, M, N, K, Y, ydt, nullptr, nullptr, stream));
    return hip_status(launch_gemm(xq, xs, Wq, w_scale, stride, bias, M, N, K, Y, ydt, nullptr, nullptr, stream));
}

bool fused_decode(int xdt, int64_t M, int64_t K) { return xdt == SQ_F16 && M <= 2 && K <= 8192; }

}  // namespace

extern "C" {

const char* sq_status_string(int st) {
    switch (st) {
        case SQ_OK: return "SQ_OK";
        case SQ_ERR_NULL: return "SQ_ERR_NULL: a required pointer is NULL";
        case SQ_ERR_SHAPE: return "SQ_ERR_SHAPE: M, N >= 1 and 16 <= K <= 131056 with K % 16 == 0 are required";
        case SQ_ERR_ALIGN: return "SQ_ERR_ALIGN: pointers must be 16-byte aligned";
        case SQ_ERR_DTYPE: return "SQ_ERR_DTYPE: unsupported dtype or granularity";
        case SQ_ERR_VALUE:
            return "SQ_ERR_VALUE: alpha must be in [0,1]; threshold finite and >= 0; eps finite and > 0; "
                   "percentile in (0, 100]; margin finite and > 0";
        case SQ_ERR_WORKSPACE: return "SQ_ERR_WORKSPACE: workspace missing or too small";
        case SQ_ERR_HIP: return "SQ_ERR_HIP: a HIP launch failed";
    }
    return "unknown sq_status";
}

size_t sq_workspace_size(int op, int64_t M, int64_t N, int64_t K) {
    if (op == SQ_OP_QUANT_WEIGHT) {
        if (bad_shape(1, N, K)) return 0;
        return 256;
    }
    if (op == SQ_OP_OUTLIER) {
        if (bad_shape(M, N, K)) return 0;
        return outlier_layout(M, N, K).total;
    }
    if (op == SQ_OP_CALIB_STATIC) {
        if (bad_shape(M, 1, K)) return 0;
        return kStaticWorkspaceBytes;
    }
    if (op == SQ_OP_LINEAR) {
        if (bad_shape(M, N, K)) return 0;
        return align256((size_t)M * (size_t)K) + align256((size_t)M * 4);
    }
    return 0;
}

sq_status sq_smooth_scales(const void* X_cal, int xdt, int64_t M_cal, const void* W, int wdt, int64_t N,
                           int64_t K, float alpha, float* act_max, float* s, hipStream_t stream) {
    if (!act_max) return SQ_ERR_NULL;
    if (M_cal > 0 && !X_cal) return SQ_ERR_NULL;
    if (W && !s) return SQ_ERR_NULL;
    if (M_cal < 0 || bad_shape(M_cal > 0 ? M_cal : 1, W ? N : 1, K)) return SQ_ERR_SHAPE;
    if ((M_cal > 0 && bad_dtype(xdt)) || (W && bad_dtype(wdt))) return SQ_ERR_DTYPE;
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_VALUE;
    if (misaligned(act_max) || (X_cal && misaligned(X_cal)) || (W && misaligned(W)) || (s && misaligned(s)))
        return SQ_ERR_ALIGN;
    if (M_cal > 0) SQ_TRY(launch_colmax(X_cal, xdt, M_cal, K, reinterpret_cast<uint32_t*>(act_max), stream));
    if (W) {
        SQ_TRY(launch_fill_u32(reinterpret_cast<uint32_t*>(s), K, 0u, stream));
        SQ_TRY(launch_colmax(W, wdt, N, K, reinterpret_cast<uint32_t*>(s), stream));
        SQ_TRY(launch_smooth_pow(act_max, s, K, alpha, stream));
    }
    return SQ_OK;
}

sq_status sq_quantize_per_token(const void* X, int xdt, int64_t M, int64_t K, const float* s, int8_t* Xq,
                                float* x_scale, hipStream_t stream) {
    if (!X || !Xq || !x_scale) return SQ_ERR_NULL;
    if (bad_shape(M, 1, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(xdt)) return SQ_ERR_DTYPE;
    if (misaligned(X) || misaligned(Xq) || misaligned(x_scale) || (s && misaligned(s))) return SQ_ERR_ALIGN;
    return hip_status(launch_quant_rows(X, xdt, M, K, s, s ? 1 : 0, Xq, x_scale, nullptr, nullptr, stream));
}

sq_status sq_quantize_weight(const void* W, int wdt, int64_t N, int64_t K, const float* s, int g,
                             int8_t* Wq, float* w_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!W || !Wq || !w_scale) return SQ_ERR_NULL;
    if (bad_shape(1, N, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(wdt) || (g != SQ_PER_CHANNEL && g != SQ_PER_TENSOR)) return SQ_ERR_DTYPE;
    if (misaligned(W) || misaligned(Wq) || misaligned(w_scale) || (s && misaligned(s))) return SQ_ERR_ALIGN;
    if (g == SQ_PER_CHANNEL)
        return hip_status(launch_quant_rows(W, wdt, N, K, s, s ? 2 : 0, Wq, w_scale, nullptr, nullptr, stream));
    if (!ws || ws_bytes < sq_workspace_size(SQ_OP_QUANT_WEIGHT, 0, N, K)) return SQ_ERR_WORKSPACE;
    if (misaligned(ws)) return SQ_ERR_ALIGN;
    uint32_t* gmax = reinterpret_cast<uint32_t*>(ws);
    SQ_TRY(launch_fill_u32(gmax, 1, 0u, stream));
    return hip_status(launch_quant_tensor(W, wdt, N, K, s, Wq, w_scale, gmax, stream));
}

sq_status w8a8_gemm_dequant(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                            int g, const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int ydt,
                            int32_t* acc_out, hipStream_t stream) {
    if (!Xq || !x_scale || !Wq || !w_scale || !Y) return SQ_ERR_NULL;
    if (bad_shape(M, N, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(ydt) || (g != SQ_PER_CHANNEL && g != SQ_PER_TENSOR)) return SQ_ERR_DTYPE;
    if (misaligned(Xq) || misaligned(x_scale) || misaligned(Wq) || misaligned(w_scale) || misaligned(Y) ||
        (bias && misaligned(bias)) || (acc_out && misaligned(acc_out)))
        return SQ_ERR_ALIGN;
    const int stride = g == SQ_PER_CHANNEL ? 1 : 0;
    if (M <= 16)
        return hip_status(launch_gemv(Xq, x_scale, Wq, w_scale, stride, bias, M, N, K, Y, ydt, acc_out, nullptr, stream));
    return hip_status(launch_gemm(Xq, x_scale, Wq, w_scale, stride, bias, M, N, K, Y, ydt, acc_out, nullptr, stream));
}

sq_status int8_outlier_matmul(const void* X, const void* W16, const int8_t* Wq, const float* w_scale, const float* bias,
                              int64_t M, int64_t N, int64_t K, float threshold, void* Y, void* ws, size_t ws_bytes,
                              int32_t* n_outliers, int32_t* outlier_idx, int32_t* acc_out, hipStream_t stream) {
    if (!X || !W16 || !Wq || !w_scale || !Y) return SQ_ERR_NULL;
    if (bad_shape(M, N, K)) return SQ_ERR_SHAPE;
    if (!(threshold >= 0.0f)) return SQ_ERR_VALUE;
    if (!ws || ws_bytes < sq_workspace_size(SQ_OP_OUTLIER, M, N, K)) return SQ_ERR_WORKSPACE;
    if (misaligned(X) || misaligned(W16) || misaligned(Wq) || misaligned(w_scale) || misaligned(Y) ||
        misaligned(ws) || (bias && misaligned(bias)) || (acc_out && misaligned(acc_out)) ||
        (outlier_idx && misaligned(outlier_idx)) || (n_outliers && ((uintptr_t)n_outliers & 3u)))
        return SQ_ERR_ALIGN;
    const OutlierLayout L = outlier_layout(M, N, K);
    char* base = static_cast<char*>(ws);
    uint32_t* cmax = reinterpret_cast<uint32_t*>(base + L.cmax);
    int32_t* pos = reinterpret_cast<int32_t*>(base + L.pos);
    int32_t* idx = reinterpret_cast<int32_t*>(base + L.idx);
    int32_t* count = reinterpret_cast<int32_t*>(base + L.count);
    float* xs = reinterpret_cast<float*>(base + L.xs);
    int8_t* xq = reinterpret_cast<int8_t*>(base + L.xq);
    _Float16* xo = reinterpret_cast<_Float16*>(base + L.xo);

    SQ_TRY(launch_colmax_fresh(static_cast<const _Float16*>(X), M, K, cmax, stream));
    if (quant_stream_applies(M, K, false, true)) {
        // the compaction and the activation gather inside the streaming quantizer
        const OutlierSplit os{cmax, threshold, idx, count, n_outliers, outlier_idx, xo};
        SQ_TRY(launch_quant_stream(static_cast<const _Float16*>(X), M, K, nullptr, xq, xs, &os, stream));
    } else {
        SQ_TRY(launch_outlier_compact(cmax, K, threshold, idx, pos, count, n_outliers, outlier_idx, stream));
        SQ_TRY(launch_quant_rows(X, SQ_F16, M, K, nullptr, 0, xq, xs, pos, xo, stream));
    }
    SideArgs side{xo, static_cast<const _Float16*>(W16), idx, count, K};
    return hip_status(launch_gemm(xq, xs, Wq, w_scale, 1, bias, M, N, K, Y, SQ_F16, acc_out, &side, stream));
}

sq_status sq_w8a8_linear(const void* X, int xdt, int64_t M, int64_t K, const float* s, const int8_t* Wq,
                         const float* w_scale, int g, const float* bias, int64_t N, void* Y, int ydt,
                         float* x_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!X || !Wq || !w_scale || !Y) return SQ_ERR_NULL;
    if (bad_shape(M, N, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(xdt) || bad_dtype(ydt) || (g != SQ_PER_CHANNEL && g != SQ_PER_TENSOR)) return SQ_ERR_DTYPE;
    if (!ws || ws_bytes < sq_workspace_size(SQ_OP_LINEAR, M, N, K)) return SQ_ERR_WORKSPACE;
    if (misaligned(X) || misaligned(Wq) || misaligned(w_scale) || misaligned(Y) || misaligned(ws) ||
        (s && misaligned(s)) || (bias && misaligned(bias)) || (x_scale && misaligned(x_scale)))
        return SQ_ERR_ALIGN;
    if (fused_decode(xdt, M, K))
        return hip_status(launch_linear_decode(static_cast<const _Float16*>(X), s, Wq, w_scale,
                                               g == SQ_PER_CHANNEL ? 1 : 0, bias, M, N, K, Y, ydt, x_scale, stream));
    int8_t* xq = static_cast<int8_t*>(ws);
    float* xs = x_scale ? x_scale : reinterpret_cast<float*>(static_cast<char*>(ws) + align256((size_t)M * K));
    return linear_body(X, xdt, M, K, s, Wq, w_scale, g, bias, N, Y, ydt, x_scale, xq, xs, stream);
}

sq_status sq_w8a8_linear_noalloc(const void* X, int xdt, int64_t M, int64_t K, const float* s, const int8_t* Wq,
                                 const float* w_scale, int g, const float* bias, int64_t N, void* Y, int ydt,
                                 float* x_scale, hipStream_t stream) {
    if (!X || !Wq || !w_scale || !Y) return SQ_ERR_NULL;
    if (bad_shape(M, N, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(xdt) || bad_dtype(ydt) || (g != SQ_PER_CHANNEL && g != SQ_PER_TENSOR)) return SQ_ERR_DTYPE;
    if ((uint64_t)M * (uint64_t)K > (uint64_t)SQ_NOALLOC_XQ_BYTES || (!x_scale && M > SQ_NOALLOC_MAX_M))
        return SQ_ERR_WORKSPACE;
    if (misaligned(X) || misaligned(Wq) || misaligned(w_scale) || misaligned(Y) || (s && misaligned(s)) ||
        (bias && misaligned(bias)) || (x_scale && misaligned(x_scale)))
        return SQ_ERR_ALIGN;
    if (fused_decode(xdt, M, K))
        return hip_status(launch_linear_decode(static_cast<const _Float16*>(X), s, Wq, w_scale,
                                               g == SQ_PER_CHANNEL ? 1 : 0, bias, M, N, K, Y, ydt, x_scale, stream));
    int8_t* base = scratch_base();
    if (!base) return SQ_ERR_HIP;
    float* xs = x_scale ? x_scale : reinterpret_cast<float*>(base + SQ_NOALLOC_XQ_BYTES);
    return linear_body(X, xdt, M, K, s, Wq, w_scale, g, bias, N, Y, ydt, x_scale, base, xs, stream);
}

sq_status sq_quantize_per_token_fp8(const void* X, int xdt, int64_t M, int64_t K, const float* s, uint8_t* Xq,
                                    float* x_scale, hipStream_t stream) {
    if (!X || !Xq || !x_scale) return SQ_ERR_NULL;
    if (bad_shape(M, 1, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(xdt)) return SQ_ERR_DTYPE;
    if (misaligned(X) || misaligned(Xq) || misaligned(x_scale) || (s && misaligned(s))) return SQ_ERR_ALIGN;
    return hip_status(launch_quant_rows(X, xdt, M, K, s, s ? 1 : 0, reinterpret_cast<int8_t*>(Xq), x_scale, nullptr,
                                        nullptr, stream, 1));
}

sq_status sq_quantize_per_token_asym(const void* X, int xdt, int64_t M, int64_t K, const float* s, int8_t* Xq,
                                     float* x_scale, int32_t* x_zero, hipStream_t stream) {
    if (!X || !Xq || !x_scale || !x_zero) return SQ_ERR_NULL;
    if (bad_shape(M, 1, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(xdt)) return SQ_ERR_DTYPE;
    if (misaligned(X) || misaligned(Xq) || misaligned(x_scale) || misaligned(x_zero) || (s && misaligned(s)))
        return SQ_ERR_ALIGN;
    return hip_status(launch_quant_rows(X, xdt, M, K, s, s ? 1 : 0, Xq, x_scale, nullptr, nullptr, stream, 2, x_zero));
}

sq_status sq_weight_rowsum(const int8_t* Wq, int64_t N, int64_t K, int32_t* rowsum, hipStream_t stream) {
    if (!Wq || !rowsum) return SQ_ERR_NULL;
    if (bad_shape(1, N, K)) return SQ_ERR_SHAPE;
    if (misaligned(Wq) || misaligned(rowsum)) return SQ_ERR_ALIGN;
    return hip_status(launch_weight_rowsum(Wq, N, K, rowsum, stream));
}

sq_status w8a8_asym_gemm_dequant(const int8_t* Xq, const float* x_scale, const int32_t* x_zero, const int8_t* Wq,
                                 const float* w_scale, int g, const int32_t* w_rowsum, const float* bias, int64_t M,
                                 int64_t N, int64_t K, void* Y, int ydt, int32_t* acc_out, hipStream_t stream) {
    if (!Xq || !x_scale || !x_zero || !Wq || !w_scale || !w_rowsum || !Y) return SQ_ERR_NULL;
    if (bad_shape(M, N, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(ydt) || (g != SQ_PER_CHANNEL && g != SQ_PER_TENSOR)) return SQ_ERR_DTYPE;
    if (misaligned(Xq) || misaligned(x_scale) || misaligned(x_zero) || misaligned(Wq) || misaligned(w_scale) ||
        misaligned(w_rowsum) || misaligned(Y) || (bias && misaligned(bias)) || (acc_out && misaligned(acc_out)))
        return SQ_ERR_ALIGN;
    const int stride = g == SQ_PER_CHANNEL ? 1 : 0;
    if (M <= 16)
        return hip_status(launch_gemv_asym(Xq, x_scale, x_zero, Wq, w_scale, stride, w_rowsum, bias, M, N, K, Y, ydt,
                                           acc_out, stream));
    return hip_status(launch_gemm_asym(Xq, x_scale, x_zero, Wq, w_scale, stride, w_rowsum, bias, M, N, K, Y, ydt,
                                       acc_out, stream));
}

sq_status sq_quantize_weight_fp8(const void* W, int wdt, int64_t N, int64_t K, const float* s, int g,
                                 uint8_t* Wq, float* w_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (!W || !Wq || !w_scale) return SQ_ERR_NULL;
    if (bad_shape(1, N, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(wdt) || (g != SQ_PER_CHANNEL && g != SQ_PER_TENSOR)) return SQ_ERR_DTYPE;
    if (misaligned(W) || misaligned(Wq) || misaligned(w_scale) || (s && misaligned(s))) return SQ_ERR_ALIGN;
    int8_t* q = reinterpret_cast<int8_t*>(Wq);
    if (g == SQ_PER_CHANNEL)
        return hip_status(launch_quant_rows(W, wdt, N, K, s, s ? 2 : 0, q, w_scale, nullptr, nullptr, stream, 1));
    if (!ws || ws_bytes < sq_workspace_size(SQ_OP_QUANT_WEIGHT, 0, N, K)) return SQ_ERR_WORKSPACE;
    if (misaligned(ws)) return SQ_ERR_ALIGN;
    uint32_t* gmax = reinterpret_cast<uint32_t*>(ws);
    SQ_TRY(launch_fill_u32(gmax, 1, 0u, stream));
    return hip_status(launch_quant_tensor(W, wdt, N, K, s, q, w_scale, gmax, stream, 1));
}

sq_status fp8_gemm_dequant(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                           int g, const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int ydt,
                           float* acc_out, hipStream_t stream) {
    if (!Xq || !x_scale || !Wq || !w_scale || !Y) return SQ_ERR_NULL;
    if (bad_shape(M, N, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(ydt) || (g != SQ_PER_CHANNEL && g != SQ_PER_TENSOR)) return SQ_ERR_DTYPE;
    if (misaligned(Xq) || misaligned(x_scale) || misaligned(Wq) || misaligned(w_scale) || misaligned(Y) ||
        (bias && misaligned(bias)) || (acc_out && misaligned(acc_out)))
        return SQ_ERR_ALIGN;
    const int stride = g == SQ_PER_CHANNEL ? 1 : 0;
    if (M <= 16)
        return hip_status(launch_gemv_fp8(Xq, x_scale, Wq, w_scale, stride, bias, M, N, K, Y, ydt, acc_out, stream));
    return hip_status(launch_gemm_fp8(Xq, x_scale, Wq, w_scale, stride, bias, M, N, K, Y, ydt, acc_out, stream));
}

sq_status sq_fold_smoothing_layernorm(const float* gamma, const float* beta, const float* s, int64_t K,
                                      float* gamma_out, float* beta_out, hipStream_t stream) {
    if (!gamma || !s || !gamma_out || (!beta) != (!beta_out)) return SQ_ERR_NULL;
    if (bad_shape(1, 1, K)) return SQ_ERR_SHAPE;
    if (misaligned(gamma) || misaligned(s) || misaligned(gamma_out) || (beta && (misaligned(beta) || misaligned(beta_out))))
        return SQ_ERR_ALIGN;
    return hip_status(launch_fold_layernorm(gamma, beta, s, K, gamma_out, beta_out, stream));
}

sq_status sq_layernorm_quantize_per_token(const void* X, int xdt, int64_t M, int64_t K, const float* gamma,
                                          const float* beta, float eps, int8_t* Xq, float* x_scale,
                                          hipStream_t stream) {
    if (!X || !gamma || !Xq || !x_scale) return SQ_ERR_NULL;
    if (bad_shape(M, 1, K)) return SQ_ERR_SHAPE;
    if (xdt != SQ_F16) return SQ_ERR_DTYPE;
    if (!(eps > 0.0f && eps <= 3.4028235e38f)) return SQ_ERR_VALUE;
    if (misaligned(X) || misaligned(gamma) || (beta && misaligned(beta)) || misaligned(Xq) || misaligned(x_scale))
        return SQ_ERR_ALIGN;
    return hip_status(launch_ln_quant(static_cast<const _Float16*>(X), M, K, gamma, beta, eps, Xq, x_scale, stream));
}

sq_status sq_calibrate_static_scale(const void* X_cal, int xdt, int64_t M_cal, int64_t K, const float* s,
                                    double percentile, float* x_scale, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
    if (!X_cal || !x_scale) return SQ_ERR_NULL;
    if (bad_shape(M_cal, 1, K) || (uint64_t)M_cal * (uint64_t)K >= (1ull << 32)) return SQ_ERR_SHAPE;
    if (bad_dtype(xdt)) return SQ_ERR_DTYPE;
    if (!(percentile > 0.0 && percentile <= 100.0)) return SQ_ERR_VALUE;
    if (!ws || ws_bytes < kStaticWorkspaceBytes) return SQ_ERR_WORKSPACE;
    if (misaligned(X_cal) || misaligned(x_scale) || misaligned(ws) || (s && misaligned(s))) return SQ_ERR_ALIGN;
    const int64_t n = M_cal * K;
    int64_t r = (int64_t)ceil(percentile * (double)n / 100.0);   // nearest rank, 1-based
    if (r < 1) r = 1;
    if (r > n) r = n;
    return hip_status(launch_static_calibrate(X_cal, xdt, M_cal, K, s, (uint32_t)r, x_scale, ws, stream));
}

sq_status sq_quantize_static(const void* X, int xdt, int64_t M, int64_t K, const float* s, const float* x_scale,
                             int8_t* Xq, float* x_scale_rows, hipStream_t stream) {
    if (!X || !x_scale || !Xq) return SQ_ERR_NULL;
    if (bad_shape(M, 1, K)) return SQ_ERR_SHAPE;
    if (bad_dtype(xdt)) return SQ_ERR_DTYPE;
    if (misaligned(X) || misaligned(x_scale) || misaligned(Xq) || (s && misaligned(s)) ||
        (x_scale_rows && misaligned(x_scale_rows)))
        return SQ_ERR_ALIGN;
    return hip_status(launch_static_quant(X, xdt, M, K, s, x_scale, K, Xq, x_scale_rows, stream));
}

sq_status sq_kv_calibrate_per_head(const void* KV, int dt, int64_t T, int64_t H, int64_t D, float margin,
                                   float* scale, hipStream_t stream) {
    if (!KV || !scale) return SQ_ERR_NULL;
    if (H < 1 || D < 16 || (D % 16) != 0 || H > kMaxK / D || bad_shape(T, 1, H * D)) return SQ_ERR_SHAPE;
    if (bad_dtype(dt)) return SQ_ERR_DTYPE;
    if (!(margin > 0.0f && margin <= 3.4028235e38f)) return SQ_ERR_VALUE;
    if (misaligned(KV) || misaligned(scale)) return SQ_ERR_ALIGN;
    return hip_status(launch_kv_calibrate(KV, dt, T, H, D, margin, scale, stream));
}

sq_status sq_kv_quantize_per_head(const void* KV, int dt, int64_t T, int64_t H, int64_t D, const float* scale,
                                  int8_t* q, hipStream_t stream) {
    if (!KV || !scale || !q) return SQ_ERR_NULL;
    if (H < 1 || D < 16 || (D % 16) != 0 || H > kMaxK / D || bad_shape(T, 1, H * D)) return SQ_ERR_SHAPE;
    if (bad_dtype(dt)) return SQ_ERR_DTYPE;
    if (misaligned(KV) || misaligned(scale) || misaligned(q)) return SQ_ERR_ALIGN;
    return hip_status(launch_static_quant(KV, dt, T, H * D, nullptr, scale, D, q, nullptr, stream));
}

sq_status sq_dequantize(const int8_t* q, int64_t M, int64_t K, const float* scale, int64_t scale_row_stride,
                        int64_t group, void* Y, int ydt, hipStream_t stream) {
    if (!q || !scale || !Y) return SQ_ERR_NULL;
    if (bad_shape(M, 1, K) || group < 16 || (group % 16) != 0 || (K % group) != 0 || scale_row_stride < 0 ||
        scale_row_stride > kMaxK)
        return SQ_ERR_SHAPE;
    if (bad_dtype(ydt)) return SQ_ERR_DTYPE;
    if (misaligned(q) || misaligned(Y) || ((uintptr_t)scale & 3u)) return SQ_ERR_ALIGN;
    return hip_status(launch_dequantize(q, M, K, scale, scale_row_stride, group, Y, ydt, stream));
}

}  // extern "C"
