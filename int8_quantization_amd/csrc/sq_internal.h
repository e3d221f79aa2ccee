// Internal declarations shared by the HIP sources of libsq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sq.h"

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));

namespace sq {

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

// 1/b in fp64 to within 2^-52.9 (relative): v_rcp_f64, then two Newton steps
// r <- r + r(1 - b r) with fused multiply-adds (each step squares the error and adds
// at most 2^-53).  Much shorter than the IEEE fp64 division sequence, and accurate
// enough for div_rcp64 below.
__device__ __forceinline__ double rcp64(double b) {
    double r = __builtin_amdgcn_rcp(b);
    r = __builtin_fma(r, __builtin_fma(-b, r, 1.0), r);
    return __builtin_fma(r, __builtin_fma(-b, r, 1.0), r);
}

// Correctly rounded fp32 quotient a/b from rb = rcp64(b), i.e. within 2^-52.9 of 1/b.
// t = RN64(a * rb) is then within 2^-51.9 (relative) of a/b, while a quotient of two
// binary32 numbers in the normal range lies at least 2^-49 (relative) away from every
// binary32 rounding midpoint and is never one itself; so rounding t to binary32 gives
// the same result as the IEEE division.  Quotients below the normal range take the
// IEEE division itself.
__device__ __forceinline__ float div_rcp64(float a, double rb, float b) {
    float q = (float)((double)a * rb);
    if (__builtin_fabsf(q) < 1.17549435e-38f && a != 0.0f) q = a / b;
    return q;
}

// Integer code: round half to even (v_rndne_f32), clamp to [-128, 127].
__device__ __forceinline__ int code_of(float v) {
    const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(v), -128.0f, 127.0f);
    return (int)r;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------------------
// Host-side launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------

// Device properties cached once per device.
struct DevInfo {
    int cus;
    int xcds;
};
const DevInfo& dev_info();

// Fill n 32-bit words with a value (kernel, so it is safe inside stream capture).
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st);

// Grid of an elementwise pass over M rows of nchunk 16-byte chunks with 256-thread
// blocks: a block covers P = min(256, pow2 >= nchunk) chunks (grid x) of each of
// 256 / P consecutive rows, so short rows still fill every lane; grid y walks the
// row groups, about rows_per_thread rows per thread, but with at least min_blocks
// blocks when there are rows for them.  Thread t of block (x, y) takes chunk
// x * P + (t % P) of rows (y * 256/P + t / P) + k * gridDim.y * 256/P.
struct RowPack {
    int lgp;      // log2 P
    dim3 grid;
};
inline RowPack row_pack(int64_t M, int64_t nchunk, int64_t rows_per_thread, int64_t min_blocks) {
    int lgp = 0;
    while (lgp < 8 && ((int64_t)1 << lgp) < nchunk) ++lgp;
    const int64_t P = (int64_t)1 << lgp, R = 256 / P;
    const int64_t gx = (nchunk + P - 1) / P;
    const int64_t groups = (M + R - 1) / R;
    int64_t gy = (groups + rows_per_thread - 1) / rows_per_thread;
    const int64_t want = (min_blocks + gx - 1) / gx;
    if (gy < want) gy = want < groups ? want : groups;
    if (gy > 65535) gy = 65535;
    return RowPack{lgp, dim3((unsigned)gx, (unsigned)gy)};
}

// Per-row smoothing + absmax quantization (activations per token, weights per channel).
// mode 0: no smoothing; 1: x / s_j; 2: x * s_j.  pos/Xo (LLM.int8() only): pos[j] >= 0
// marks an outlier column, whose value is copied to Xo[m*K + pos[j]] and whose code is 0.
// fmt 0: int8 codes, scale max/127; fmt 1: FP8 E4M3 code bytes, scale max/448 (no pos).
hipError_t launch_quant_rows(const void* X, sq_dtype dt, int64_t M, int64_t K, const float* s,
                             int mode, int8_t* Xq, float* scale, const int32_t* pos, _Float16* Xo,
                             hipStream_t st, int fmt = 0);

// Running column absolute maximum: amax_bits[j] = max(amax_bits[j], bits(max_m |X[m,j]|)),
// where amax_bits holds non-negative floats as their bit patterns (monotone as uint32).
hipError_t launch_colmax(const void* X, sq_dtype dt, int64_t M, int64_t K, uint32_t* amax_bits,
                         hipStream_t st);

// s_j from act_max and the W column maxima held in s (overwritten in place).
hipError_t launch_smooth_pow(const float* act_max, float* s_wmax, int64_t K, float alpha,
                             hipStream_t st);

// Per-tensor weight quantization: global max then codes.
hipError_t launch_quant_tensor(const void* W, sq_dtype dt, int64_t N, int64_t K, const float* s,
                               int8_t* Wq, float* w_scale, uint32_t* gmax_bits, hipStream_t st, int fmt = 0);

// int8 GEMM + dequant epilogue (M > 16).  side != nullptr adds the LLM.int8() fp16 side
// product over the first *count columns of Xo [M x ldo] and Wo [N x ldo].
struct SideArgs {
    const _Float16* Xo;
    const _Float16* Wo;
    const int32_t* count;
    int64_t ldo;
};
hipError_t launch_gemm(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws,
                       int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                       sq_dtype ydt, int32_t* acc_out, const SideArgs* side, hipStream_t st);
// FP8 E4M3 GEMM (fp32 accumulation) + the same dequant epilogue; acc_out receives the
// fp32 accumulators' bits.
hipError_t launch_gemm_fp8(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                           int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                           sq_dtype ydt, float* acc_out, hipStream_t st);

// Weight-streaming decode kernel, M <= 16.
hipError_t launch_gemv(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws,
                       int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                       sq_dtype ydt, int32_t* acc_out, const SideArgs* side, hipStream_t st);
// Fused decode layer (M <= 2, K <= 8192, fp16 X): per-token quantization of X (with
// x / s_j when s is given) in every block's prologue, then the decode kernel; x_scale
// (may be null) receives the per-token scales.
hipError_t launch_linear_decode(const _Float16* X, const float* s, const int8_t* Wq, const float* ws,
                                int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                                sq_dtype ydt, float* x_scale, hipStream_t st);
// Its FP8 E4M3 variant (fp32 partial sums; acc_out receives their bits).
hipError_t launch_gemv_fp8(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                           int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                           sq_dtype ydt, float* acc_out, hipStream_t st);

// LLM.int8(): outlier columns from the column maxima (bit patterns), ascending list,
// per-column slot (or -1), device-side count; optional copies to user buffers.
hipError_t launch_outlier_compact(const uint32_t* cmax_bits, int64_t K, float threshold,
                                  int32_t* idx, int32_t* pos, int32_t* count, int32_t* user_count,
                                  int32_t* user_idx, hipStream_t st);

// Wo[n, t] = W16[n, idx[t]] for t < *count.
hipError_t launch_gather_cols(const _Float16* W16, int64_t N, int64_t K, const int32_t* idx,
                              const int32_t* count, _Float16* Wo, hipStream_t st);

// LayerNorm (weights with the smoothing folded in) + per-token quantization, fp16 rows.
hipError_t launch_ln_quant(const _Float16* X, int64_t M, int64_t K, const float* gamma, const float* beta,
                           float eps, int8_t* Xq, float* scale, hipStream_t st);

// Static per-tensor activation scale: exact nearest-rank percentile of |x'| (radix
// select in the workspace: a 2048-bin histogram, then the selection state).
constexpr size_t kStaticHistBytes = 2048 * 4;
constexpr size_t kStaticWorkspaceBytes = 8448;
hipError_t launch_static_calibrate(const void* X, sq_dtype dt, int64_t M, int64_t K, const float* s, uint32_t rank,
                                   float* x_scale, void* ws, hipStream_t st);
// Quantization with calibrated scales: column j uses xs[j / group]; xs_rows (may be null)
// receives xs[0] per row.
hipError_t launch_static_quant(const void* X, sq_dtype dt, int64_t M, int64_t K, const float* s, const float* xs,
                               int64_t group, int8_t* Xq, float* xs_rows, hipStream_t st);

// KV cache [T x H x D]: per-head calibration scale_h = fl32(fl32(margin * max|x|) / 127).
hipError_t launch_kv_calibrate(const void* KV, sq_dtype dt, int64_t T, int64_t H, int64_t D, float margin,
                               float* scale, hipStream_t st);
// y[m, j] = fl32(q[m, j] * scale[m * row_stride + j / group]), stored as ydt.
hipError_t launch_dequantize(const int8_t* q, int64_t M, int64_t K, const float* scale, int64_t row_stride,
                             int64_t group, void* Y, sq_dtype ydt, hipStream_t st);

// gamma_out = gamma / s, beta_out = beta / s (beta may be null).
hipError_t launch_fold_layernorm(const float* gamma, const float* beta, const float* s, int64_t K,
                                 float* gamma_out, float* beta_out, hipStream_t st);

}  // namespace sq
