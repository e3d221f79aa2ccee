// Internal declarations shared by the HIP sources of libsq (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

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

// FP8 E4M3 (OCP e4m3fn) codes of four values, one per byte, nearest-even
// (v_cvt_pk_fp8_f32).  Callers clamp to [-448, 448] first, so no value overflows.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}
__device__ __forceinline__ float fp8_clamp(float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); }

// Maximum over the wave of non-negative floats, returned to every lane (all 64 lanes active).
// Four DPP steps give each row of 16 lanes its maximum (quad swaps 1 and 2, then the
// half-row and row mirrors), and the four row maxima are read out (v_readlane) and
// combined: a few cycles per step, against an LDS round trip per step for the
// ds_bpermute butterfly of __shfl_xor.  The maximum is exact in any order.
__device__ __forceinline__ float wave_max(float v) {
    auto step = [](float x, int ctrl) -> float {
        int y;
        switch (ctrl) {
            case 0: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
            case 1: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
            case 2: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false); break;  // row_half_mirror
            default: y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false); break; // row_mirror
        }
        return __builtin_fmaxf(x, __int_as_float(y));
    };
    v = step(v, 0);
    v = step(v, 1);
    v = step(v, 2);
    v = step(v, 3);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return __builtin_fmaxf(__builtin_fmaxf(r0, r1), __builtin_fmaxf(r2, r3));
}

// 16 bytes per lane from a buffer resource straight into LDS: the wave's 1 KB
// lands at LDS byte address lds_addr (through M0), lane l at lds_addr + 16 l.
// Offsets outside the resource's record range read as zeros.  The resource is
// the four descriptor words in scalar registers.  M0 is written here only: the
// kernels that use this helper leave M0 to it (a CPU test checks their ISA).
// Issued from inline asm: the compiler models the builtin form as an LDS store of
// unknown address and then waits for it before every later LDS read, which would
// serialize a prefetch with the reads of the previous stage; callers order it
// with their own s_waitcnt and barriers.
__device__ __forceinline__ void dma_to_lds(const v4i& rsrc, uint32_t lds_addr, uint32_t voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 ::"s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}

// Buffer resource over [p, p + nrec) bytes, raw (unformatted) 32-bit records.
__device__ __forceinline__ v4i buffer_desc(const void* p, uint32_t nrec) {
    const uint64_t a = (uint64_t)p;
    return v4i{__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)(a >> 32)),
               __builtin_amdgcn_readfirstlane((int)nrec), 0x00020000};
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------------------
// Host-side launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------

// Kernel launch that reports this launch's own status, hipLaunchKernel's return value
// (hipGetLastError() would also return, and clear, an error left by an earlier,
// unrelated HIP call on the thread).  The arguments are first converted to the
// kernel's parameter types, because hipLaunchKernel reads each one through a pointer
// to that type.
template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t st, A&&... args) {
    static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
    std::tuple<P...> vals(static_cast<P>(std::forward<A>(args))...);
    void* ptrs[sizeof...(P) == 0 ? 1 : sizeof...(P)];
    std::apply([&ptrs](auto&... v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void*>(&v)), ...);
    }, vals);
    return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, st);
}
// Launch, and return from the enclosing launcher on a failed launch.
#define SQ_LAUNCH(...)                                      \
    do {                                                    \
        const hipError_t sq_e_ = ::sq::launch(__VA_ARGS__); \
        if (sq_e_ != hipSuccess) return sq_e_;              \
    } while (0)

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
// fmt 0: int8 codes, scale max/127; fmt 1: FP8 E4M3 code bytes, scale max/448 (no pos);
// fmt 2: zero-point int8 codes over the row range extended to 0, scale (hi - lo)/255, the
// zero point (minus 128) to zero[m] (mode 0 or 1, no pos).
hipError_t launch_quant_rows(const void* X, int dt, int64_t M, int64_t K, const float* s,
                             int mode, int8_t* Xq, float* scale, const int32_t* pos, _Float16* Xo,
                             hipStream_t st, int fmt = 0, int32_t* zero = nullptr);

// The LLM.int8() split done inside the streaming quantizer: from the column maxima (float
// bits) and the threshold, the ascending outlier list and count (written to idx / count and
// the optional user copies) and the outlier activations Xo [M x K] (row stride K, the first
// count columns used).
struct OutlierSplit {
    const uint32_t* cmax;
    float threshold;
    int32_t* idx;
    int32_t* count;
    int32_t* user_count;
    int32_t* user_idx;
    _Float16* Xo;
};

// The streaming fp16 per-token quantizer (int8 codes; s == nullptr: no smoothing; os: the
// LLM.int8() variant, without smoothing), for the shapes where quant_stream_applies()
// holds; launch_quant_rows dispatches to it for plain and smoothed rows.
bool quant_stream_applies(int64_t M, int64_t K, bool smooth, bool outliers);
hipError_t launch_quant_stream(const _Float16* X, int64_t M, int64_t K, const float* s, int8_t* Xq, float* scale,
                               const OutlierSplit* os, hipStream_t st);
// FP8 E4M3 codes of fp16 rows (scale max/448), one wave per row: for at least four rows
// per CU (quant_stream_applies) and rows of up to 4096 values.
hipError_t launch_quant_wave_fp8(const _Float16* X, int64_t M, int64_t K, const float* s, int8_t* q, float* scale,
                                 hipStream_t st);

// Running column absolute maximum: amax_bits[j] = max(amax_bits[j], bits(max_m |X[m,j]|)),
// where amax_bits holds non-negative floats as their bit patterns (monotone as uint32).
hipError_t launch_colmax(const void* X, int dt, int64_t M, int64_t K, uint32_t* amax_bits,
                         hipStream_t st);

// Column absolute maxima of an fp16 matrix, written as float bits (any previous
// contents of out_bits are overwritten; nothing needs zeroing first).
hipError_t launch_colmax_fresh(const _Float16* X, int64_t M, int64_t K, uint32_t* out_bits, hipStream_t st);

// s_j from act_max and the W column maxima held in s (overwritten in place).
hipError_t launch_smooth_pow(const float* act_max, float* s_wmax, int64_t K, float alpha,
                             hipStream_t st);

// Per-tensor weight quantization: global max then codes.
hipError_t launch_quant_tensor(const void* W, int dt, int64_t N, int64_t K, const float* s,
                               int8_t* Wq, float* w_scale, uint32_t* gmax_bits, hipStream_t st, int fmt = 0);

// int8 GEMM + dequant epilogue (M > 16).  side != nullptr adds the LLM.int8() fp16 side
// product sum_{t < *count} Xo[m, t] * W16[n, idx[t]]: Xo [M x ldo] the gathered outlier
// activations, W16 [N x K] the fp16 weight, idx the ascending outlier columns.
struct SideArgs {
    const _Float16* Xo;
    const _Float16* W16;
    const int32_t* idx;
    const int32_t* count;
    int64_t ldo;
};
// Zero-point activations: per-row zero points (minus 128) and per-output-row sums of Wq.
struct AsymArgs {
    const int32_t* xz;
    const int32_t* wrs;
};

hipError_t launch_gemm(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws,
                       int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                       int ydt, int32_t* acc_out, const SideArgs* side, hipStream_t st);
// FP8 E4M3 GEMM (fp32 accumulation) + the same dequant epilogue; acc_out receives the
// fp32 accumulators' bits.
hipError_t launch_gemm_fp8(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                           int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                           int ydt, float* acc_out, hipStream_t st);

// Weight-streaming decode kernel, M <= 16.
hipError_t launch_gemv(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws,
                       int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                       int ydt, int32_t* acc_out, const SideArgs* side, hipStream_t st);
// Zero-point activations (x_zero: zero point minus 128 per row, w_rowsum: sum of each Wq
// row): the same GEMM and decode kernels with acc - x_zero[m] * w_rowsum[n] dequantized.
hipError_t launch_gemm_asym(const int8_t* Xq, const float* xs, const int32_t* xz, const int8_t* Wq, const float* ws,
                            int ws_stride, const int32_t* wrs, const float* bias, int64_t M, int64_t N, int64_t K,
                            void* Y, int ydt, int32_t* acc_out, hipStream_t st);
hipError_t launch_gemv_asym(const int8_t* Xq, const float* xs, const int32_t* xz, const int8_t* Wq, const float* ws,
                            int ws_stride, const int32_t* wrs, const float* bias, int64_t M, int64_t N, int64_t K,
                            void* Y, int ydt, int32_t* acc_out, hipStream_t st);
// Row sums of an int8 matrix [N x K] (K % 16 == 0), int32.
hipError_t launch_weight_rowsum(const int8_t* Wq, int64_t N, int64_t K, int32_t* rowsum, hipStream_t st);
// Fused decode layer (M <= 2, K <= 8192, fp16 X): per-token quantization of X (with
// x / s_j when s is given) in every block's prologue, then the decode kernel; x_scale
// (may be null) receives the per-token scales.
hipError_t launch_linear_decode(const _Float16* X, const float* s, const int8_t* Wq, const float* ws,
                                int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                                int ydt, float* x_scale, hipStream_t st);
// Its FP8 E4M3 variant (fp32 partial sums; acc_out receives their bits).
hipError_t launch_gemv_fp8(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws,
                           int ws_stride, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                           int ydt, float* acc_out, hipStream_t st);

// LLM.int8(): outlier columns from the column maxima (bit patterns), ascending list,
// per-column slot (or -1), device-side count; optional copies to user buffers.
hipError_t launch_outlier_compact(const uint32_t* cmax_bits, int64_t K, float threshold,
                                  int32_t* idx, int32_t* pos, int32_t* count, int32_t* user_count,
                                  int32_t* user_idx, hipStream_t st);


// LayerNorm (weights with the smoothing folded in) + per-token quantization, fp16 rows.
hipError_t launch_ln_quant(const _Float16* X, int64_t M, int64_t K, const float* gamma, const float* beta,
                           float eps, int8_t* Xq, float* scale, hipStream_t st);

// Static per-tensor activation scale: exact nearest-rank percentile of |x'| (radix
// select in the workspace: a 2048-bin histogram, then the selection state).
constexpr size_t kStaticHistBytes = 2048 * 4;
constexpr size_t kStaticWorkspaceBytes = 8448;
hipError_t launch_static_calibrate(const void* X, int dt, int64_t M, int64_t K, const float* s, uint32_t rank,
                                   float* x_scale, void* ws, hipStream_t st);
// Quantization with calibrated scales: column j uses xs[j / group]; xs_rows (may be null)
// receives xs[0] per row.
hipError_t launch_static_quant(const void* X, int dt, int64_t M, int64_t K, const float* s, const float* xs,
                               int64_t group, int8_t* Xq, float* xs_rows, hipStream_t st);

// KV cache [T x H x D]: per-head calibration scale_h = fl32(fl32(margin * max|x|) / 127).
hipError_t launch_kv_calibrate(const void* KV, int dt, int64_t T, int64_t H, int64_t D, float margin,
                               float* scale, hipStream_t st);
// y[m, j] = fl32(q[m, j] * scale[m * row_stride + j / group]), stored as ydt.
hipError_t launch_dequantize(const int8_t* q, int64_t M, int64_t K, const float* scale, int64_t row_stride,
                             int64_t group, void* Y, int ydt, hipStream_t st);

// gamma_out = gamma / s, beta_out = beta / s (beta may be null).
hipError_t launch_fold_layernorm(const float* gamma, const float* beta, const float* s, int64_t K,
                                 float* gamma_out, float* beta_out, hipStream_t st);

}  // namespace sq
