// INT8 KV cache with per-head scales ["SmoothQuant量化实战", section 5.2: the KV
// cache is quantized to INT8 with one scale per attention head, because the
// heads' value ranges differ; as the cache grows, a scale fixed at calibration
// time with a safety factor avoids recomputing it every step].
//
// Layout: KV [T x H x D] row-major (tokens, heads, head dim), i.e. T rows of
// H*D values in which head h owns columns [h*D, (h+1)*D).
//   calibration:  scale_h = fl32( fl32(margin * max_{t,d} |x[t,h,d]|) / 127 )
//   quantization: the static quantizer with one scale per D-column group
//   dequantization (general): y[m,j] = fl32(q[m,j] * scale[m*row_stride + j/group])
//     (row_stride 0, group D: per head; row_stride 1, group K: one scale per row,
//      e.g. the per-token-per-head scales of sq_quantize_per_token over [T*H x D]).
// All three are HBM-bound elementwise passes.
#include <type_traits>

#include "sq_internal.h"

namespace sq {

namespace {

// Maximum of |x| over the rows, folded per head: each block reduces its columns'
// heads in LDS, then takes one global atomic max per head on the float bit
// patterns (non-negative floats order like their bits; the maximum ignores NaN).
// A block's P*N columns span at most P*N/D + 1 <= 129 heads (D >= 16, N <= 8).
template <typename T>
__global__ __launch_bounds__(256) void kv_headmax_kernel(const T* __restrict__ KV, int64_t T_, int64_t HD,
                                                         int64_t D, uint32_t* __restrict__ hmax_bits, int lgp) {
    constexpr int N = 16 / sizeof(T);
    using V = T __attribute__((ext_vector_type(N)));
    __shared__ uint32_t smax[132];
    const int64_t nchunk = HD / N;
    const int64_t col0 = ((int64_t)blockIdx.x << lgp) * N;          // first column of the block
    const int64_t h0 = col0 / D;
    const int64_t c = ((int64_t)blockIdx.x << lgp) + (threadIdx.x & ((1u << lgp) - 1));
    const int64_t R = 256 >> lgp;
    if (threadIdx.x < 132) smax[threadIdx.x] = 0u;
    float m = 0.0f;
    if (c < nchunk) {
        const V* src = reinterpret_cast<const V*>(KV) + c;
        for (int64_t t = blockIdx.y * R + (threadIdx.x >> lgp); t < T_; t += gridDim.y * R) {
            const V v = __builtin_nontemporal_load(src + t * nchunk);
#pragma unroll
            for (int e = 0; e < N; ++e) m = __builtin_fmaxf(m, __builtin_fabsf((float)v[e]));
        }
    }
    __syncthreads();
    if (c < nchunk) atomicMax(&smax[(c * N) / D - h0], __builtin_bit_cast(uint32_t, m));
    __syncthreads();
    const int64_t nh = (((col0 + ((int64_t)N << lgp) - 1) < HD ? col0 + ((int64_t)N << lgp) - 1 : HD - 1)) / D - h0 + 1;
    if (threadIdx.x < nh && smax[threadIdx.x] != 0u) atomicMax(&hmax_bits[h0 + threadIdx.x], smax[threadIdx.x]);
}

__global__ void kv_scale_kernel(float* __restrict__ scale, int64_t H, float margin) {
    for (int64_t h = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; h < H; h += (int64_t)gridDim.x * blockDim.x) {
        const float m = __builtin_bit_cast(float, reinterpret_cast<const uint32_t*>(scale)[h]);
        scale[h] = (margin * m) / 127.0f;
    }
}

// y = fl32(q * scale) with the chunk's one scale.  A thread takes 16 / sizeof(OutT)
// codes of a row, so its output is one 16-byte store and each store instruction of
// a wave covers 1 KiB contiguously (two 16-byte stores per lane, interleaved across
// lanes, measured 20% slower).  The codes are read once: non-temporal loads.
template <typename OutT>
__global__ __launch_bounds__(256) void dequant_kernel(const int8_t* __restrict__ q, int64_t M, int64_t K,
                                                      const float* __restrict__ scale, int64_t row_stride,
                                                      int64_t group, OutT* __restrict__ Y, int lgp) {
    constexpr int CPL = 16 / sizeof(OutT);   // codes per lane: 8 (fp16 out) or 4 (fp32 out)
    typedef int v2i __attribute__((ext_vector_type(2)));
    using QV = typename std::conditional<CPL == 8, v2i, int>::type;
    const int64_t nchunk = K / CPL;
    const int64_t c = ((int64_t)blockIdx.x << lgp) + (threadIdx.x & ((1u << lgp) - 1));
    if (c >= nchunk) return;
    const int64_t g = (c * CPL) / group;
    const int64_t R = 256 >> lgp;
    const int64_t step = gridDim.y * R;
    for (int64_t m = blockIdx.y * R + (threadIdx.x >> lgp); m < M; m += step) {
        const float sc = scale[m * row_stride + g];
        const QV w = __builtin_nontemporal_load(reinterpret_cast<const QV*>(q + m * K) + c);
        uint32_t wb[CPL / 4];
        if constexpr (CPL == 8) {
            wb[0] = (uint32_t)w[0];
            wb[1] = (uint32_t)w[1];
        } else {
            wb[0] = (uint32_t)w;
        }
        float y[CPL];
#pragma unroll
        for (int e = 0; e < CPL; ++e) y[e] = (float)(int8_t)(wb[e >> 2] >> (8 * (e & 3))) * sc;
        if constexpr (CPL == 8) {
            typedef float f2 __attribute__((ext_vector_type(2)));
            typedef _Float16 hf2 __attribute__((ext_vector_type(2)));
            uint32_t o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{y[2 * k], y[2 * k + 1]}, hf2));
            *reinterpret_cast<v4i*>(Y + m * K + c * CPL) = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
        } else {
            *reinterpret_cast<v4f*>(Y + m * K + c * CPL) = v4f{y[0], y[1], y[2], y[3]};
        }
    }
}

}  // namespace

hipError_t launch_kv_calibrate(const void* KV, int dt, int64_t T, int64_t H, int64_t D, float margin,
                               float* scale, hipStream_t st) {
    uint32_t* bits = reinterpret_cast<uint32_t*>(scale);   // the output holds the maxima meanwhile
    hipError_t e = launch_fill_u32(bits, H, 0u, st);
    if (e != hipSuccess) return e;
    const int64_t HD = H * D;
    if (dt == SQ_F16) {
        const RowPack g = row_pack(T, HD / 8, 32, 256);
        SQ_LAUNCH(kv_headmax_kernel<_Float16>, g.grid, dim3(256), 0, st, static_cast<const _Float16*>(KV),
                           T, HD, D, bits, g.lgp);
    } else {
        const RowPack g = row_pack(T, HD / 4, 32, 256);
        SQ_LAUNCH(kv_headmax_kernel<float>, g.grid, dim3(256), 0, st, static_cast<const float*>(KV), T,
                           HD, D, bits, g.lgp);
    }
    SQ_LAUNCH(kv_scale_kernel, dim3((unsigned)((H + 255) / 256)), dim3(256), 0, st, scale, H, margin);
    return hipSuccess;
}

hipError_t launch_dequantize(const int8_t* q, int64_t M, int64_t K, const float* scale, int64_t row_stride,
                             int64_t group, void* Y, int ydt, hipStream_t st) {
    if (ydt == SQ_F16) {
        const RowPack g = row_pack(M, K / 8, 8, 2048);
        SQ_LAUNCH(dequant_kernel<_Float16>, g.grid, dim3(256), 0, st, q, M, K, scale, row_stride, group,
                           static_cast<_Float16*>(Y), g.lgp);
    } else {
        const RowPack g = row_pack(M, K / 4, 8, 2048);
        SQ_LAUNCH(dequant_kernel<float>, g.grid, dim3(256), 0, st, q, M, K, scale, row_stride, group,
                           static_cast<float*>(Y), g.lgp);
    }
    return hipSuccess;
}

}  // namespace sq
