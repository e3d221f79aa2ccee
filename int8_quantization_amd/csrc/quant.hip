// Quantization-side kernels for gfx950:
//  - fused smoothing + per-row absmax int8 quantization (activations per token,
//    weights per output channel) ["量化基础与INT8", 量化粒度 / 量化流程示例;
//    "SmoothQuant量化实战", sections 3.3-3.4];
//  - calibration column absmax and the smoothing factors [SmoothQuant page,
//    sections 2.1, 3.2, 3.3];
//  - per-tensor weight quantization [basics notes, 量化粒度].
// All of these are HBM-bound: 16-byte coalesced loads, wave-shuffle reductions,
// packed int8 stores.
#include <atomic>
#include <mutex>
#include <type_traits>

#include "sq_internal.h"

namespace sq {

// ---------------------------------------------------------------------------
// Device info
// ---------------------------------------------------------------------------
const DevInfo& dev_info() {
    static DevInfo info[64];
    static std::once_flag once[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    std::call_once(once[dev], [dev]() {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        info[dev].cus = cus;
        info[dev].xcds = 8;
    });
    return info[dev];
}

// ---------------------------------------------------------------------------
// Fill
// ---------------------------------------------------------------------------
__global__ void fill_u32_kernel(uint32_t* p, int64_t n, uint32_t v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    SQ_LAUNCH(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// 16-byte chunk types
// ---------------------------------------------------------------------------
template <typename T> struct Chunk;
template <> struct Chunk<_Float16> {
    using V = h8;
    static constexpr int N = 8;
};
template <> struct Chunk<float> {
    using V = v4f;
    static constexpr int N = 4;
};
template <typename T, int VEC> struct VecOf { typedef T V __attribute__((ext_vector_type(VEC))); };

template <int VEC> struct CodeStore;
template <> struct CodeStore<8> {
    static __device__ __forceinline__ void store(int8_t* p, const int* q) {
        uint32_t lo = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                      ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
        uint32_t hi = (uint32_t)(q[4] & 0xff) | ((uint32_t)(q[5] & 0xff) << 8) |
                      ((uint32_t)(q[6] & 0xff) << 16) | ((uint32_t)(q[7] & 0xff) << 24);
        *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
    }
};
template <> struct CodeStore<4> {
    static __device__ __forceinline__ void store(int8_t* p, const int* q) {
        *reinterpret_cast<uint32_t*>(p) = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                                          ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
    }
};

// Codes of VEC quotients x'/scale: int8 (FMT 0) or FP8 E4M3 (FMT 1); `zero` marks
// elements whose code is 0 (scale 0, LLM.int8() outlier columns).
template <int VEC, int FMT>
__device__ __forceinline__ void store_codes(int8_t* p, const float* v, const bool* zero) {
    if constexpr (FMT == 0) {
        int q[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) q[e] = zero[e] ? 0 : code_of(v[e]);
        CodeStore<VEC>::store(p, q);
    } else {
        float c[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) c[e] = zero[e] ? 0.0f : fp8_clamp(v[e]);
        if constexpr (VEC == 8)
            *reinterpret_cast<uint2*>(p) = make_uint2(fp8x4(c[0], c[1], c[2], c[3]), fp8x4(c[4], c[5], c[6], c[7]));
        else
            *reinterpret_cast<uint32_t*>(p) = fp8x4(c[0], c[1], c[2], c[3]);
    }
}

// ---------------------------------------------------------------------------
// Fused smoothing + per-row quantization, register-resident rows.
//
// A block holds G row groups of TPG threads; thread t of a group owns the
// 16-byte chunks t, t+TPG, ... (CH of them) of every row the group visits.
// The per-column constants (fp64 reciprocal of s_j, or s_j, or the outlier
// slot) are computed once per block and kept in registers while the block
// walks rows m = (blockIdx.x + i*gridDim.x)*G + g; the next row's loads are
// issued before the current row's reduction.
//   mode 0: x' = x;   mode 1: x' = fl32(x / s_j);   mode 2: x' = fl32(x * s_j)
//   xs = fl32(max |x'| / 127) over non-outlier columns
//   q  = clamp(rne(fl32(x' / xs)), -128, 127), 0 for outlier columns or xs == 0
// FMT 1 (FP8 E4M3): xs = fl32(max |x'| / 448), q = e4m3(clamp(fl32(x' / xs), -448, 448)).
// Both divisions are exact fp32 quotients computed as RN32(RN64(a * RN64(1/b)))
// (see div_rcp64).  A quotient below the fp32 normal range takes the IEEE
// division for x / s_j (only possible for fp32 inputs or s_j > 2^100); for
// x' / xs such a quotient is below 0.5 and its code is 0 either way.
// ---------------------------------------------------------------------------
// Barrier for LDS traffic only: __syncthreads() would also wait for every
// outstanding global load, i.e. drain the row prefetch.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename T, int VEC, int CH, int MODE, bool OUTL, int FMT>
__global__ __launch_bounds__(1024) void quant_rows_fast(const T* __restrict__ X, int64_t M, int64_t K,
                                                        const float* __restrict__ s, int8_t* __restrict__ Xq,
                                                        float* __restrict__ scale, const int32_t* __restrict__ pos,
                                                        _Float16* __restrict__ Xo, int32_t* __restrict__ zero, int tpg,
                                                        int G) {
    using V = typename VecOf<T, VEC>::V;
    static_assert(FMT != 2 || (!OUTL && MODE != 2), "zero-point codes are for activation rows");
    __shared__ float red[2][16];
    __shared__ float red2[FMT == 2 ? 2 : 1][16];   // FMT 2: max(-x'), the bottom of the range
    const int g = threadIdx.x / tpg;          // row group
    const int tid = threadIdx.x - g * tpg;    // thread within the group
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int w0 = (g * tpg) >> 6, nw = tpg >> 6;   // this group's waves
    const int64_t nchunk = K / VEC;


    bool valid[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) valid[i] = tid + (int64_t)i * tpg < nchunk;
    // Rows are prefetched PF iterations ahead (PF = 2 when registers allow).
    constexpr int PF = (CH <= 2) ? 2 : 1;
    V buf[PF + 1][CH];
    auto load_row = [&](int64_t row, V* r) {
        const V* src = reinterpret_cast<const V*>(X + row * K);
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int64_t c = tid + (int64_t)i * tpg;
            if (valid[i] && row < M) r[i] = src[c];
            else r[i] = V{};
        }
    };

    const int64_t step = (int64_t)gridDim.x * G;
    int64_t m = (int64_t)blockIdx.x * G + g;
#pragma unroll
    for (int p = 0; p < PF; ++p) load_row(m + p * step, buf[p]);
    // per-column constants, computed while the first rows are in flight
    double rs[MODE == 1 ? CH : 1][VEC];
    float sv[MODE == 2 ? CH : 1][VEC];
    unsigned omask[OUTL ? CH : 1];            // bit e: element e of the chunk is an outlier column
    int opos[OUTL ? CH : 1][OUTL ? VEC : 1];  // its slot among the outlier columns (kept in registers: a
                                              // load in the row loop would also wait for the row prefetch)
    bool guard = false;                       // some x/s_j may fall below the normal range
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int64_t c = tid + (int64_t)i * tpg;
        const int64_t cc = valid[i] ? c : 0;
        if constexpr (OUTL) {
            // the chunk's VEC slots in 16-byte loads: every block reads this same small array at
            // start-up, and one 4-byte load per element made that a hot spot in L2
            static_assert(VEC % 4 == 0, "slot loads are 16 bytes");
            omask[i] = 0;
#pragma unroll
            for (int q = 0; q < VEC / 4; ++q) {
                const v4i pq = valid[i] ? *reinterpret_cast<const v4i*>(pos + cc * VEC + 4 * q) : v4i{-1, -1, -1, -1};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    opos[i][4 * q + u] = pq[u];
                    if (pq[u] >= 0) omask[i] |= 1u << (4 * q + u);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if constexpr (MODE == 1) {
                const float sj = s[cc * VEC + e];
                rs[i][e] = rcp64((double)sj);
                guard = guard || !(sj < 0x1p100f);
            }
            if constexpr (MODE == 2) sv[i][e] = s[cc * VEC + e];
        }
    }
    if constexpr (sizeof(T) == 4) guard = true;   // fp32 inputs can be subnormal
    // every group runs the same number of iterations (barriers are block wide)
    const int64_t first = (int64_t)blockIdx.x * G;
    const int64_t iters = first < M ? (M - first + step - 1) / step : 0;
    for (int64_t it = 0; it < iters; ++it, m += step) {
        load_row(m + PF * step, buf[PF]);       // in flight during this whole row
        const bool live = m < M;
        V* rc = buf[0];
        float xv[CH][VEC];
        float amax = 0.0f;   // max |x'| (FMT 2: max x', the top of a range that contains 0)
        float nlo = 0.0f;    // FMT 2: max(-x')
        auto pass1 = [&](auto guarded) {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int64_t c = tid + (int64_t)i * tpg;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    float x = (float)rc[i][e];
                    if constexpr (MODE == 1) {
                        float q = (float)((double)x * rs[i][e]);
                        if constexpr (decltype(guarded)::value)
                            if (__builtin_fabsf(q) < 1.17549435e-38f && x != 0.0f) q = x / s[c * VEC + e];
                        x = q;
                    }
                    if constexpr (MODE == 2) x = x * sv[i][e];
                    xv[i][e] = x;
                    bool skip = false;
                    if constexpr (OUTL) {
                        skip = (omask[i] >> e) & 1u;
                        if (skip && live) Xo[m * K + opos[i][e]] = (_Float16)rc[i][e];
                    }
                    if constexpr (FMT == 2) {
                        amax = __builtin_fmaxf(amax, x);
                        nlo = __builtin_fmaxf(nlo, -x);
                    } else {
                        if (!skip) amax = __builtin_fmaxf(amax, __builtin_fabsf(x));
                    }
                }
            }
        };
        if (MODE == 1 && guard) pass1(std::true_type{});
        else pass1(std::false_type{});

        amax = wave_max(amax);
        if (lane == 0) red[it & 1][wave] = amax;
        if constexpr (FMT == 2) {
            nlo = wave_max(nlo);
            if (lane == 0) red2[it & 1][wave] = nlo;
        }
        lds_barrier();
        float a = red[it & 1][w0];
        for (int w = 1; w < nw; ++w) a = __builtin_fmaxf(a, red[it & 1][w0 + w]);
        if constexpr (FMT == 2) {
            // zero-point codes: scale = fl32(fl32(hi - lo) / 255), z = clamp(rne(fl32(-lo / scale)), 0, 255),
            // u = clamp(rne(fl32(x' / scale)) + z, 0, 255), stored as u - 128 with the zero point z - 128
            float b = red2[it & 1][w0];
            for (int w = 1; w < nw; ++w) b = __builtin_fmaxf(b, red2[it & 1][w0 + w]);
            const float sc = (a + b) / 255.0f;   // hi - lo with lo = -b
            int z = 0;
            if (sc != 0.0f) z = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(b / sc), 0.0f, 255.0f);
            if (live) {
                if (tid == 0) {
                    scale[m] = sc;
                    zero[m] = z - 128;
                }
                const double rx = sc != 0.0f ? rcp64((double)sc) : 0.0;
                const float zf = (float)z;
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    if (!valid[i]) continue;
                    const int64_t c = tid + (int64_t)i * tpg;
                    int q[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        // the quotient is exact in the normal range; below it, it rounds to 0 either way
                        const float v = __builtin_rintf((float)((double)xv[i][e] * rx)) + zf;
                        q[e] = sc == 0.0f ? -128 : (int)__builtin_amdgcn_fmed3f(v, 0.0f, 255.0f) - 128;
                    }
                    CodeStore<VEC>::store(Xq + m * K + c * VEC, q);
                }
            }
        }
        const float xs = a / (FMT == 0 ? 127.0f : 448.0f);
        if (FMT != 2 && live) {
            if (tid == 0) scale[m] = xs;
            const double rx = xs != 0.0f ? rcp64((double)xs) : 0.0;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                if (!valid[i]) continue;
                const int64_t c = tid + (int64_t)i * tpg;
                float v[VEC];
                bool zero[VEC];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    zero[e] = xs == 0.0f;
                    if constexpr (OUTL) zero[e] = zero[e] || ((omask[i] >> e) & 1u);
                    v[e] = (float)((double)xv[i][e] * rx);
                }
                store_codes<VEC, FMT>(Xq + m * K + c * VEC, v, zero);
            }
        }
#pragma unroll
        for (int p = 0; p < PF; ++p)
#pragma unroll
            for (int i = 0; i < CH; ++i) buf[p][i] = buf[p + 1][i];
    }
}

// Fallback for rows too long to keep in registers: two passes over the row
// (the second from cache), IEEE divisions.
template <typename T, int MODE, bool OUTL, int FMT>
__global__ __launch_bounds__(1024) void quant_rows_generic(const T* __restrict__ X, int64_t M, int64_t K,
                                                           const float* __restrict__ s, int8_t* __restrict__ Xq,
                                                           float* __restrict__ scale,
                                                           const int32_t* __restrict__ pos,
                                                           _Float16* __restrict__ Xo, int32_t* __restrict__ zero) {
    __shared__ float red[2][16];
    __shared__ float red2[2][16];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int wave = tid >> 6, lane = tid & 63, nwaves = nthr >> 6;
    int it = 0;
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x, ++it) {
        const T* row = X + m * K;
        float amax = 0.0f, nlo = 0.0f;
        for (int64_t j = tid; j < K; j += nthr) {
            float x = (float)row[j];
            if constexpr (MODE == 1) x = x / s[j];
            if constexpr (MODE == 2) x = x * s[j];
            bool skip = false;
            if constexpr (OUTL) {
                int p = pos[j];
                skip = p >= 0;
                if (skip) Xo[m * K + p] = (_Float16)row[j];
            }
            if constexpr (FMT == 2) {
                amax = __builtin_fmaxf(amax, x);
                nlo = __builtin_fmaxf(nlo, -x);
            } else {
                if (!skip) amax = __builtin_fmaxf(amax, __builtin_fabsf(x));
            }
        }
        amax = wave_max(amax);
        if (lane == 0) red[it & 1][wave] = amax;
        if constexpr (FMT == 2) {
            nlo = wave_max(nlo);
            if (lane == 0) red2[it & 1][wave] = nlo;
        }
        __syncthreads();
        float a = red[it & 1][0];
        for (int w = 1; w < nwaves; ++w) a = __builtin_fmaxf(a, red[it & 1][w]);
        if constexpr (FMT == 2) {
            float b = red2[it & 1][0];
            for (int w = 1; w < nwaves; ++w) b = __builtin_fmaxf(b, red2[it & 1][w]);
            const float sc = (a + b) / 255.0f;
            int z = 0;
            if (sc != 0.0f) z = (int)__builtin_amdgcn_fmed3f(__builtin_rintf(b / sc), 0.0f, 255.0f);
            if (tid == 0) {
                scale[m] = sc;
                zero[m] = z - 128;
            }
            for (int64_t j = tid; j < K; j += nthr) {
                float x = (float)row[j];
                if constexpr (MODE == 1) x = x / s[j];
                const float v = __builtin_rintf(x / sc) + (float)z;
                Xq[m * K + j] = (int8_t)(sc == 0.0f ? -128 : (int)__builtin_amdgcn_fmed3f(v, 0.0f, 255.0f) - 128);
            }
            continue;
        }
        const float xs = a / (FMT == 0 ? 127.0f : 448.0f);
        if (tid == 0) scale[m] = xs;
        for (int64_t j = tid; j < K; j += nthr) {
            float x = (float)row[j];
            if constexpr (MODE == 1) x = x / s[j];
            if constexpr (MODE == 2) x = x * s[j];
            bool zero = xs == 0.0f;
            if constexpr (OUTL) zero = zero || pos[j] >= 0;
            if constexpr (FMT == 0) Xq[m * K + j] = (int8_t)(zero ? 0 : code_of(x / xs));
            else Xq[m * K + j] = (int8_t)(fp8x4(zero ? 0.0f : fp8_clamp(x / xs), 0.0f, 0.0f, 0.0f) & 0xffu);
        }
    }
}

template <typename Kern>
static int blocks_per_cu(Kern k, int threads) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, k, threads, 0) != hipSuccess || nb <= 0) nb = 1;
    return nb;
}

template <typename T, int VEC, int CH, int MODE, bool OUTL, int FMT>
static hipError_t launch_fast(const T* X, int64_t M, int64_t K, const float* s, int8_t* Xq, float* scale,
                              const int32_t* pos, _Float16* Xo, int32_t* zero, hipStream_t st) {
    const int64_t nchunk = K / VEC;
    const int tpg = (int)((((nchunk + CH - 1) / CH) + 63) / 64 * 64);   // threads per row group
    const int G = 1024 / tpg;                                          // row groups per block
    const int threads = G * tpg;
    auto k = quant_rows_fast<T, VEC, CH, MODE, OUTL, FMT>;
    // occupancy per block size, computed once (a race between threads only repeats the query)
    static std::atomic<int> nb_cache[1025];
    int nb = nb_cache[threads].load(std::memory_order_relaxed);
    if (nb == 0) {
        nb = blocks_per_cu(k, threads);
        nb_cache[threads].store(nb, std::memory_order_relaxed);
    }
    const int64_t rows_blocks = (M + G - 1) / G;
    const int64_t g = (int64_t)dev_info().cus * nb;
    SQ_LAUNCH(k, dim3((unsigned)(g < rows_blocks ? g : rows_blocks)), dim3(threads), 0, st, X, M, K, s, Xq,
                       scale, pos, Xo, zero, tpg, G);
    return hipSuccess;
}

// Register-resident variants by row length (elements per thread <= 20), else the
// two-pass fallback.
template <typename T, int MODE, bool OUTL, int FMT>
static hipError_t quant_rows_t(const T* X, int64_t M, int64_t K, const float* s, int8_t* Xq, float* scale,
                               const int32_t* pos, _Float16* Xo, hipStream_t st, int32_t* zero = nullptr) {
    if constexpr (sizeof(T) == 2) {
        // one 16-byte chunk per thread (one row per block) when there are few rows: the per-block
        // setup is then split over the most threads
        if (K <= 1024 || (K <= 8192 && M <= dev_info().cus))
            return launch_fast<T, 8, 1, MODE, OUTL, FMT>(X, M, K, s, Xq, scale, pos, Xo, zero, st);
        if (K <= 16384) return launch_fast<T, 8, 2, MODE, OUTL, FMT>(X, M, K, s, Xq, scale, pos, Xo, zero, st);
        if (K <= 20480) return launch_fast<T, 4, 5, MODE, OUTL, FMT>(X, M, K, s, Xq, scale, pos, Xo, zero, st);
    } else {
        if (K <= 4096) return launch_fast<T, 4, 1, MODE, OUTL, FMT>(X, M, K, s, Xq, scale, pos, Xo, zero, st);
        if (K <= 8192) return launch_fast<T, 4, 2, MODE, OUTL, FMT>(X, M, K, s, Xq, scale, pos, Xo, zero, st);
        if (K <= 12288) return launch_fast<T, 4, 3, MODE, OUTL, FMT>(X, M, K, s, Xq, scale, pos, Xo, zero, st);
    }
    auto k = quant_rows_generic<T, MODE, OUTL, FMT>;
    const int64_t g = (int64_t)dev_info().cus * 2;
    SQ_LAUNCH(k, dim3((unsigned)(g < M ? g : M)), dim3(1024), 0, st, X, M, K, s, Xq, scale, pos, Xo, zero);
    return hipSuccess;
}

hipError_t launch_quant_rows(const void* X, int dt, int64_t M, int64_t K, const float* s, int mode,
                             int8_t* Xq, float* scale, const int32_t* pos, _Float16* Xo, hipStream_t st, int fmt,
                             int32_t* zero) {
    const bool outl = pos != nullptr;
    if (fmt == 2) {   // zero-point int8 codes of activation rows (mode 0 or 1, no outlier variant)
        if (dt == SQ_F16) {
            if (mode == 1)
                return quant_rows_t<_Float16, 1, false, 2>((const _Float16*)X, M, K, s, Xq, scale, nullptr, nullptr, st, zero);
            return quant_rows_t<_Float16, 0, false, 2>((const _Float16*)X, M, K, s, Xq, scale, nullptr, nullptr, st, zero);
        }
        if (mode == 1) return quant_rows_t<float, 1, false, 2>((const float*)X, M, K, s, Xq, scale, nullptr, nullptr, st, zero);
        return quant_rows_t<float, 0, false, 2>((const float*)X, M, K, s, Xq, scale, nullptr, nullptr, st, zero);
    }
    if (dt == SQ_F16 && fmt == 0 && !outl && (mode == 0 || mode == 1) && quant_stream_applies(M, K, mode == 1, false))
        return launch_quant_stream(static_cast<const _Float16*>(X), M, K, mode == 1 ? s : nullptr, Xq, scale, nullptr,
                                   st);
    if (dt == SQ_F16 && fmt == 1 && !outl && (mode == 0 || mode == 1) && K <= 4096 &&
        quant_stream_applies(M, K, mode == 1, false))
        return launch_quant_wave_fp8(static_cast<const _Float16*>(X), M, K, mode == 1 ? s : nullptr, Xq, scale, st);
    if (fmt == 1) {   // FP8 E4M3 codes (no outlier variant)
#define SQ_QR8(T, MD) return quant_rows_t<T, MD, false, 1>((const T*)X, M, K, s, Xq, scale, nullptr, nullptr, st)
        if (dt == SQ_F16) {
            if (mode == 1) SQ_QR8(_Float16, 1);
            if (mode == 2) SQ_QR8(_Float16, 2);
            SQ_QR8(_Float16, 0);
        }
        if (mode == 1) SQ_QR8(float, 1);
        if (mode == 2) SQ_QR8(float, 2);
        SQ_QR8(float, 0);
#undef SQ_QR8
    }
#define SQ_QR(T, MD, OL) return quant_rows_t<T, MD, OL, 0>((const T*)X, M, K, s, Xq, scale, pos, Xo, st)
    if (dt == SQ_F16) {
        if (outl) SQ_QR(_Float16, 0, true);
        if (mode == 1) SQ_QR(_Float16, 1, false);
        if (mode == 2) SQ_QR(_Float16, 2, false);
        SQ_QR(_Float16, 0, false);
    } else {
        if (mode == 1) SQ_QR(float, 1, false);
        if (mode == 2) SQ_QR(float, 2, false);
        SQ_QR(float, 0, false);
    }
#undef SQ_QR
}

// ---------------------------------------------------------------------------
// Column absolute maximum (calibration statistic, W column maxima, LLM.int8()
// outlier detection).  Block = 32 chunk-columns x 8 row lanes; each block
// reduces a band of rows and issues one atomic max per column.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void colmax_kernel(const T* __restrict__ X, int64_t M, int64_t K,
                                                     int64_t rows_per_block, uint32_t* __restrict__ amax_bits) {
    using V = typename Chunk<T>::V;
    constexpr int VEC = Chunk<T>::N;
    __shared__ float red[8][32][VEC + 1];
    const int lc = threadIdx.x & 31, lr = threadIdx.x >> 5;
    const int64_t nchunk = K / VEC;
    const int64_t c = (int64_t)blockIdx.x * 32 + lc;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < M ? r0 + rows_per_block : M;
    float mx[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) mx[e] = 0.0f;
    if (c < nchunk) {
        // 8 rows per batch: the loads of a batch are all in flight before the first max
        int64_t r = r0 + lr;
        for (; r + 7 * 8 < r1; r += 8 * 8) {
            V v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const V*>(X + (r + 8 * u) * K + c * VEC);
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int e = 0; e < VEC; ++e) mx[e] = __builtin_fmaxf(mx[e], __builtin_fabsf((float)v[u][e]));
        }
        for (; r < r1; r += 8) {
            V v = *reinterpret_cast<const V*>(X + r * K + c * VEC);
#pragma unroll
            for (int e = 0; e < VEC; ++e) mx[e] = __builtin_fmaxf(mx[e], __builtin_fabsf((float)v[e]));
        }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) red[lr][lc][e] = mx[e];
    __syncthreads();
    if (lr == 0 && c < nchunk) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float m = red[0][lc][e];
            for (int r = 1; r < 8; ++r) m = __builtin_fmaxf(m, red[r][lc][e]);
            atomicMax(&amax_bits[c * VEC + e], __float_as_uint(m));
        }
    }
}

hipError_t launch_colmax(const void* X, int dt, int64_t M, int64_t K, uint32_t* amax_bits, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    const int vec = dt == SQ_F16 ? 8 : 4;
    const int64_t nchunk = K / vec;
    int64_t rpb = 256;
    if ((M + rpb - 1) / rpb > 65535) rpb = (M + 65534) / 65535;   // grid.y limit
    dim3 grid((unsigned)((nchunk + 31) / 32), (unsigned)((M + rpb - 1) / rpb));
    if (dt == SQ_F16)
        SQ_LAUNCH(colmax_kernel<_Float16>, grid, dim3(256), 0, st, (const _Float16*)X, M, K, rpb, amax_bits);
    else
        SQ_LAUNCH(colmax_kernel<float>, grid, dim3(256), 0, st, (const float*)X, M, K, rpb, amax_bits);
    return hipSuccess;
}

// Column absolute maxima of an fp16 matrix, written (not accumulated): block b owns a
// strip of 8L columns over all M rows, so there are no atomics and the output needs no
// zeroing launch beforehand.  Thread t reads 16 bytes (8 columns, chunk t % L of the strip)
// of rows t / L, t / L + 1024 / L, ... four rows at a time; the maxima then meet across
// the wave's lanes of the same chunk (shuffles) and across the 16 waves (LDS).
// Strips sharing a 128-byte line (64 / (8L) of them) go to blocks b, b + 8, ..., which
// the dispatcher places on the same XCD, so each line is fetched into one L2 only.
template <int L>
__global__ __launch_bounds__(1024) void colmax_strip_kernel(const _Float16* __restrict__ X, int64_t M, int64_t K,
                                                            uint32_t* __restrict__ out_bits) {
    constexpr int W = 8 * L;                 // columns per strip
    constexpr int G = 64 / W;                // strips per 128-byte line
    constexpr int R = 1024 / L;              // rows per pass
    __shared__ float red[16][W];
    const int S = (int)((K + W - 1) / W);
    const int b = blockIdx.x;
    const int full = (S / (8 * G)) * (8 * G);
    const int strip = b < full ? G * ((b / (8 * G)) * 8 + b % 8) + (b / 8) % G : b;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = tid % L;
    const int64_t c0 = (int64_t)strip * W + 8 * g;
    float mx[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) mx[e] = 0.0f;
    if (c0 < K) {
        const _Float16* p = X + c0;
        int64_t m = tid / L;
        for (; m + 3 * R < M; m += 4 * R) {
            h8 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(reinterpret_cast<const h8*>(p + (m + u * R) * K));
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) mx[e] = __builtin_fmaxf(mx[e], __builtin_fabsf((float)v[u][e]));
        }
        for (; m < M; m += R) {
            const h8 v = __builtin_nontemporal_load(reinterpret_cast<const h8*>(p + m * K));
#pragma unroll
            for (int e = 0; e < 8; ++e) mx[e] = __builtin_fmaxf(mx[e], __builtin_fabsf((float)v[e]));
        }
    }
    // lanes of one chunk differ in lane bits log2(L) and up
#pragma unroll
    for (int off = L; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) mx[e] = __builtin_fmaxf(mx[e], __shfl_xor(mx[e], off, 64));
    if (lane < L)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][8 * lane + e] = mx[e];
    __syncthreads();
    if (tid < W && (int64_t)strip * W + tid < K) {
        float a = red[0][tid];
#pragma unroll
        for (int w = 1; w < 16; ++w) a = __builtin_fmaxf(a, red[w][tid]);
        out_bits[(int64_t)strip * W + tid] = __float_as_uint(a);
    }
}

hipError_t launch_colmax_fresh(const _Float16* X, int64_t M, int64_t K, uint32_t* out_bits, hipStream_t st) {
    const int64_t cus = dev_info().cus;
    // the widest strip that still gives every CU a block
    if (K / 32 >= cus)
        SQ_LAUNCH(colmax_strip_kernel<4>, dim3((unsigned)((K + 31) / 32)), dim3(1024), 0, st, X, M, K, out_bits);
    else if (K / 16 >= cus)
        SQ_LAUNCH(colmax_strip_kernel<2>, dim3((unsigned)(K / 16)), dim3(1024), 0, st, X, M, K, out_bits);
    else
        SQ_LAUNCH(colmax_strip_kernel<1>, dim3((unsigned)(K / 8)), dim3(1024), 0, st, X, M, K, out_bits);
    return hipSuccess;
}

// Row sums of an int8 matrix (the weight term of the zero-point correction, computed once
// per weight): one wave per row, 16 bytes per lane per step, then a wave sum.
__global__ __launch_bounds__(256) void rowsum_kernel(const int8_t* __restrict__ Wq, int64_t N, int64_t K,
                                                     int32_t* __restrict__ rowsum) {
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (n >= N) return;   // wave-uniform
    const v4i* row = reinterpret_cast<const v4i*>(Wq + n * K);
    int t = 0;
    for (int64_t c = lane; c < K / 16; c += 64) {
        const v4i v = row[c];
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
            for (int b = 0; b < 4; ++b) t += (int)(int8_t)((uint32_t)v[w] >> (8 * b));
    }
    t = wave_sum_int(t);
    if (lane == 0) rowsum[n] = t;
}

hipError_t launch_weight_rowsum(const int8_t* Wq, int64_t N, int64_t K, int32_t* rowsum, hipStream_t st) {
    SQ_LAUNCH(rowsum_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, st, Wq, N, K, rowsum);
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Smoothing factors: s_j = max(a_j,1e-8)^alpha / max(w_j,1e-8)^(1-alpha) in fp64.
// ---------------------------------------------------------------------------
__global__ void smooth_pow_kernel(const float* __restrict__ act_max, float* __restrict__ s_wmax, int64_t K,
                                  float alpha) {
    int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (j >= K) return;
    float a = act_max[j];
    float w = s_wmax[j];
    a = a > 1e-8f ? a : 1e-8f;
    w = w > 1e-8f ? w : 1e-8f;
    double al = (double)alpha;
    s_wmax[j] = (float)(pow((double)a, al) / pow((double)w, 1.0 - al));
}

hipError_t launch_smooth_pow(const float* act_max, float* s_wmax, int64_t K, float alpha, hipStream_t st) {
    SQ_LAUNCH(smooth_pow_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, act_max, s_wmax, K,
                       alpha);
    return hipSuccess;
}

// ---------------------------------------------------------------------------
// Per-tensor weight quantization: pass 1 global max of |W * s|, pass 2 codes.
// ---------------------------------------------------------------------------
template <typename T, bool SMOOTH>
__global__ __launch_bounds__(256) void tensor_max_kernel(const T* __restrict__ W, int64_t nchunks, int64_t kchunks,
                                                         const float* __restrict__ s, uint32_t* __restrict__ gmax) {
    using V = typename Chunk<T>::V;
    constexpr int VEC = Chunk<T>::N;
    __shared__ float red[4];
    float m = 0.0f;
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * blockDim.x) {
        V v = reinterpret_cast<const V*>(W)[c];
        int64_t jc = c % kchunks;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float x = (float)v[e];
            if constexpr (SMOOTH) x = x * s[jc * VEC + e];
            m = __builtin_fmaxf(m, __builtin_fabsf(x));
        }
    }
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float a = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
        atomicMax(gmax, __float_as_uint(a));
    }
}

template <typename T, bool SMOOTH, int FMT>
__global__ __launch_bounds__(256) void tensor_code_kernel(const T* __restrict__ W, int64_t nchunks, int64_t kchunks,
                                                          const float* __restrict__ s,
                                                          const uint32_t* __restrict__ gmax,
                                                          int8_t* __restrict__ Wq, float* __restrict__ w_scale) {
    using V = typename Chunk<T>::V;
    constexpr int VEC = Chunk<T>::N;
    const float sc = __uint_as_float(*gmax) / (FMT == 0 ? 127.0f : 448.0f);
    const double rx = sc != 0.0f ? rcp64((double)sc) : 0.0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *w_scale = sc;
    for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * blockDim.x) {
        V v = reinterpret_cast<const V*>(W)[c];
        int64_t jc = c % kchunks;
        float q[VEC];
        bool zero[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float x = (float)v[e];
            if constexpr (SMOOTH) x = x * s[jc * VEC + e];
            zero[e] = sc == 0.0f;
            q[e] = div_rcp64(x, rx, sc);
        }
        store_codes<VEC, FMT>(Wq + c * VEC, q, zero);
    }
}

template <typename T, int FMT>
static hipError_t quant_tensor_t(const T* W, int64_t N, int64_t K, const float* s, int8_t* Wq, float* w_scale,
                                 uint32_t* gmax, hipStream_t st) {
    constexpr int VEC = Chunk<T>::N;
    const int64_t kchunks = K / VEC, nchunks = N * kchunks;
    int64_t blocks = (nchunks + 255) / 256;
    const int64_t cap = (int64_t)dev_info().cus * 8;
    if (blocks > cap) blocks = cap;
    if (s) {
        SQ_LAUNCH((tensor_max_kernel<T, true>), dim3((unsigned)blocks), dim3(256), 0, st, W, nchunks, kchunks, s, gmax);
        SQ_LAUNCH((tensor_code_kernel<T, true, FMT>), dim3((unsigned)blocks), dim3(256), 0, st, W, nchunks, kchunks, s, gmax, Wq, w_scale);
    } else {
        SQ_LAUNCH((tensor_max_kernel<T, false>), dim3((unsigned)blocks), dim3(256), 0, st, W, nchunks, kchunks, s, gmax);
        SQ_LAUNCH((tensor_code_kernel<T, false, FMT>), dim3((unsigned)blocks), dim3(256), 0, st, W, nchunks, kchunks, s, gmax, Wq, w_scale);
    }
    return hipSuccess;
}

hipError_t launch_quant_tensor(const void* W, int dt, int64_t N, int64_t K, const float* s, int8_t* Wq,
                               float* w_scale, uint32_t* gmax_bits, hipStream_t st, int fmt) {
    if (fmt == 1) {
        if (dt == SQ_F16) return quant_tensor_t<_Float16, 1>((const _Float16*)W, N, K, s, Wq, w_scale, gmax_bits, st);
        return quant_tensor_t<float, 1>((const float*)W, N, K, s, Wq, w_scale, gmax_bits, st);
    }
    if (dt == SQ_F16) return quant_tensor_t<_Float16, 0>((const _Float16*)W, N, K, s, Wq, w_scale, gmax_bits, st);
    return quant_tensor_t<float, 0>((const float*)W, N, K, s, Wq, w_scale, gmax_bits, st);
}

}  // namespace sq
