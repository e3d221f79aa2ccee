// LayerNorm with the SmoothQuant division folded into its weights, fused with
// per-token int8 quantization ["SmoothQuant量化实战", sections 2.3, 4.2 and 4.5:
// the per-channel X/s is absorbed into the output of the preceding LayerNorm,
// so it costs nothing per forward].
//
// Offline: gamma' = fl32(gamma / s), beta' = fl32(beta / s).
// Per forward, for each row of X (binary16, K values):
//   every finite x is n * 2^-24 with an integer n, |n| < 2^40, so
//   S1 = sum n (int64) and S2 = sum n^2 (128-bit, accumulated as two exact fp64
//   sums) are exact and independent of the order of summation;
//   mu   = fl64( fl64(S1) / (K * 2^24) )
//   var  = fl64( fl64(K*S2 - S1^2) / (K^2 * 2^48) )          population variance
//   rstd = fl64( 1 / fl64(sqrt( fl64(var + eps) )) )
//   z_j  = fl32( fl32(x_j - fl32(mu)) * fl32(rstd) )
//   y_j  = fl32( fl32(z_j * gamma'_j) + beta'_j )             (no add without beta)
//   xs   = fl32( max_j |y_j| / 127 ),  q_j = clamp(rne(fl32(y_j / xs)), -128, 127)
// (q = 0 and xs = 0 for an all-zero y).  HBM-bound: 2 B read and 1 B written per
// element, 4 B per row for the scale.
//
// Layout: rows up to 16384 values are held in registers by groups of threads
// (one 16-byte chunk per thread and pass, one or two passes); each row needs
// two block reductions (the integer sums, then the absolute maximum).  Longer
// rows take one block per row and three passes over the row (sums, maximum,
// codes), reading it from L2 the second and third time.
#include "sq_internal.h"

namespace sq {

namespace {

// Barrier for LDS traffic only (does not wait for the row prefetch).
__device__ __forceinline__ void lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Partial sums of one thread.  Each binary16 x is n * 2^-24 for an integer n with at
// most 11 significant bits (|n| < 2^40).  S1 = sum n: a thread adds at most 2^13
// values, so the fp64 sum of x * 2^24 stays an integer below 2^53 and is exact.
// S2 = sum n^2: n^2 has at most 22 significant bits, so it is exact in fp64, and it is
// split exactly into q * 2^40 + r with q = floor(n^2 / 2^40) and r = n^2 - q 2^40,
// both integers below 2^40; their per-thread sums stay below 2^53, exact in fp64.
// Before the cross-lane reduction the thread's sums become integers: S1 in int64 and
// S2 = Q 2^40 + R as a 128-bit (hi, lo) pair.
struct Sums {
    int64_t s1;
    uint64_t lo, hi;
};

struct Acc {
    double s1, q, r;
};

__device__ __forceinline__ void add_half(Acc& t, float x) {
    const double n = (double)x * 0x1p24;                       // exact
    t.s1 += n;
    const double n2 = n * n;                                   // exact (22 significant bits)
    const double q = __builtin_floor(n2 * 0x1p-40);            // exact
    t.q += q;
    t.r += __builtin_fma(-q, 0x1p40, n2);                      // exact: n^2 - q 2^40 in [0, 2^40)
}

__device__ __forceinline__ Sums to_sums(const Acc& a) {
    const uint64_t q = (uint64_t)a.q, r = (uint64_t)a.r;      // exact integers below 2^53
    const uint64_t lo = (q << 40) + r;
    return Sums{(int64_t)a.s1, lo, (q >> 24) + (lo < r ? 1u : 0u)};
}

__device__ __forceinline__ Sums wave_sums(Sums t) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const int64_t s1 = __shfl_xor(t.s1, off, 64);
        const uint64_t lo = __shfl_xor(t.lo, off, 64), hi = __shfl_xor(t.hi, off, 64);
        t.s1 += s1;
        const uint64_t nl = t.lo + lo;
        t.hi += hi + (nl < lo ? 1u : 0u);
        t.lo = nl;
    }
    return t;
}

__device__ __forceinline__ void add_sums(Sums& t, const Sums& o) {
    t.s1 += o.s1;
    const uint64_t nl = t.lo + o.lo;
    t.hi += o.hi + (nl < o.lo ? 1u : 0u);
    t.lo = nl;
}

// Round-to-nearest-even conversions of exact integers: the two halves of a
// 64-bit value are exact doubles, so their sum rounds once; a 128-bit value is
// first cut to its top 64 bits with the dropped bits folded into bit 0 (far
// below the rounding position of a 53-bit significand).
__device__ __forceinline__ double u64_to_f64(uint64_t x) {
    return (double)(uint32_t)(x >> 32) * 0x1p32 + (double)(uint32_t)x;
}
__device__ __forceinline__ double u128_to_f64(unsigned __int128 v) {
    const uint64_t hi = (uint64_t)(v >> 64);
    if (hi == 0) return u64_to_f64((uint64_t)v);
    const int sh = 64 - __builtin_clzll(hi);
    uint64_t top = (uint64_t)(v >> sh);
    top |= (uint64_t)((v << (128 - sh)) != 0);
    return __builtin_ldexp(u64_to_f64(top), sh);
}

// Row statistics from the exact sums (same operation sequence on every thread).
__device__ __forceinline__ void row_stats(const Sums& t, int64_t K, float eps, float& mu32, float& r32) {
    const unsigned __int128 s2 = ((unsigned __int128)t.hi << 64) | t.lo;
    const uint64_t as1 = t.s1 < 0 ? (uint64_t)(-t.s1) : (uint64_t)t.s1;
    const unsigned __int128 v = (unsigned __int128)(uint64_t)K * s2 - (unsigned __int128)as1 * as1;
    const double d1 = t.s1 < 0 ? -u64_to_f64(as1) : u64_to_f64(as1);
    const double mu = d1 / ((double)K * 0x1p24);
    const double var = u128_to_f64(v) / (((double)K * (double)K) * 0x1p48);
    const double rstd = 1.0 / __builtin_sqrt(var + (double)eps);
    mu32 = (float)mu;
    r32 = (float)rstd;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

struct U16x8 {
    uint16_t v[8];
};

// binary16 bit pattern e (0..7) of a 16-byte chunk held as four dwords
__device__ __forceinline__ uint16_t hbits(const v4i& c, int e) {
    return (uint16_t)((uint32_t)c[e >> 1] >> (16 * (e & 1)));
}

// One wave per row (rows up to 8192 values): lane l holds the 16-byte chunks
// l, l + 64, ... (CPL of them), so the two row reductions are wave shuffles and
// the waves of a CU run independently (no block barrier after the prologue).
// gamma' and beta' sit in LDS; the normalised values are computed twice (for the
// row maximum, then for the codes) instead of being kept in registers.  With
// PF, each wave loads its next row while it works on the current one.
template <int CPL, bool BETA, bool PF>
__global__ __launch_bounds__(256) void ln_quant_wave(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                     const float* __restrict__ gamma,
                                                     const float* __restrict__ beta, float eps,
                                                     int8_t* __restrict__ Xq, float* __restrict__ scale) {
    extern __shared__ v4f sgb[];             // gamma' [K], then beta' [K]
    const v4f* sg = sgb;
    const v4f* sb = sgb + K / 4;
    for (int64_t j = threadIdx.x; j < K / 4; j += blockDim.x) {
        sgb[j] = reinterpret_cast<const v4f*>(gamma)[j];
        if constexpr (BETA) sgb[K / 4 + j] = reinterpret_cast<const v4f*>(beta)[j];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wpb = blockDim.x >> 6;
    const int64_t nwv = (int64_t)gridDim.x * wpb;
    const int nchunk = (int)(K / 8);
    int64_t m = (int64_t)blockIdx.x * wpb + (threadIdx.x >> 6);   // uniform per wave
    v4i cur[CPL], nxt[PF ? CPL : 1];
    auto load = [&](int64_t row, v4i* r) {
        const v4i* src = reinterpret_cast<const v4i*>(X + row * K);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            r[i] = (row < M && c < nchunk) ? src[c] : v4i{0, 0, 0, 0};
        }
    };
    load(m, cur);
    // y for the 8 values of chunk c (clamped into the row for the LDS reads; chunks past
    // the row end are computed on zeros and never used)
    uint32_t lbase = 0;                       // LDS offset, re-read per row (see below)
    auto yval = [&](const v4i& h, int c, float mu, float rs, float* y) {
        const int cc = (c < nchunk ? c : 0) + (int)lbase;
        const v4f g0 = sg[2 * cc], g1 = sg[2 * cc + 1];
        v4f b0{}, b1{};
        if constexpr (BETA) {
            b0 = sb[2 * cc];
            b1 = sb[2 * cc + 1];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = ((half_bits_to_float(hbits(h, e)) - mu) * rs) * (e < 4 ? g0[e] : g1[e - 4]);
            if constexpr (BETA) v = v + (e < 4 ? b0[e] : b1[e - 4]);
            y[e] = v;
        }
    };
    for (; m < M; m += nwv) {
        // an opaque zero: keeps the compiler from hoisting every gamma'/beta' read out of
        // the row loop into registers (which would cost the occupancy that hides latency)
        asm volatile("" : "+s"(lbase));
        if constexpr (PF) load(m + nwv, nxt);
        Acc ta{0.0, 0.0, 0.0};
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
#pragma unroll
            for (int e = 0; e < 8; ++e) add_half(ta, half_bits_to_float(hbits(cur[i], e)));   // zeros add nothing
            __builtin_amdgcn_sched_barrier(0);
        }
        const Sums t = wave_sums(to_sums(ta));
        float mu, rs;
        row_stats(t, K, eps, mu, rs);
        constexpr bool KEEP = CPL <= 8;           // keep y in registers for the code pass
        float yk[KEEP ? CPL : 1][8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            float* y = yk[KEEP ? i : 0];
            yval(cur[i], c, mu, rs, y);
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(y[e]));
            amax = c < nchunk ? __builtin_fmaxf(amax, a) : amax;
            __builtin_amdgcn_sched_barrier(0);   // one chunk's values live at a time
        }
        amax = wave_max(amax);
        const float xs = amax / 127.0f;
        if (lane == 0) scale[m] = xs;
        const double rx = xs != 0.0f ? rcp64((double)xs) : 0.0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            float* y = yk[KEEP ? i : 0];
            if (!KEEP) yval(cur[i], c, mu, rs, y);
            int q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = xs == 0.0f ? 0 : code_of((float)((double)y[e] * rx));
            const uint32_t lo = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                                ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
            const uint32_t hi = (uint32_t)(q[4] & 0xff) | ((uint32_t)(q[5] & 0xff) << 8) |
                                ((uint32_t)(q[6] & 0xff) << 16) | ((uint32_t)(q[7] & 0xff) << 24);
            if (c < nchunk) *reinterpret_cast<uint2*>(Xq + m * K + c * 8) = make_uint2(lo, hi);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (PF) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) cur[i] = nxt[i];
        } else {
            load(m + nwv, cur);
        }
    }
}

// Register-resident rows: CH 16-byte chunks per thread per row.
template <int CH, bool BETA>
__global__ __launch_bounds__(1024) void ln_quant_rows(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ beta, float eps,
                                                      int8_t* __restrict__ Xq, float* __restrict__ scale, int tpg,
                                                      int G) {
    __shared__ Sums sred[2][16];
    __shared__ float fred[2][16];
    const int g = threadIdx.x / tpg;          // row group
    const int tid = threadIdx.x - g * tpg;    // thread within the group
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int w0 = (g * tpg) >> 6, nw = tpg >> 6;
    const int64_t nchunk = K / 8;

    bool valid[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) valid[i] = tid + (int64_t)i * tpg < nchunk;
    v4i buf[2][CH];
    auto load_row = [&](int64_t row, v4i* r) {
        const v4i* src = reinterpret_cast<const v4i*>(X + row * K);
#pragma unroll
        for (int i = 0; i < CH; ++i) r[i] = (valid[i] && row < M) ? src[tid + (int64_t)i * tpg] : v4i{0, 0, 0, 0};
    };
    const int64_t step = (int64_t)gridDim.x * G;
    int64_t m = (int64_t)blockIdx.x * G + g;
    load_row(m, buf[0]);
    // per-column weights, while the first row is in flight
    float gv[CH][8], bv[BETA ? CH : 1][8];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
        const int64_t c = valid[i] ? tid + (int64_t)i * tpg : 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gv[i][e] = gamma[c * 8 + e];
            if constexpr (BETA) bv[i][e] = beta[c * 8 + e];
        }
    }
    const int64_t first = (int64_t)blockIdx.x * G;
    const int64_t iters = first < M ? (M - first + step - 1) / step : 0;   // equal for every group
    for (int64_t it = 0; it < iters; ++it, m += step) {
        const int p = (int)(it & 1);         // LDS buffer parity
        load_row(m + step, buf[1]);          // next row, in flight during this one
        const bool live = m < M;
        U16x8 h[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) h[i] = __builtin_bit_cast(U16x8, buf[0][i]);
        // exact integer sums
        Acc ta{0.0, 0.0, 0.0};
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) add_half(ta, half_bits_to_float(h[i].v[e]));   // zeros for invalid chunks
        Sums t = wave_sums(to_sums(ta));
        if (lane == 0) sred[p][wave] = t;
        lds_sync();
        Sums r = sred[p][w0];
        for (int w = 1; w < nw; ++w) add_sums(r, sred[p][w0 + w]);
        float mu, rs;
        row_stats(r, K, eps, mu, rs);
        // normalise, scale, shift; row maximum
        float y[CH][8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < CH; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float z = (half_bits_to_float(h[i].v[e]) - mu) * rs;
                float v = z * gv[i][e];
                if constexpr (BETA) v = v + bv[i][e];
                y[i][e] = v;
                if (valid[i]) amax = __builtin_fmaxf(amax, __builtin_fabsf(v));
            }
        amax = wave_max(amax);
        if (lane == 0) fred[p][wave] = amax;
        lds_sync();
        float a = fred[p][w0];
        for (int w = 1; w < nw; ++w) a = __builtin_fmaxf(a, fred[p][w0 + w]);
        const float xs = a / 127.0f;
        if (live) {
            if (tid == 0) scale[m] = xs;
            const double rx = xs != 0.0f ? rcp64((double)xs) : 0.0;
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                if (!valid[i]) continue;
                int q[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) q[e] = xs == 0.0f ? 0 : code_of((float)((double)y[i][e] * rx));
                const uint32_t lo = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                                    ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
                const uint32_t hi = (uint32_t)(q[4] & 0xff) | ((uint32_t)(q[5] & 0xff) << 8) |
                                    ((uint32_t)(q[6] & 0xff) << 16) | ((uint32_t)(q[7] & 0xff) << 24);
                *reinterpret_cast<uint2*>(Xq + m * K + (tid + (int64_t)i * tpg) * 8) = make_uint2(lo, hi);
            }
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) buf[0][i] = buf[1][i];
    }
}

// Rows too long for registers: one block per row, three passes over the row.
template <bool BETA>
__global__ __launch_bounds__(1024) void ln_quant_long(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ beta, float eps,
                                                      int8_t* __restrict__ Xq, float* __restrict__ scale) {
    __shared__ Sums sred[16];
    __shared__ float fred[16];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int64_t nchunk = K / 8;
    for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
        const v4i* src = reinterpret_cast<const v4i*>(X + m * K);
        Sums t{0, 0, 0};
        for (int64_t c0 = threadIdx.x; c0 < nchunk; c0 += 16 * (int64_t)blockDim.x) {
            Acc ta{0.0, 0.0, 0.0};             // at most 128 values per fp64 partial sum
            for (int64_t c = c0; c < nchunk && c < c0 + 16 * (int64_t)blockDim.x; c += blockDim.x) {
                const U16x8 h = __builtin_bit_cast(U16x8, src[c]);
#pragma unroll
                for (int e = 0; e < 8; ++e) add_half(ta, half_bits_to_float(h.v[e]));
            }
            add_sums(t, to_sums(ta));
        }
        t = wave_sums(t);
        __syncthreads();                      // the previous row is done with sred/fred
        if (lane == 0) sred[wave] = t;
        __syncthreads();
        Sums r = sred[0];
        for (int w = 1; w < nw; ++w) add_sums(r, sred[w]);
        float mu, rs;
        row_stats(r, K, eps, mu, rs);
        auto yval = [&](uint16_t hb, int64_t j) {
            float v = ((half_bits_to_float(hb) - mu) * rs) * gamma[j];
            if constexpr (BETA) v = v + beta[j];
            return v;
        };
        float amax = 0.0f;
        for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
            const U16x8 h = __builtin_bit_cast(U16x8, src[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(yval(h.v[e], c * 8 + e)));
        }
        amax = wave_max(amax);
        if (lane == 0) fred[wave] = amax;
        __syncthreads();
        float a = fred[0];
        for (int w = 1; w < nw; ++w) a = __builtin_fmaxf(a, fred[w]);
        const float xs = a / 127.0f;
        if (threadIdx.x == 0) scale[m] = xs;
        const double rx = xs != 0.0f ? rcp64((double)xs) : 0.0;
        for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
            const U16x8 h = __builtin_bit_cast(U16x8, src[c]);
            int q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = xs == 0.0f ? 0 : code_of((float)((double)yval(h.v[e], c * 8 + e) * rx));
            const uint32_t lo = (uint32_t)(q[0] & 0xff) | ((uint32_t)(q[1] & 0xff) << 8) |
                                ((uint32_t)(q[2] & 0xff) << 16) | ((uint32_t)(q[3] & 0xff) << 24);
            const uint32_t hi = (uint32_t)(q[4] & 0xff) | ((uint32_t)(q[5] & 0xff) << 8) |
                                ((uint32_t)(q[6] & 0xff) << 16) | ((uint32_t)(q[7] & 0xff) << 24);
            *reinterpret_cast<uint2*>(Xq + m * K + c * 8) = make_uint2(lo, hi);
        }
    }
}

__global__ void fold_kernel(const float* __restrict__ gamma, const float* __restrict__ beta,
                            const float* __restrict__ s, int64_t K, float* __restrict__ gamma_out,
                            float* __restrict__ beta_out) {
    for (int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; j < K; j += (int64_t)gridDim.x * blockDim.x) {
        gamma_out[j] = gamma[j] / s[j];
        if (beta) beta_out[j] = beta[j] / s[j];
    }
}

template <int CH, bool BETA>
hipError_t launch_rows(const uint16_t* X, int64_t M, int64_t K, const float* gamma, const float* beta, float eps,
                       int8_t* Xq, float* scale, hipStream_t st) {
    const int64_t nchunk = K / 8;
    const int tpg = (int)((((nchunk + CH - 1) / CH) + 63) / 64 * 64);   // threads per row group
    const int G = 1024 / tpg;                                          // row groups per block
    const int64_t rows_blocks = (M + G - 1) / G;
    const int64_t cap = (int64_t)dev_info().cus;                       // one 1024-thread block per CU
    SQ_LAUNCH((ln_quant_rows<CH, BETA>), dim3((unsigned)(rows_blocks < cap ? rows_blocks : cap)),
                       dim3(G * tpg), 0, st, X, M, K, gamma, beta, eps, Xq, scale, tpg, G);
    return hipSuccess;
}

template <int CPL, bool BETA, bool PF>
hipError_t launch_wave(const uint16_t* X, int64_t M, int64_t K, const float* gamma, const float* beta, float eps,
                       int8_t* Xq, float* scale, hipStream_t st) {
    constexpr int kWaves = 4;                                          // rows in flight per block
    const int64_t blocks = (M + kWaves - 1) / kWaves;
    const int64_t cap = (int64_t)dev_info().cus * 8;
    const size_t lds = (size_t)K * sizeof(float) * (BETA ? 2 : 1);
    SQ_LAUNCH((ln_quant_wave<CPL, BETA, PF>), dim3((unsigned)(blocks < cap ? blocks : cap)),
                       dim3(64 * kWaves), lds, st, X, M, K, gamma, beta, eps, Xq, scale);
    return hipSuccess;
}

template <bool BETA>
hipError_t launch_ln(const uint16_t* X, int64_t M, int64_t K, const float* gamma, const float* beta, float eps,
                     int8_t* Xq, float* scale, hipStream_t st) {
    // few rows: spread each row over a group of threads (up to 1024) instead of one wave
    if (K <= 8192 && M < 4 * (int64_t)dev_info().cus)
        return launch_rows<1, BETA>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 512) return launch_wave<1, BETA, true>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 1024) return launch_wave<2, BETA, true>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 2048) return launch_wave<4, BETA, true>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 4096) return launch_wave<8, BETA, true>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 8192) return launch_wave<16, BETA, false>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 16384) return launch_rows<2, BETA>(X, M, K, gamma, beta, eps, Xq, scale, st);
    const int64_t cap = (int64_t)dev_info().cus * 2;
    SQ_LAUNCH((ln_quant_long<BETA>), dim3((unsigned)(M < cap ? M : cap)), dim3(1024), 0, st, X, M, K,
                       gamma, beta, eps, Xq, scale);
    return hipSuccess;
}

}  // namespace

hipError_t launch_ln_quant(const _Float16* X, int64_t M, int64_t K, const float* gamma, const float* beta, float eps,
                           int8_t* Xq, float* scale, hipStream_t st) {
    const uint16_t* Xb = reinterpret_cast<const uint16_t*>(X);
    if (beta) return launch_ln<true>(Xb, M, K, gamma, beta, eps, Xq, scale, st);
    return launch_ln<false>(Xb, M, K, gamma, beta, eps, Xq, scale, st);
}

hipError_t launch_fold_layernorm(const float* gamma, const float* beta, const float* s, int64_t K, float* gamma_out,
                                 float* beta_out, hipStream_t st) {
    const int64_t blocks = (K + 255) / 256;
    SQ_LAUNCH(fold_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0, st, gamma, beta,
                       s, K, gamma_out, beta_out);
    return hipSuccess;
}

}  // namespace sq
