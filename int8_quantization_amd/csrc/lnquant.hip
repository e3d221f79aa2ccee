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
// (q = 0 and xs = 0 for an all-zero y).  2 B read and 1 B written per element, 4 B
// per row for the scale; with the exact sums and the fp64 quotient, about 20 vector
// instructions per element, so the kernels are bound by vector ALU issue rather than
// by HBM.
//
// Layout: with at least four rows per CU and rows up to 8192 values, one wave per row
// (ln_quant_wave: both reductions inside the wave).  Fewer rows, or rows up to 16384
// values: a group of up to 1024 threads per row, values held in registers, two block
// reductions per row (ln_quant_rows).  Longer rows: one block per row and three passes
// over the row (sums, maximum, codes), reading it from L2 the second and third time
// (ln_quant_long).
#include "sq_internal.h"

namespace sq {

namespace {

typedef unsigned int v2u __attribute__((ext_vector_type(2)));

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

// Lane-to-lane copy of an fp64 value through DPP (CTRL is the dpp_ctrl code); every
// lane of the wave must be active.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ double readlane_f64(double x, int l) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum over the wave of fp64 values whose every partial sum is exact (integer multiples
// of one power of two below 2^53 times it), so the order does not matter: the quad
// swaps, the half-row and row mirrors give each row of 16 lanes its sum, and the four
// row sums are read out and added.  All 64 lanes must be active.
__device__ __forceinline__ double wave_sum_exact(double v) {
    v += dpp_f64<0xB1>(v);    // quad_perm 1,0,3,2
    v += dpp_f64<0x4E>(v);    // quad_perm 2,3,0,1
    v += dpp_f64<0x141>(v);   // row_half_mirror
    v += dpp_f64<0x140>(v);   // row_mirror
    return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Four codes, each the low byte of fl32(t + 1.5 2^23) for t = clamp(q, -128, 127): the
// add rounds t to the nearest integer, ties to even, into the low mantissa bits (the
// same code as clamping the rounded q); v_perm_b32 gathers the four low bytes.
__device__ __forceinline__ uint32_t pack_codes(float q0, float q1, float q2, float q3) {
    auto rb = [](float q) {
        return __float_as_uint(__builtin_amdgcn_fmed3f(q, -128.0f, 127.0f) + 12582912.0f);
    };
    const uint32_t a = __builtin_amdgcn_perm(rb(q1), rb(q0), 0x0c0c0400u);   // bytes q0, q1, 0, 0
    const uint32_t b = __builtin_amdgcn_perm(rb(q3), rb(q2), 0x0c0c0400u);   // bytes q2, q3, 0, 0
    return __builtin_amdgcn_perm(b, a, 0x05040100u);                          // q0, q1, q2, q3
}

// One wave per row (rows up to 8192 values): lane l holds the 16-byte chunks l, l + 64,
// ... (CPL of them), so the two row reductions stay inside the wave and the waves of a
// CU run independently (one block barrier, after the prologue).  gamma' and beta' sit
// in LDS; the prologue issues the first row's loads before it waits for the weights.
//
// Row sums, in units of x (each binary16 x is n 2^-24, |n| < 2^40): S1 = sum x, and
// x^2 (exact in fp64: 22 significant bits) split as q 2^-8 + r with q = floor(x^2 2^8)
// and r = x^2 - q 2^-8 in [0, 2^-8), a multiple of 2^-48.  Over a row of at most 8192
// values every partial sum of x, of q and of r is an integer multiple of 2^-24, 1 and
// 2^-48 below 2^53 times it, so the fp64 sums are exact in any order; then
// S1 = 2^24 sum x and S2 = sum n^2 = 2^40 sum q + 2^48 sum r as a 128-bit integer.
//
// Up to 4096 values per row (KEEP), the values stay in registers as fp32 from the sums
// to the codes, and the next row's loads are issued as soon as the current row has been
// converted; longer rows are read again from the chunk registers for the maximum and
// for the codes.
template <int CPL, bool BETA>
__global__ __launch_bounds__(256) void ln_quant_wave(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                     const float* __restrict__ gamma,
                                                     const float* __restrict__ beta, float eps,
                                                     int8_t* __restrict__ Xq, float* __restrict__ scale) {
    constexpr int kThreads = 256, kWaves = kThreads / 64;
    constexpr bool KEEP = CPL <= 8;
    extern __shared__ v4f sgb[];             // gamma' [K], then beta' [K]
    const int lane = threadIdx.x & 63;
    const int64_t nwv = (int64_t)gridDim.x * kWaves;
    const int nchunk = (int)(K / 8);
    const int nv4 = (int)(K / 4);
    int64_t m = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    // rows through buffer resources: a read past the row (or of a row past M, whose
    // record count is 0) returns zeros, a write there is dropped
    auto row_rsrc = [&](const void* base, int64_t row, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, row < M ? bytes : 0, 0x00020000);
    };
    auto load = [&](int64_t row, v4i* r) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(X + (row < M ? row : 0) * K, row, (int)(2 * K));
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            r[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (lane + 64 * i), 0, 0));
    };
    // gamma'/beta' (K/4 <= 128 CPL vectors each): every thread loads FPT vectors of each
    // (index clamped into the array) and writes them to LDS unconditionally (slots past K/4
    // are slack, never read).  The weight loads are issued before the first row's loads, so
    // the LDS writes and the barrier wait for the weights only, not for the row.
    constexpr int FPT = (CPL + 1) / 2;
    constexpr int NW = kThreads * FPT;       // LDS vectors per array
    v4f fg[FPT], fb[BETA ? FPT : 1];
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
        const int j = (int)threadIdx.x + kThreads * i;
        const int jj = j < nv4 ? j : nv4 - 1;
        fg[i] = reinterpret_cast<const v4f*>(gamma)[jj];
        if constexpr (BETA) fb[i] = reinterpret_cast<const v4f*>(beta)[jj];
    }
    __builtin_amdgcn_sched_barrier(0);
    v4i cur[CPL];
    load(m, cur);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
        const int j = (int)threadIdx.x + kThreads * i;
        sgb[j] = fg[i];
        if constexpr (BETA) sgb[NW + j] = fb[i];
    }
    lds_sync();
    const v4f* sg = sgb;
    const v4f* sb = sgb + NW;
    uint32_t lbase = 0;                       // LDS offset, re-read per row (see below)
    // y for the 8 values of chunk c, from their fp32 values (chunks past the row end read
    // the weights of chunk 0 and are never used)
    auto yval = [&](const float* x, int c, float mu, float rs, float* y) {
        const int cc = (c < nchunk ? c : 0) + (int)lbase;
        const v4f g0 = sg[2 * cc], g1 = sg[2 * cc + 1];
        v4f b0{}, b1{};
        if constexpr (BETA) {
            b0 = sb[2 * cc];
            b1 = sb[2 * cc + 1];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = ((x[e] - mu) * rs) * (e < 4 ? g0[e] : g1[e - 4]);
            if constexpr (BETA) v = v + (e < 4 ? b0[e] : b1[e - 4]);
            y[e] = v;
        }
    };
    auto xval = [&](const v4i& h, float* x) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = half_bits_to_float(hbits(h, e));
    };
    // the first row's pass runs on every wave (a wave without a row reads zeros, and its
    // code stores are dropped), so that its loads stay ahead of the barrier above
    do {
        // an opaque zero: keeps the compiler from hoisting every gamma'/beta' read out of
        // the row loop into registers (which would cost the occupancy that hides latency)
        asm volatile("" : "+s"(lbase));
        float xk[KEEP ? CPL : 1][8];
        double s1 = -0.0, sq = -0.0, sr = -0.0;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            float* x = xk[KEEP ? i : 0];
            xval(cur[i], x);                                        // zeros past the row end
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double d = (double)x[e];
                const double d2 = d * d;                            // exact
                const double q = __builtin_floor(d2 * 256.0);       // exact
                s1 += d;
                sq += q;
                sr += __builtin_fma(-q, 0x1p-8, d2);                // exact
            }
        }
        if constexpr (KEEP) load(m + nwv, cur);                     // next row, in flight from here
        s1 = wave_sum_exact(s1);
        sq = wave_sum_exact(sq);
        sr = wave_sum_exact(sr);
        Sums t;
        t.s1 = (int64_t)(s1 * 0x1p24);
        {
            const uint64_t Q = (uint64_t)sq, R = (uint64_t)(sr * 0x1p48);   // exact integers below 2^53
            t.lo = (Q << 40) + R;
            t.hi = (Q >> 24) + (t.lo < R ? 1u : 0u);
        }
        float mu, rs;
        row_stats(t, K, eps, mu, rs);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            float xt[8];
            float* x = xk[KEEP ? i : 0];
            if constexpr (!KEEP) {
                xval(cur[i], xt);
                x = xt;
            }
            float y[8];
            yval(x, c, mu, rs, y);
            float a = __builtin_fmaxf(__builtin_fabsf(y[0]), __builtin_fabsf(y[1]));
#pragma unroll
            for (int e = 2; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(y[e]));
            amax = c < nchunk ? __builtin_fmaxf(amax, a) : amax;
            if constexpr (KEEP) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = y[e];            // y replaces x
            }
        }
        amax = wave_max(amax);
        const float xs = amax / 127.0f;
        if (lane == 0 && m < M) scale[m] = xs;
        const bool zero = xs == 0.0f;
        const double rx = zero ? 0.0 : rcp64((double)xs);
        const __amdgpu_buffer_rsrc_t rq = row_rsrc(Xq + m * K, m, (int)K);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            float yt[8];
            const float* y = xk[KEEP ? i : 0];
            if constexpr (!KEEP) {
                float xt[8];
                xval(cur[i], xt);
                yval(xt, c, mu, rs, yt);
                y = yt;
            }
            float q[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) q[e] = (float)((double)y[e] * rx);   // = fl32(y / xs)
            uint32_t lo = pack_codes(q[0], q[1], q[2], q[3]);
            uint32_t hi = pack_codes(q[4], q[5], q[6], q[7]);
            if (zero) lo = hi = 0;
            __builtin_amdgcn_raw_buffer_store_b64(v2u{lo, hi}, rq, 8 * c, 0, 0);
        }
        if constexpr (!KEEP) load(m + nwv, cur);
        m += nwv;
    } while (m < M);
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

template <int CPL, bool BETA>
hipError_t launch_wave(const uint16_t* X, int64_t M, int64_t K, const float* gamma, const float* beta, float eps,
                       int8_t* Xq, float* scale, hipStream_t st) {
    constexpr int kWaves = 4;                                          // rows in flight per block
    const int64_t blocks = (M + kWaves - 1) / kWaves;
    const int64_t cap = (int64_t)dev_info().cus * 8;
    const size_t lds = (size_t)(64 * kWaves) * ((CPL + 1) / 2) * sizeof(v4f) * (BETA ? 2 : 1);   // >= 4K (or 8K) B
    SQ_LAUNCH((ln_quant_wave<CPL, BETA>), dim3((unsigned)(blocks < cap ? blocks : cap)),
                       dim3(64 * kWaves), lds, st, X, M, K, gamma, beta, eps, Xq, scale);
    return hipSuccess;
}

template <bool BETA>
hipError_t launch_ln(const uint16_t* X, int64_t M, int64_t K, const float* gamma, const float* beta, float eps,
                     int8_t* Xq, float* scale, hipStream_t st) {
    // few rows: spread each row over a group of threads (up to 1024) instead of one wave
    if (K <= 8192 && M < 4 * (int64_t)dev_info().cus)
        return launch_rows<1, BETA>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 512) return launch_wave<1, BETA>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 1024) return launch_wave<2, BETA>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 2048) return launch_wave<4, BETA>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 4096) return launch_wave<8, BETA>(X, M, K, gamma, beta, eps, Xq, scale, st);
    if (K <= 8192) return launch_wave<16, BETA>(X, M, K, gamma, beta, eps, Xq, scale, st);
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
