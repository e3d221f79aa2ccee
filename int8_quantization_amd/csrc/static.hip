// Static per-tensor activation scale from calibration data, and quantization
// with it ["量化基础与INT8", 静态量化: activation ranges precomputed on a
// calibration set; the deployment page's calibrator takes a percentile (99.99) of
// the activation distribution].
//
// Calibration: T = the nearest-rank p-th percentile of |x'| over all M*K
// calibration values (x' = fl32(x / s_j), or x), i.e. the value at 1-based rank
// r = ceil(p*n/100) in ascending order; scale = fl32(T / 127).  Non-negative
// floats order like their bit patterns, so T is found exactly by a radix select
// on the bits: three histogram passes over bits 30..20, 19..9 and 8..0 (bit 31 is
// the sign, always 0), each followed by a one-block scan that picks the bucket
// holding rank r and narrows the rank.  Everything stays on the device.
//
// Forward: q = clamp(rne(fl32(x' / scale)), -128, 127) with the one calibrated
// scale, so there is no per-row reduction: a thread owns a 16-byte column chunk
// (its fp64 reciprocals of s computed once) and walks down the rows; short rows
// are packed several to a block.  X is read once: non-temporal loads (measured
// 10-15% faster on HBM-sized inputs).
#include <type_traits>

#include "sq_internal.h"

namespace sq {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerThread = 16;

template <typename T> struct Chunk16;
template <> struct Chunk16<_Float16> {
    using V = h8;
    static constexpr int N = 8;
};
template <> struct Chunk16<float> {
    using V = v4f;
    static constexpr int N = 4;
};

// Selection state between the passes (device memory).
struct SelState {
    uint32_t prefix;   // bits of T fixed so far
    uint32_t rank;     // 1-based rank of T among the values sharing that prefix
};

// Per-thread column constants: the exact smoothing divide x / s_j, as the fp64
// reciprocal product.  A quotient can fall below the fp32 normal range (where the
// IEEE division itself is taken) only for fp32 inputs or some s_j >= 2^100: a
// nonzero binary16 x is at least 2^-24.  `guard` marks such threads.
template <typename T, bool SMOOTH>
struct Cols {
    static constexpr int N = Chunk16<T>::N;
    double rs[SMOOTH ? N : 1];
    float sv[SMOOTH ? N : 1];
    bool guard = false;
    __device__ void init(const float* s, int64_t c) {
        if constexpr (SMOOTH) {
#pragma unroll
            for (int e = 0; e < N; ++e) {
                sv[e] = s[c * N + e];
                rs[e] = rcp64((double)sv[e]);
                guard = guard || !(sv[e] < 0x1p100f);
            }
            if constexpr (sizeof(T) == 4) guard = true;
        }
    }
    template <bool G>
    __device__ float apply(float x, int e) const {
        if constexpr (!SMOOTH) return x;
        else if constexpr (G) return div_rcp64(x, rs[e], sv[e]);
        else return (float)((double)x * rs[e]);
    }
};

// Column j uses the scale xs_in[j / group] (group = K: one scale; group = D: one per
// attention head of a [T x H*D] KV block); a 16-byte chunk never straddles a group.
template <typename T, bool SMOOTH>
__global__ __launch_bounds__(kThreads) void static_quant_kernel(const T* __restrict__ X, int64_t M, int64_t K,
                                                                const float* __restrict__ s,
                                                                const float* __restrict__ xs_in, int64_t group,
                                                                int8_t* __restrict__ Xq,
                                                                float* __restrict__ xs_rows, int lgp) {
    using V = typename Chunk16<T>::V;
    constexpr int N = Chunk16<T>::N;
    const int64_t nchunk = K / N;
    const int64_t c = ((int64_t)blockIdx.x << lgp) + (threadIdx.x & ((1u << lgp) - 1));
    if (xs_rows != nullptr && blockIdx.x == 0 && threadIdx.x == 0)
        for (int64_t m = blockIdx.y; m < M; m += gridDim.y) xs_rows[m] = xs_in[0];
    if (c >= nchunk) return;
    const float xs = xs_in[(c * N) / group];
    const double rx = xs != 0.0f ? rcp64((double)xs) : 0.0;
    Cols<T, SMOOTH> cols;
    cols.init(s, c);
    // rows in batches of RB: the batch's loads are all in flight before its codes are
    // formed (two rows when the smoothing divide lengthens the per-row work; one
    // otherwise, measured best on HBM-sized inputs)
    constexpr int RB = SMOOTH ? 2 : 1;
    const int64_t R = kThreads >> lgp;
    const int64_t step = gridDim.y * R;
    const int64_t first = blockIdx.y * R + (threadIdx.x >> lgp);
    auto rows = [&](auto guarded) {
        for (int64_t m0 = first; m0 < M; m0 += RB * step) {
            V v[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t m = m0 + r * step;
                v[r] = m < M ? __builtin_nontemporal_load(reinterpret_cast<const V*>(X + m * K) + c) : V{};
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t m = m0 + r * step;
                int q[N];
#pragma unroll
                for (int e = 0; e < N; ++e) {
                    const float x = cols.template apply<decltype(guarded)::value>((float)v[r][e], e);
                    // a quotient below the fp32 normal range codes to 0 either way
                    q[e] = xs == 0.0f ? 0 : code_of((float)((double)x * rx));
                }
                uint32_t w[N / 4];
#pragma unroll
                for (int k = 0; k < N / 4; ++k)
                    w[k] = (uint32_t)(q[4 * k] & 0xff) | ((uint32_t)(q[4 * k + 1] & 0xff) << 8) |
                           ((uint32_t)(q[4 * k + 2] & 0xff) << 16) | ((uint32_t)(q[4 * k + 3] & 0xff) << 24);
                if (m < M) {
                    if constexpr (N == 8) *reinterpret_cast<uint2*>(Xq + m * K + c * N) = make_uint2(w[0], w[1]);
                    else *reinterpret_cast<uint32_t*>(Xq + m * K + c * N) = w[0];
                }
            }
        }
    };
    if (cols.guard) rows(std::true_type{});
    else rows(std::false_type{});
}

// Pass PASS of the radix select: histogram of one bit field of |x'| over the values
// whose higher bits equal the prefix fixed so far.
template <int PASS> struct Field;
template <> struct Field<0> { static constexpr int lo = 20, bits = 11; };
template <> struct Field<1> { static constexpr int lo = 9, bits = 11; };
template <> struct Field<2> { static constexpr int lo = 0, bits = 9; };

template <typename T, bool SMOOTH, int PASS>
__global__ __launch_bounds__(kThreads) void hist_kernel(const T* __restrict__ X, int64_t M, int64_t K,
                                                        const float* __restrict__ s,
                                                        const SelState* __restrict__ state,
                                                        uint32_t* __restrict__ hist) {
    using V = typename Chunk16<T>::V;
    constexpr int N = Chunk16<T>::N;
    constexpr int NB = 1 << Field<PASS>::bits;
    constexpr int LO = Field<PASS>::lo;
    constexpr int HI = LO + Field<PASS>::bits;          // bits at and above HI are fixed
    __shared__ uint32_t lh[NB];
    for (int b = threadIdx.x; b < NB; b += kThreads) lh[b] = 0;
    __syncthreads();
    const uint32_t want = PASS == 0 ? 0u : (state->prefix >> HI);
    const int64_t nchunk = K / N;
    const int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (c < nchunk) {
        Cols<T, SMOOTH> cols;
        cols.init(s, c);
        for (int64_t m = blockIdx.y; m < M; m += gridDim.y) {
            const V v = reinterpret_cast<const V*>(X + m * K)[c];
#pragma unroll
            for (int e = 0; e < N; ++e) {
                const uint32_t bits =
                    __builtin_bit_cast(uint32_t, __builtin_fabsf(cols.template apply<true>((float)v[e], e)));
                if ((bits >> HI) == want) atomicAdd(&lh[(bits >> LO) & (NB - 1)], 1u);
            }
        }
    }
    __syncthreads();
    for (int b = threadIdx.x; b < NB; b += kThreads)
        if (lh[b] != 0) atomicAdd(&hist[b], lh[b]);
}

// One block: find the bucket holding the current rank, fix its bits, narrow the
// rank, and clear the histogram for the next pass.
template <int PASS>
__global__ __launch_bounds__(1024) void select_kernel(uint32_t* __restrict__ hist, SelState* __restrict__ state) {
    constexpr int NB = 1 << Field<PASS>::bits;
    constexpr int PER = (NB + 1023) / 1024;             // buckets per thread (2 or 1)
    __shared__ uint32_t part[1024];
    const int t = threadIdx.x;
    const uint32_t rank = state->rank;
    uint32_t h[PER], own = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int b = t * PER + k;
        h[k] = b < NB ? hist[b] : 0u;
        own += h[k];
    }
    // inclusive scan of the per-thread totals (Hillis-Steele over 1024 entries)
    part[t] = own;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const uint32_t add = t >= off ? part[t - off] : 0u;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    uint32_t before = part[t] - own;                     // values in lower buckets
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int b = t * PER + k;
        if (b < NB && before < rank && rank <= before + h[k]) {
            state->prefix |= (uint32_t)b << Field<PASS>::lo;
            state->rank = rank - before;
        }
        before += h[k];
        if (b < NB) hist[b] = 0u;
    }
}

__global__ void select_init_kernel(uint32_t* __restrict__ hist, SelState* __restrict__ state, uint32_t rank) {
    for (int b = threadIdx.x; b < 2048; b += blockDim.x) hist[b] = 0u;
    if (threadIdx.x == 0) {
        state->prefix = 0u;
        state->rank = rank;
    }
}

__global__ void select_finish_kernel(const SelState* __restrict__ state, float* __restrict__ x_scale) {
    if (threadIdx.x == 0) x_scale[0] = __builtin_bit_cast(float, state->prefix) / 127.0f;
}

// Up to kRowsPerThread rows per thread, but at least ~64K threads when there are
// enough rows (few rows: one row per block row).
dim3 grid_of(int64_t M, int64_t K, int vec) {
    const int64_t nchunk = K / vec;
    const int64_t gx = (nchunk + kThreads - 1) / kThreads;
    int64_t gy = (M + kRowsPerThread - 1) / kRowsPerThread;
    const int64_t want = (65536 / kThreads + gx - 1) / gx;
    if (gy < want) gy = want < M ? want : M;
    if (gy > 65535) gy = 65535;
    return dim3((unsigned)gx, (unsigned)gy);
}

template <typename T, bool SMOOTH>
hipError_t calibrate_t(const T* X, int64_t M, int64_t K, const float* s, uint32_t rank, float* x_scale, void* ws,
                       hipStream_t st) {
    uint32_t* hist = static_cast<uint32_t*>(ws);
    SelState* state = reinterpret_cast<SelState*>(static_cast<char*>(ws) + kStaticHistBytes);
    const dim3 g = grid_of(M, K, Chunk16<T>::N);
    SQ_LAUNCH(select_init_kernel, dim3(1), dim3(256), 0, st, hist, state, rank);
    SQ_LAUNCH((hist_kernel<T, SMOOTH, 0>), g, dim3(kThreads), 0, st, X, M, K, s, state, hist);
    SQ_LAUNCH(select_kernel<0>, dim3(1), dim3(1024), 0, st, hist, state);
    SQ_LAUNCH((hist_kernel<T, SMOOTH, 1>), g, dim3(kThreads), 0, st, X, M, K, s, state, hist);
    SQ_LAUNCH(select_kernel<1>, dim3(1), dim3(1024), 0, st, hist, state);
    SQ_LAUNCH((hist_kernel<T, SMOOTH, 2>), g, dim3(kThreads), 0, st, X, M, K, s, state, hist);
    SQ_LAUNCH(select_kernel<2>, dim3(1), dim3(1024), 0, st, hist, state);
    SQ_LAUNCH(select_finish_kernel, dim3(1), dim3(64), 0, st, state, x_scale);
    return hipSuccess;
}

template <typename T, bool SMOOTH>
hipError_t quant_t(const T* X, int64_t M, int64_t K, const float* s, const float* xs, int64_t group, int8_t* Xq,
                   float* xs_rows, hipStream_t st) {
    const RowPack g = row_pack(M, K / Chunk16<T>::N, 8, 1024);
    SQ_LAUNCH((static_quant_kernel<T, SMOOTH>), g.grid, dim3(kThreads), 0, st, X, M, K, s, xs, group, Xq,
                       xs_rows, g.lgp);
    return hipSuccess;
}

}  // namespace

hipError_t launch_static_calibrate(const void* X, int dt, int64_t M, int64_t K, const float* s, uint32_t rank,
                                   float* x_scale, void* ws, hipStream_t st) {
    if (dt == SQ_F16) {
        if (s) return calibrate_t<_Float16, true>((const _Float16*)X, M, K, s, rank, x_scale, ws, st);
        return calibrate_t<_Float16, false>((const _Float16*)X, M, K, s, rank, x_scale, ws, st);
    }
    if (s) return calibrate_t<float, true>((const float*)X, M, K, s, rank, x_scale, ws, st);
    return calibrate_t<float, false>((const float*)X, M, K, s, rank, x_scale, ws, st);
}

hipError_t launch_static_quant(const void* X, int dt, int64_t M, int64_t K, const float* s, const float* xs,
                               int64_t group, int8_t* Xq, float* xs_rows, hipStream_t st) {
    if (dt == SQ_F16) {
        if (s) return quant_t<_Float16, true>((const _Float16*)X, M, K, s, xs, group, Xq, xs_rows, st);
        return quant_t<_Float16, false>((const _Float16*)X, M, K, s, xs, group, Xq, xs_rows, st);
    }
    if (s) return quant_t<float, true>((const float*)X, M, K, s, xs, group, Xq, xs_rows, st);
    return quant_t<float, false>((const float*)X, M, K, s, xs, group, Xq, xs_rows, st);
}

}  // namespace sq
