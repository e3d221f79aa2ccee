// int8 x int8 -> int32 GEMM with the dequantizing epilogue fused in registers,
// for gfx950 (CDNA4) ["量化基础与INT8", INT8推理流程 / 量化流程示例: int32
// accumulation then acc * x_scale * w_scale; "SmoothQuant量化实战", section 3.4].
//
// Layout: Xq [M x K] and Wq [N x K] row-major int8, both K-contiguous ("NT"),
// Y [M x N].  A 256-thread block (4 waves in a 2 x 2 grid) computes a BM x BN
// tile with v_mfma_i32_32x32x32_i8; K is walked in BK = 128-byte tiles staged in
// LDS, double buffered (global -> registers for tile k+1 while tile k feeds the
// MFMAs).  LDS rows are 128 bytes; the 16-byte chunk c of row r sits at slot
// c ^ (r & 7), so the fragment reads (lane -> row lane%32, chunk lane/32) of a
// wave hit distinct banks.
//
// MFMA operand use: lane l supplies 16 k-consecutive bytes of A row (l % 32) and
// of B row (l % 32), k-chunk (l / 32); A and B use the same k placement, so any
// internal pairing of k slots the instruction applies is the same on both sides
// and the dot product is exact.  Result lane l, register r holds
// D[8*(r/4) + 4*(l/32) + r%4][l % 32].
//
// LLM.int8() ["LLM.int8()技术解析", section 3.1]: when a side product is
// requested, the dequantized tile becomes the C input of
// v_mfma_f32_32x32x16_f16 over the gathered fp16 outlier columns, so the fp16
// result adds onto the int8 result inside the same kernel.
#include "sq_internal.h"

namespace sq {

namespace {

constexpr int kThreads = 256;

template <int BM, int BN, bool OUT_F16, bool SIDE>
__global__ __launch_bounds__(kThreads, 1) void gemm_i8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ xs, const int8_t* __restrict__ B,
    const float* __restrict__ ws, int ws_stride, const float* __restrict__ bias, int M, int N, int K,
    void* __restrict__ Yv, int32_t* __restrict__ acc_out, const _Float16* __restrict__ Xo,
    const _Float16* __restrict__ Wo, const int32_t* __restrict__ cnt, int64_t ldo, int tiles_m, int tiles_n) {
    constexpr int BK = 128;
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    constexpr int KCH = BK / 16;
    constexpr int A_CH = BM * KCH / kThreads;
    constexpr int B_CH = BN * KCH / kThreads;
    constexpr int STAGE = (BM + BN) * BK;
    __shared__ __attribute__((aligned(16))) int8_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 1, wn = wave & 1;

    // Tile order: blocks are dealt to the 8 XCDs round-robin; give each XCD a
    // contiguous range of logical tiles, ordered in groups of 8 tile-rows so the
    // tiles that run together on one XCD share A and B panels in its L2.
    const int T = tiles_m * tiles_n;
    int t;
    {
        const int b = blockIdx.x;
        const int q = T / 8, r = T % 8, x = b % 8, loc = b / 8;
        t = x < r ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
    }
    constexpr int GROUP = 8;
    const int per_group = GROUP * tiles_n;
    const int first_m = (t / per_group) * GROUP;
    const int gsz = tiles_m - first_m < GROUP ? tiles_m - first_m : GROUP;
    const int tm = first_m + (t % per_group) % gsz;
    const int tn = (t % per_group) / gsz;
    const int m0 = tm * BM, n0 = tn * BN;

    // global -> register staging
    v4i ra[A_CH], rb[B_CH];
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int id = tid + i * kThreads;
            const int row = id / KCH, kc = id % KCH;
            const int gr = m0 + row, gk = k0 + kc * 16;
            if (gr < M && gk < K) ra[i] = *reinterpret_cast<const v4i*>(A + (int64_t)gr * K + gk);
            else ra[i] = v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int id = tid + i * kThreads;
            const int row = id / KCH, kc = id % KCH;
            const int gr = n0 + row, gk = k0 + kc * 16;
            if (gr < N && gk < K) rb[i] = *reinterpret_cast<const v4i*>(B + (int64_t)gr * K + gk);
            else rb[i] = v4i{0, 0, 0, 0};
        }
    };
    auto lstore = [&](int buf) {
        int8_t* base = lds + buf * STAGE;
#pragma unroll
        for (int i = 0; i < A_CH; ++i) {
            const int id = tid + i * kThreads;
            const int row = id / KCH, kc = id % KCH;
            *reinterpret_cast<v4i*>(base + row * BK + ((kc ^ (row & 7)) << 4)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_CH; ++i) {
            const int id = tid + i * kThreads;
            const int row = id / KCH, kc = id % KCH;
            *reinterpret_cast<v4i*>(base + BM * BK + row * BK + ((kc ^ (row & 7)) << 4)) = rb[i];
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    const int lrow = lane & 31, lk = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const int8_t* As = lds + buf * STAGE;
        const int8_t* Bs = As + BM * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int kc = ks * 2 + lk;
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WTM + i * 32 + lrow;
                af[i] = *reinterpret_cast<const v4i*>(As + row * BK + ((kc ^ (row & 7)) << 4));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WTN + j * 32 + lrow;
                bf[j] = *reinterpret_cast<const v4i*>(Bs + row * BK + ((kc ^ (row & 7)) << 4));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue, one 32 x 32 tile at a time (keeps register pressure at the
    // accumulators): y = ((float)acc * xs[m]) * ws[n] (+ bias[n]) [+ fp16 side]
    const int rbase = m0 + wm * WTM + 4 * lk;   // + i*32 + 8*(r/4) + r%4
    const int cbase = n0 + wn * WTN + lrow;     // + j*32
    const int side_cnt = SIDE ? *cnt : 0;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = cbase + j * 32;
            const bool cok = col < N;
            const float wsv = cok ? ws[(int64_t)col * ws_stride] : 0.0f;
            const float bv = (bias != nullptr && cok) ? bias[col] : 0.0f;
            v16f y;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
                const float xsv = row < M ? xs[row] : 0.0f;
                float v = (float)acc[i][j][r];
                v = v * xsv;
                v = v * wsv;
                if (bias != nullptr) v = v + bv;
                y[r] = v;
            }
            if (acc_out != nullptr && cok) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
                    if (row < M) acc_out[(int64_t)row * N + col] = acc[i][j][r];
                }
            }
            if constexpr (SIDE) {
                const int arow = m0 + wm * WTM + i * 32 + lrow;
                const int bcol = n0 + wn * WTN + j * 32 + lrow;
                for (int t0 = 0; t0 < side_cnt; t0 += 16) {
                    const int tk = t0 + 8 * lk;   // this lane's 8 k-slots
                    h8 xa{}, wb{};
                    if (arow < M) {
                        const _Float16* p = Xo + (int64_t)arow * ldo + tk;
                        if (tk + 8 <= side_cnt) xa = *reinterpret_cast<const h8*>(p);
                        else
                            for (int e = 0; e < 8; ++e) xa[e] = tk + e < side_cnt ? p[e] : (_Float16)0.0f;
                    }
                    if (bcol < N) {
                        const _Float16* p = Wo + (int64_t)bcol * ldo + tk;
                        if (tk + 8 <= side_cnt) wb = *reinterpret_cast<const h8*>(p);
                        else
                            for (int e = 0; e < 8; ++e) wb[e] = tk + e < side_cnt ? p[e] : (_Float16)0.0f;
                    }
                    y = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa, wb, y, 0, 0, 0);
                }
            }
            if (!cok) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
                if (row >= M) continue;
                if constexpr (OUT_F16)
                    reinterpret_cast<_Float16*>(Yv)[(int64_t)row * N + col] = (_Float16)y[r];
                else
                    reinterpret_cast<float*>(Yv)[(int64_t)row * N + col] = y[r];
            }
        }
    }
}

template <int BM, int BN, bool OUT_F16, bool SIDE>
hipError_t run(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
               const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int32_t* acc_out, const SideArgs* side,
               hipStream_t st) {
    const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
    const _Float16* Xo = side ? side->Xo : nullptr;
    const _Float16* Wo = side ? side->Wo : nullptr;
    const int32_t* cnt = side ? side->count : nullptr;
    const int64_t ldo = side ? side->ldo : 0;
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, OUT_F16, SIDE>), dim3((unsigned)(tm * tn)), dim3(kThreads), 0, st,
                       Xq, xs, Wq, ws, ws_stride, bias, (int)M, (int)N, (int)K, Y, acc_out, Xo, Wo, cnt, ldo, tm, tn);
    return hipGetLastError();
}

template <int BM, int BN>
hipError_t dispatch(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
                    const float* bias, int64_t M, int64_t N, int64_t K, void* Y, sq_dtype ydt, int32_t* acc_out,
                    const SideArgs* side, hipStream_t st) {
    if (ydt == SQ_F16) {
        if (side) return run<BM, BN, true, true>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, acc_out, side, st);
        return run<BM, BN, true, false>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, acc_out, side, st);
    }
    if (side) return run<BM, BN, false, true>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, acc_out, side, st);
    return run<BM, BN, false, false>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, acc_out, side, st);
}

}  // namespace

hipError_t launch_gemm(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
                       const float* bias, int64_t M, int64_t N, int64_t K, void* Y, sq_dtype ydt, int32_t* acc_out,
                       const SideArgs* side, hipStream_t st) {
    // Large problems: 256 x 256 tiles; otherwise 128 x 128 to keep more blocks.
    const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (big_tiles >= (int64_t)dev_info().cus)
        return dispatch<256, 256>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ydt, acc_out, side, st);
    return dispatch<128, 128>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ydt, acc_out, side, st);
}

}  // namespace sq
