// Decode (skinny-M, M <= 16) int8 GEMM + dequant for gfx950.
//
// At M <= 16 the layer streams the N x K int8 weight bytes once and reuses each
// of them at most 16 times, so it is bound by HBM bandwidth, not by the matrix
// cores ["量化基础与INT8", INT8推理流程: int32 accumulation, then
// acc * x_scale * w_scale].  Two things decide the bandwidth on MI355X: the
// shape of each wave-wide load (HBM streams best when one load instruction
// covers few rows with long contiguous runs; the 16-row x 64-byte operand shape
// of v_mfma_i32_16x16x64_i8 reads measurably slower than 4 rows x 256 bytes),
// and the order in which the chip walks the matrix (a compact front of rows in
// flight beats every block streaming its own far-apart rows).
//
// Load shape.  With RPI rows per load (4 or 8), lane l reads 16 bytes of weight
// row l % RPI at k0 + 16 * (l / RPI): one instruction covers RPI rows x
// 1024 / RPI contiguous bytes.  The activation fragment uses the same pattern
// with tokens in place of rows.  Fed as the A (activations) and B (weights)
// operands of v_mfma_i32_16x16x64_i8, output (t, c) pairs A lanes 16g + t with
// B lanes 16g + c; both hold the same k bytes exactly when t / RPI == c / RPI,
// so those outputs are partial dot products of token t % RPI with row c % RPI
// over the 16-byte chunks {(t / RPI) + (16 / RPI) * g}.  Summing them over the
// 16 / RPI diagonal blocks gives the full product over the span; the other
// outputs are ignored.  The matrix cores do 4x (RPI 4) or 2x (RPI 8) the
// arithmetic of a dense layout, which they have to spare at this M.
//
// Work split.  A block of 8 waves owns tiles of TROWS = RG * RPI weight rows;
// wave w owns a contiguous slice of every row's k range, so its activation
// fragments are the same for every tile and stay in registers when they fit
// (HOIST), else they are reloaded per k chunk (from L2).  Blocks are persistent
// and take tiles b, b + gridDim.x, ... (b: the block's slot, blockIdx.x or, at M = 5..16,
// blockIdx.x permuted so that one XCD's blocks hold consecutive slots), so the rows in flight
// across the chip form a compact front.  Each wave loads the next tile (or
// chunk) before running the MFMAs of the current one; the 8 partial tiles are
// summed through LDS and the dequant epilogue stores Y (and acc).
//
// FP8 E4M3 variant (FP8 = true): the same loads and tiles; each MFMA,
// v_mfma_f32_16x16x128_f8f6f4, takes two consecutive steps' 16-byte chunks of a
// lane concatenated (a zero chunk past an odd step count).  A and B lanes hold
// the same k bytes in the same operand positions exactly where they do for the
// int8 instruction, so the diagonal blocks are again the partial products; the
// partial sums are fp32 and are added in a fixed order.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "sq_internal.h"

namespace sq {

namespace {

constexpr int kWaves = 8;

// Row groups per tile and persistent blocks per CU, measured on 70B-class decode shapes: for M <= 4
// with the activations held in registers (A) or reloaded per k chunk (AC), for M <= 8 (B, two
// token groups of 4) and for M <= 16 (C, four token groups of 4).
#ifndef SQ_GV_A_RG
#define SQ_GV_A_RG 1
#endif
#ifndef SQ_GV_A_PCU
#define SQ_GV_A_PCU 3
#endif
#ifndef SQ_GV_AC_RG
#define SQ_GV_AC_RG 2
#endif
#ifndef SQ_GV_AC_PCU
#define SQ_GV_AC_PCU 2
#endif
#ifndef SQ_GV_B_RG
#define SQ_GV_B_RG 1
#endif
#ifndef SQ_GV_B_PCU
#define SQ_GV_B_PCU 1
#endif
#ifndef SQ_GV_C_PCU
#define SQ_GV_C_PCU 1
#endif

// Inputs of the fused decode layer (FUSED kernels only): the fp16 activations, the
// smoothing factors (or null) and an optional output for the per-token scales.
struct FusedIn {
    const _Float16* X;
    const float* s;
    float* xs_out;
};

__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int RPI, int TG, int RG, int PER, bool HOIST, bool OUT_F16, bool FP8, int FUSED>
__global__ __launch_bounds__(64 * kWaves) void gemv_i8_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ xs, const int8_t* __restrict__ Wq,
    const float* __restrict__ ws, int ws_stride, const float* __restrict__ bias, int M, int N, int K,
    void* __restrict__ Yv, int32_t* __restrict__ acc_out, FusedIn fin, AsymArgs asy) {
    static_assert(!FUSED || (HOIST && TG == 1 && RPI == 4 && !FP8), "fused decode: M <= 2, register-resident X");
    constexpr int SPAN = 1024 / RPI;      // bytes of one row per load instruction
    constexpr int TROWS = RG * RPI;       // weight rows per tile
    constexpr int NB = 16 / RPI;          // diagonal blocks of one MFMA output
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lrow = lane % RPI, lchunk = lane / RPI;

    // This wave's k steps (SPAN bytes each): [s_begin, s_end), in chunks of PER.
    const int S = (K + SPAN - 1) / SPAN;
    const int per = (S + kWaves - 1) / kWaves;
    const int s_begin = wave * per;
    const int s_end = min(S, s_begin + per);
    const int nch = HOIST ? 1 : (per + PER - 1) / PER;
    const int ntiles = (N + TROWS - 1) / TROWS;
    // Block slot.  With two or four token groups (M = 5..16, one block per CU) and a grid of
    // whole XCD groups, the blocks of one XCD (blockIdx.x % 8, dealt round-robin) take
    // consecutive tiles of every round, so the 8-byte output runs of adjacent 4-row tiles meet
    // in that XCD's L2 and leave it as whole lines (4x fewer HBM write bytes; 70B FFN-up rows
    // back to back: M = 16 39.4-39.7 vs 40.6-41.2 us, M = 8 36.7-36.8 vs 37.1-37.6 us).  M <= 4,
    // with three blocks per CU, measured slower with it (M = 1: 38.2 vs 35.9 us) and keeps
    // blockIdx.x.
    const int nbk = (int)gridDim.x;
    const int slot = (TG >= 2 && nbk % 8 == 0) ? (int)(blockIdx.x % 8) * (nbk / 8) + (int)(blockIdx.x / 8)
                                              : (int)blockIdx.x;
    const int my_tiles = slot < ntiles ? (ntiles - 1 - slot) / nbk + 1 : 0;
    const int nunits = my_tiles * nch;

    // Loads go through buffer resources (record counts pass through readfirstlane so that the
    // descriptors stay in scalar registers): an offset outside the resource's record range reads as zero
    // without touching memory.  So every unit issues a fixed number of loads (the compiler's wait counts
    // stay exact while the next unit is in flight), steps past this wave's slice or past K cost nothing,
    // and the rows past N in the last tile read as zeros (their outputs are not stored).
    constexpr uint32_t kOut = 0x80000000u;   // beyond every record count used here (< 2^31)
    auto kpos = [&](int ch, int s) -> int {  // this lane's byte column at step s of chunk ch, or -1
        const int step = s_begin + ch * PER + s;
        const int k = step * SPAN + 16 * lchunk;
        return (step < s_end && k < K) ? k : -1;
    };
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(Xq), (short)0, __builtin_amdgcn_readfirstlane(M * K), 0x00020000);
    struct Buf {
        v4i w[RG][PER];
        v4i x[PER][TG];
        float wsv, bv;
        int rsv;
    };
    extern __shared__ __attribute__((aligned(16))) int8_t sxq[];   // FUSED: the block's copy of Xq [M x K]
    auto load_x = [&](int ch, v4i (&x)[PER][TG]) {
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int k = kpos(ch, s);
#pragma unroll
            for (int tg = 0; tg < TG; ++tg) {
                const int m = tg * RPI + lrow;
                if constexpr (FUSED) {
                    x[s][tg] = (k >= 0 && m < M) ? *reinterpret_cast<const v4i*>(sxq + m * K + k) : v4i{0, 0, 0, 0};
                } else {
                    const uint32_t off = (k >= 0 && m < M) ? (uint32_t)(m * K + k) : kOut;
                    x[s][tg] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
                }
            }
        }
    };
    // Fused decode: every block quantizes the (one or two) activation rows itself, exactly as
    // the per-token quantizer does (x' = fl32(x / s_j) by the fp64 reciprocal product,
    // xs = fl32(max |x'| / 127), codes of fl32(x' / xs)), into LDS.  Thread t owns the
    // 16 columns [16t, 16t + 16) of every row (K <= 8192); the row maxima meet in LDS.
    __shared__ float sred[kWaves][4];
    __shared__ float sxs[4];
    // The loads of X and s are issued first, then the first weight unit's, so the
    // prologue's arithmetic overlaps the weight latency.
    constexpr int MR = FUSED > 0 ? FUSED : 1;   // rows (tokens) of the fused layer
    const int c0 = (int)threadIdx.x * 16;
    const bool fact = FUSED > 0 && c0 < K;
    h8 fxv[MR][2];
    v4f fsv[4];
    auto fused_load = [&]() {
        if (!fact) return;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const h8* src = reinterpret_cast<const h8*>(fin.X + (int64_t)m * K + c0);
            fxv[m][0] = src[0];
            fxv[m][1] = src[1];
        }
        if (fin.s != nullptr)
#pragma unroll
            for (int q = 0; q < 4; ++q) fsv[q] = reinterpret_cast<const v4f*>(fin.s + c0)[q];
    };
    auto fused_compute = [&]() {
        static_assert(FUSED <= 4, "at most 4 fused rows");
        float xp[MR][16];
        if (fact) {
            // the smoothing division: the fp64 reciprocal product, with the IEEE division only
            // where a quotient could leave the normal range (some s_j >= 2^100)
            if (fin.s != nullptr) {
                bool guard = false;
#pragma unroll
                for (int e = 0; e < 16; ++e) guard = guard || !(fsv[e >> 2][e & 3] < 0x1p100f);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float sj = fsv[e >> 2][e & 3];
                    const double r = rcp64((double)sj);
#pragma unroll
                    for (int m = 0; m < MR; ++m) {
                        const float x = (float)fxv[m][e >> 3][e & 7];
                        xp[m][e] = guard ? div_rcp64(x, r, sj) : (float)((double)x * r);
                    }
                }
            } else {
#pragma unroll
                for (int m = 0; m < MR; ++m)
#pragma unroll
                    for (int e = 0; e < 16; ++e) xp[m][e] = (float)fxv[m][e >> 3][e & 7];
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            float mx = 0.0f;
            if (fact)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = __builtin_fmaxf(mx, __builtin_fabsf(xp[m][e]));
            mx = wave_max(mx);
            if (lane == 0) sred[wave][m] = mx;
        }
        lds_barrier();
        if ((int)threadIdx.x < MR) {
            float a = sred[0][threadIdx.x];
            for (int w = 1; w < kWaves; ++w) a = __builtin_fmaxf(a, sred[w][threadIdx.x]);
            const float x_s = a / 127.0f;
            sxs[threadIdx.x] = x_s;
            if (fin.xs_out != nullptr && blockIdx.x == 0) fin.xs_out[threadIdx.x] = x_s;
        }
        lds_barrier();
        if (fact) {
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float x_s = sxs[m];
                const double rx = x_s != 0.0f ? rcp64((double)x_s) : 0.0;
                uint32_t w[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    uint32_t v = 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int code = x_s == 0.0f ? 0 : code_of((float)((double)xp[m][4 * q + e] * rx));
                        v |= (uint32_t)(code & 0xff) << (8 * e);
                    }
                    w[q] = v;
                }
                *reinterpret_cast<v4i*>(sxq + m * K + c0) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            }
        }
        lds_barrier();
    };
    const bool eact = (int)threadIdx.x < M * TROWS;
    const int em = eact ? (int)threadIdx.x / TROWS : 0, ej = (int)threadIdx.x % TROWS;
    float xsv = FUSED ? 0.0f : xs[em];   // FUSED: set after the prologue
    // zero-point activations: acc - zq[m] * rowsum[n] (0 * 0 otherwise)
    const int xzv = (!FP8 && asy.xz != nullptr) ? asy.xz[em] : 0;
    const float* bsrc = bias != nullptr ? bias : ws;
    auto load_unit = [&](int unit, Buf& b) {
        const int tile = slot + (unit / nch) * nbk;
        const int ch = unit % nch;
        if (!HOIST) load_x(ch, b.x);
        const int rows = max(0, min(TROWS, N - tile * TROWS));   // 0 past the last tile
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<int8_t*>(Wq + (int64_t)tile * TROWS * K), (short)0,
            __builtin_amdgcn_readfirstlane(rows * K), 0x00020000);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int s = 0; s < PER; ++s) {
                const int k = kpos(ch, s);
                const uint32_t off = k >= 0 ? (uint32_t)((rg * RPI + lrow) * K + k) : kOut;
                b.w[rg][s] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2));
            }
        const int n = min(tile * TROWS + ej, N - 1);
        b.wsv = ws[(int64_t)n * ws_stride];
        b.bv = bsrc[bias != nullptr ? n : 0];
        b.rsv = (!FP8 && asy.wrs != nullptr) ? asy.wrs[n] : 0;
    };

    using AccV = typename std::conditional<FP8, v4f, v4i>::type;
    __shared__ AccV part[2][kWaves][RG][TG][64];
    AccV acc[RG][TG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int tg = 0; tg < TG; ++tg) acc[rg][tg] = AccV{};

    // One unit: MFMAs over a chunk, then (last chunk of a tile) the cross-wave sum and epilogue.
    auto cat = [](const v4i& lo, const v4i& hi) { return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]}; };
    auto run_unit = [&](int unit, const Buf& b, const v4i (&x)[PER][TG]) {
        if constexpr (FP8) {
#pragma unroll
            for (int s = 0; s < PER; s += 2)
#pragma unroll
                for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                    for (int tg = 0; tg < TG; ++tg) {
                        const v4i z{0, 0, 0, 0};
                        const v8i xa = cat(x[s][tg], s + 1 < PER ? x[s + 1][tg] : z);
                        const v8i wb = cat(b.w[rg][s], s + 1 < PER ? b.w[rg][s + 1] : z);
                        acc[rg][tg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(xa, wb, acc[rg][tg], 0, 0, 0, 0,
                                                                                       0, 0);
                    }
        } else {
#pragma unroll
            for (int s = 0; s < PER; ++s)
#pragma unroll
                for (int rg = 0; rg < RG; ++rg)
#pragma unroll
                    for (int tg = 0; tg < TG; ++tg)
                        acc[rg][tg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(x[s][tg], b.w[rg][s], acc[rg][tg], 0, 0, 0);
        }
        const int ti = unit / nch;
        if (unit % nch != nch - 1) return;
        const int par = ti & 1;
        // MFMA output lane l, register r = D[4 * (l / 16) + r][l % 16]; stored as [c][t] (16 B per lane).
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int tg = 0; tg < TG; ++tg) {
                part[par][wave][rg][tg][(lane & 15) * 4 + (lane >> 4)] = acc[rg][tg];
                acc[rg][tg] = AccV{};
            }
        // The other parity's buffer is only rewritten after every wave has passed the next barrier,
        // i.e. after every reader of this tile's buffer has finished with it.
        lds_barrier();
        const int n = (slot + ti * nbk) * TROWS + ej;
        if (eact && n < N) {
            const int rg = ej / RPI, jj = ej % RPI, tg = em / RPI, mm = em % RPI;
            using Elt = typename std::conditional<FP8, float, int>::type;
            const Elt* pb = reinterpret_cast<const Elt*>(&part[par][0][rg][tg][0]);
            Elt sum = 0;
#pragma unroll
            for (int w8 = 0; w8 < kWaves; ++w8)
#pragma unroll
                for (int bk = 0; bk < NB; ++bk) sum += pb[w8 * (RG * TG * 256) + (bk * RPI + jj) * 16 + bk * RPI + mm];
            if constexpr (!FP8) sum -= xzv * b.rsv;
            float y = (float)sum;
            y = y * xsv;
            y = y * b.wsv;
            if (bias != nullptr) y = y + b.bv;
            if constexpr (OUT_F16) reinterpret_cast<_Float16*>(Yv)[(int64_t)em * N + n] = (_Float16)y;
            else reinterpret_cast<float*>(Yv)[(int64_t)em * N + n] = y;
            if (acc_out != nullptr) acc_out[(int64_t)em * N + n] = __builtin_bit_cast(int32_t, sum);
        }
    };

    Buf ba, bb;
    if constexpr (FUSED) {
        fused_load();
        if (nunits > 0) load_unit(0, ba);
        fused_compute();
        xsv = sxs[em];
        load_x(0, ba.x);
    } else {
        if (HOIST) load_x(0, ba.x);
        if (nunits > 0) load_unit(0, ba);
    }
    // Drain the prologue loads so that the waits inside the loop count only the loads in flight there.
    __builtin_amdgcn_s_waitcnt(0x0070);
    // Ping-pong between two buffers.  The next unit is always loaded, also past the end (every load of
    // a tile past the last one is out of range and touches no memory), so both halves are straight-line
    // code and each MFMA waits only for its own operands.
    int u = 0;
    while (u < nunits) {
        load_unit(u + 1, bb);
        run_unit(u, ba, ba.x);
        if (++u >= nunits) break;
        load_unit(u + 1, ba);
        run_unit(u, bb, HOIST ? ba.x : bb.x);
        ++u;
    }
}

template <int RPI, int TG, int RG, int PER, bool HOIST, bool FP8, int FUSED = 0>
hipError_t launch_cfg(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
                      const float* bias, int M, int N, int K, void* Y, int ydt, int32_t* acc_out, int grid,
                      hipStream_t st, FusedIn fin = FusedIn{nullptr, nullptr, nullptr}, AsymArgs asy = AsymArgs{}) {
    const size_t dyn = FUSED ? (size_t)FUSED * K : 0;   // the block's Xq copy
    if (ydt == SQ_F16)
        SQ_LAUNCH((gemv_i8_kernel<RPI, TG, RG, PER, HOIST, true, FP8, FUSED>), dim3(grid), dim3(64 * kWaves),
                           dyn, st, Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, acc_out, fin, asy);
    else
        SQ_LAUNCH((gemv_i8_kernel<RPI, TG, RG, PER, HOIST, false, FP8, FUSED>), dim3(grid),
                           dim3(64 * kWaves), dyn, st, Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, acc_out, fin,
                           asy);
    return hipSuccess;
}


template <bool FP8>
hipError_t gemv_dispatch(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
                         const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int ydt, int32_t* acc_out,
                         hipStream_t st, AsymArgs asy = AsymArgs{}) {
    const int cus = dev_info().cus;
    const int m = (int)M, n = (int)N, k = (int)K;
    // Steps per wave for a load span of `span` bytes; the register-resident chunk is the next power of two.
    auto per_of = [&](int span) { return ((k + span - 1) / span + kWaves - 1) / kWaves; };
    auto grid_of = [&](int trows, int per_cu) {
        const int64_t tiles = (N + trows - 1) / trows;
        return (int)(tiles < (int64_t)per_cu * cus ? tiles : (int64_t)per_cu * cus);
    };
#define SQ_GEMV(RPI, TG, RG, PER, HOIST, PER_CU) \
    launch_cfg<RPI, TG, RG, PER, HOIST, FP8>(Xq, xs, Wq, ws, ws_stride, bias, m, n, k, Y, ydt, acc_out, \
                                        grid_of(RG * RPI, PER_CU), st, FusedIn{nullptr, nullptr, nullptr}, asy)
    if (M <= 4) {
        // 4 rows x 256 bytes per load, one token group.
        const int per = per_of(256);
        if (per <= 1) return SQ_GEMV(4, 1, SQ_GV_A_RG, 1, true, SQ_GV_A_PCU);
        if (per <= 2) return SQ_GEMV(4, 1, SQ_GV_A_RG, 2, true, SQ_GV_A_PCU);
        if (per <= 4) return SQ_GEMV(4, 1, SQ_GV_A_RG, 4, true, SQ_GV_A_PCU);
        if (per <= 8) return SQ_GEMV(4, 1, SQ_GV_A_RG, 8, true, SQ_GV_A_PCU);
        return SQ_GEMV(4, 1, SQ_GV_AC_RG, 8, false, SQ_GV_AC_PCU);
    }
    if (M <= 8) {
        // 4 rows x 256 bytes per load, two token groups of 4 (measured 6-7% faster on the 70B
        // FFN-up rows at M = 8 than 8 rows x 128 bytes with one group of 8).
        const int per = per_of(256);
        if (per <= 1) return SQ_GEMV(4, 2, SQ_GV_B_RG, 1, true, SQ_GV_B_PCU);
        if (per <= 2) return SQ_GEMV(4, 2, SQ_GV_B_RG, 2, true, SQ_GV_B_PCU);
        if (per <= 4) return SQ_GEMV(4, 2, SQ_GV_B_RG, 4, true, SQ_GV_B_PCU);
        if (per <= 8) return SQ_GEMV(4, 2, SQ_GV_B_RG, 8, true, SQ_GV_B_PCU);
        return SQ_GEMV(4, 2, SQ_GV_B_RG, 8, false, SQ_GV_B_PCU);
    }
    // 4 rows x 256 bytes per load, four token groups of 4, activations in registers (on the 70B
    // FFN-up rows at M = 16: 39.9 us back to back against 41.2 us with 8 rows x 128 bytes and two
    // groups of 8); longer rows reload the activations per chunk with 8 rows x 128 bytes.
    if (per_of(256) <= 8) {
        const int per = per_of(256);
        if (per <= 1) return SQ_GEMV(4, 4, 1, 1, true, SQ_GV_C_PCU);
        if (per <= 2) return SQ_GEMV(4, 4, 1, 2, true, SQ_GV_C_PCU);
        if (per <= 4) return SQ_GEMV(4, 4, 1, 4, true, SQ_GV_C_PCU);
        return SQ_GEMV(4, 4, 1, 8, true, SQ_GV_C_PCU);
    }
    return SQ_GEMV(8, 2, 2, 4, false, SQ_GV_C_PCU);
#undef SQ_GEMV
}

}  // namespace

hipError_t launch_gemv(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
                       const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int ydt, int32_t* acc_out,
                       const SideArgs* side, hipStream_t st) {
    (void)side;
    return gemv_dispatch<false>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ydt, acc_out, st);
}

hipError_t launch_gemv_asym(const int8_t* Xq, const float* xs, const int32_t* xz, const int8_t* Wq, const float* ws,
                            int ws_stride, const int32_t* wrs, const float* bias, int64_t M, int64_t N, int64_t K,
                            void* Y, int ydt, int32_t* acc_out, hipStream_t st) {
    return gemv_dispatch<false>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ydt, acc_out, st, AsymArgs{xz, wrs});
}

namespace {
template <int PER, bool OUT_F16, int MR>
int fused_blocks_per_cu() {
    static std::atomic<int> cached{0};
    int nb = cached.load(std::memory_order_relaxed);
    if (nb == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &nb, gemv_i8_kernel<4, 1, SQ_GV_A_RG, PER, true, OUT_F16, false, MR>, 64 * kWaves, MR * 8192) !=
                hipSuccess ||
            nb <= 0)
            nb = 1;
        nb = nb < SQ_GV_A_PCU ? nb : SQ_GV_A_PCU;
        cached.store(nb, std::memory_order_relaxed);
    }
    return nb;
}
}  // namespace

// Fused decode layer, M <= 2, K <= 8192, fp16 X: quantization in every block's prologue
// (measured on the 70B FFN-up rows: M = 1 38.2 vs 40.7 us for quantizer + decode kernel,
// M = 2 39.3 vs 40.4; from M = 3 the prologue costs what the separate launch saves).
hipError_t launch_linear_decode(const _Float16* X, const float* s, const int8_t* Wq, const float* ws, int ws_stride,
                                const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int ydt,
                                float* x_scale, hipStream_t st) {
    const int cus = dev_info().cus;
    const int m = (int)M, n = (int)N, k = (int)K;
    const FusedIn fin{X, s, x_scale};
    const int per = ((k + 255) / 256 + kWaves - 1) / kWaves;
    const int64_t tiles = (N + SQ_GV_A_RG * 4 - 1) / (SQ_GV_A_RG * 4);
    // Persistent blocks: as many per CU as are resident at once (the prologue's registers
    // can lower it below the unfused kernel's count; the LDS copy of Xq, at most 32 KB,
    // never does).  Queried once per kernel.
#define SQ_FUSED(PER, MR)                                                                                        \
    launch_cfg<4, 1, SQ_GV_A_RG, PER, true, false, MR>(                                                          \
        nullptr, nullptr, Wq, ws, ws_stride, bias, m, n, k, Y, ydt, nullptr,                                     \
        (int)std::min<int64_t>(tiles, (int64_t)cus * (ydt == SQ_F16 ? fused_blocks_per_cu<PER, true, MR>()      \
                                                                    : fused_blocks_per_cu<PER, false, MR>())),   \
        st, fin)
    if (per <= 1) return m == 1 ? SQ_FUSED(1, 1) : SQ_FUSED(1, 2);
    if (per <= 2) return m == 1 ? SQ_FUSED(2, 1) : SQ_FUSED(2, 2);
    return m == 1 ? SQ_FUSED(4, 1) : SQ_FUSED(4, 2);
#undef SQ_FUSED
}

hipError_t launch_gemv_fp8(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws, int ws_stride,
                           const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int ydt, float* acc_out,
                           hipStream_t st) {
    return gemv_dispatch<true>(reinterpret_cast<const int8_t*>(Xq), xs, reinterpret_cast<const int8_t*>(Wq), ws,
                               ws_stride, bias, M, N, K, Y, ydt, reinterpret_cast<int32_t*>(acc_out), st);
}

}  // namespace sq
