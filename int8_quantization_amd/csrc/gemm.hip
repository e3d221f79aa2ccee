// int8 x int8 -> int32 GEMM with the dequantizing epilogue fused in registers,
// for gfx950 (CDNA4) ["量化基础与INT8", INT8推理流程 / 量化流程示例: int32
// accumulation then acc * x_scale * w_scale; "SmoothQuant量化实战", section 3.4].
//
// Layout: Xq [M x K] and Wq [N x K] row-major int8, both K-contiguous ("NT"),
// Y [M x N].  A block of 8 waves (WM x WN grid, two waves per SIMD) computes a
// BM x BN tile with v_mfma_i32_32x32x32_i8.  K is walked in BK = 128-byte
// tiles (one cache line per row) held in two LDS stages: while the MFMAs read
// stage j, buffer_load ... lds (LDS DMA, 1 KB = 8 rows x 128 B per wave
// instruction) fills stage j+1 straight from global memory, with no register
// staging.  In the 256-column tiles a stage is refilled as soon as the barrier
// that ends the reads of its previous tile has passed (that tile's last k-step
// is then in registers), one or two DMA instructions after each MFMA of that
// last k-step, so the loads have four k-steps to land and their issue hides
// behind the MFMAs.  LDS rows are 128 bytes; the 16-byte chunk c of row r sits at slot
// c ^ ((r >> SWZ) & 7), so the fragment reads (lane -> row lane%32, chunk
// lane/32) of a wave hit distinct banks.  A K that is not a multiple of 128
// starts with one partial tile staged through registers with zero fill.
// The DMA is issued from inline asm: the compiler models the builtin form as an
// LDS store of unknown address and then waits for it before every later LDS
// read, which would serialize the prefetch with the fragment reads; here the
// pipeline's own waits and barriers order it.
// Blocks are dealt to the 8 XCDs round-robin; the tile order gives each XCD a
// contiguous range of tiles, grouped 8 tile-rows deep, so that concurrently
// running tiles share operand panels in that XCD's L2.
// A tile count that would leave a partial last round of large tiles is split by
// output columns: the full rounds cover the leading tile columns and the rest
// goes out as a second launch with its own (smaller) tiles.
//
// MFMA operand use: lane l supplies 16 k-consecutive bytes of a weight row
// (l % 32) as the instruction's A operand and of an activation row (l % 32) as
// its B operand, k-chunk (l / 32); both use the same k placement, so any
// internal pairing of k slots the instruction applies is the same on both sides
// and the dot product is exact.  Result lane l, register r holds
// D[8*(r/4) + 4*(l/32) + r%4][l % 32] = (output column, output row), so each
// lane owns runs of four consecutive output columns.
//
// Epilogue: the accumulators are dequantized per (row, column) in the order
// int32 -> fp32, * x_scale[row], * w_scale[col], + bias[col], converted to the
// output type and written to LDS, then copied out with 16-byte row-contiguous
// stores.
//
// FP8 E4M3 variant (FP8 = true; "SmoothQuant量化实战", section 6.1, W8A8 in FP8
// on hardware with FP8 matrix units): the same tiles, staging and epilogue with
// v_mfma_f32_32x32x64_f8f6f4 and fp32 accumulators.  That instruction takes 32
// bytes per lane; a lane concatenates the two 16-byte chunks it reads for two
// consecutive int8 k-steps, so both operands keep one k placement and the LDS
// reads are the int8 kernel's (conflict-free) pattern.
//
// LLM.int8() ["LLM.int8()技术解析", section 3.1]: when a side product is
// requested, the dequantized tile becomes the C input of
// v_mfma_f32_32x32x16_f16 over the fp16 outlier columns (activations from a
// gathered panel, weights read at the outlier columns of the fp16 weight's
// rows), so the fp16 result adds onto the int8 result inside the same kernel.
#include <algorithm>
#include <type_traits>

#include "sq_internal.h"

namespace sq {

namespace {

// Wave grids of the two large tile shapes (waves = WM x WN, 2 waves per SIMD at 8).
#ifndef SQ_W256_WM
#define SQ_W256_WM 2
#define SQ_W256_WN 4
#endif
#ifndef SQ_W192_WM
#define SQ_W192_WM 4
#define SQ_W192_WN 2
#endif

// LDS slot swizzle: 16-byte chunk c of tile row r is stored at slot c ^ ((r >> SWZ) & 7).
#ifndef SQ_GEMM_SWZ
#define SQ_GEMM_SWZ 1
#endif

// Waits and barriers.  __syncthreads() would also make the compiler wait for
// every outstanding load before the barrier; these helpers wait for exactly
// what the pipeline needs, with the s_waitcnt builtin (which the compiler's
// own wait tracking sees), and the empty asm statements keep LDS accesses from
// being moved across them.
__device__ __forceinline__ void wait_all_loads() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
}
// All but the last N vector-memory operations (loads complete in issue order) and
// every LDS access.
template <int N>
__device__ __forceinline__ void wait_loads_but() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);   // vmcnt(N) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0), vm/exp counts unconstrained
    asm volatile("" ::: "memory");
}
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int BM, int BN, int WM, int WN, bool OUT_F16, bool SIDE, bool FP8, bool ASYM>
__global__ __launch_bounds__(64 * WM * WN, 1) void gemm_i8_kernel(
    const int8_t* __restrict__ A, const float* __restrict__ xs, const int8_t* __restrict__ B,
    const float* __restrict__ ws, int ws_stride, const float* __restrict__ bias, int M, int N, int K,
    void* __restrict__ Yv, int32_t* __restrict__ acc_out, const _Float16* __restrict__ Xo,
    const _Float16* __restrict__ W16, const int32_t* __restrict__ sidx, const int32_t* __restrict__ cnt, int64_t ldo,
    int64_t ldy, int tiles_m, int tiles_n, const int32_t* __restrict__ xz, const int32_t* __restrict__ wrs) {
    constexpr int BK = 128;                  // bytes of K per stage: one cache line per row
    constexpr int S = 2;                     // LDS stages
    constexpr int KS = BK / (FP8 ? 64 : 32); // MFMA k-steps per stage
    using Frag = typename std::conditional<FP8, v8i, v4i>::type;
    using Acc = typename std::conditional<FP8, v16f, v16i>::type;
    static_assert(!(FP8 && SIDE), "the LLM.int8() side product is int8 only");
    static_assert(!ASYM || (!FP8 && !SIDE), "zero-point activations: plain int8 products only");
    constexpr int NW = WM * WN;              // waves, in a WM x WN grid over the tile
    constexpr int NT = 64 * NW;              // threads
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / 32, TN = WTN / 32;
    static_assert(TM * 32 == WTM && TN * 32 == WTN, "wave tile must be a multiple of 32");
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int NBLK = (BM + BN) / 8;      // 1 KB DMA blocks (8 rows) per stage
    constexpr int L = NBLK / NW;             // DMA instructions per wave per stage
    static_assert(NBLK % NW == 0, "stage must split evenly over the waves");
    __shared__ __attribute__((aligned(1024))) int8_t lds[S * STAGE];

    const int tid = threadIdx.x;
    const int side_cnt = SIDE ? *cnt : 0;   // LLM.int8() outlier columns (count on the device)
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // wave index is uniform
    const int wm = wave / WN, wn = wave % WN;

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

    // LDS layout of a stage: A rows [0, BM) then B rows, 128 bytes each; the
    // 16-byte chunk c of row r sits at slot c ^ swz(r).
    auto swz = [](int r) { return (r >> SQ_GEMM_SWZ) & 7; };

    // DMA addressing: wave w fills 1 KB blocks w, w+NW, ...; lane l writes row
    // (block*8 + l/8), slot l%8, so it fetches logical chunk (l%8) ^ swz(row).
    // The loads go through buffer resources over the tile's A and B rows: each
    // lane's byte offset inside them is fixed, the K position travels in the
    // scalar offset (no per-tile vector address arithmetic in the MFMA waves),
    // and rows past M (N) are outside the record range and read as zeros (they
    // only feed outputs that are never stored).
    const v4i rA = buffer_desc(A + (int64_t)m0 * K, (M - m0 < BM ? M - m0 : BM) * K);
    const v4i rB = buffer_desc(B + (int64_t)n0 * K, (N - n0 < BN ? N - n0 : BN) * K);
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds;
    uint32_t voff[L];
    int ldsoff[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
        const int blk = wave + NW * i;
        const bool isA = blk < BM / 8;
        const int row = (isA ? blk : blk - BM / 8) * 8 + (lane >> 3);
        const int kc = (lane & 7) ^ swz(row);
        voff[i] = (uint32_t)(row * K + kc * 16);
        ldsoff[i] = blk * 1024;
    }
    // Materialized here, so that the prologue's loads do not share registers with them (a
    // register still feeding an earlier load is rewritten only after that load completes).
#pragma unroll
    for (int i = 0; i < L; ++i) asm volatile("" ::"v"(voff[i]));
    auto dma = [&](int stage, int k0) {
#pragma unroll
        for (int i = 0; i < L; ++i)
            dma_to_lds(wave + NW * i < BM / 8 ? rA : rB,
                       __builtin_amdgcn_readfirstlane(lds_base + stage * STAGE + ldsoff[i]), voff[i], k0);
    };
    // Partial K tile (K % 128 != 0): through registers with zero fill.
    auto tail_tile = [&](int stage, int k0) {
        const int kc = tid & 7, r0 = tid >> 3;    // chunk tid%8 of rows tid/8 + (NT/8) i
#pragma unroll
        for (int i = 0; i < (BM + BN) / (NT / 8); ++i) {
            const int rr = r0 + (NT / 8) * i;
            const bool isA = rr < BM;
            const int row = isA ? rr : rr - BM;
            int g = (isA ? m0 : n0) + row;
            const int lim = isA ? M : N;
            g = g < lim ? g : lim - 1;
            const int8_t* p = (isA ? A : B) + (int64_t)g * K + k0 + kc * 16;
            const v4i v = (k0 + kc * 16 < K) ? *reinterpret_cast<const v4i*>(p) : v4i{0, 0, 0, 0};
            *reinterpret_cast<v4i*>(lds + stage * STAGE + rr * BK + ((kc ^ swz(row)) << 4)) = v;
        }
    };

    Acc acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = Acc{};

    const int lrow = lane & 31, lk = lane >> 5;
    Frag af[2][TM], bf[2][TN];
    // fragment of k-step ks for one LDS row: chunk 2ks + lane/32 (int8); chunks
    // 4ks + lane/32 and 4ks + 2 + lane/32, concatenated (FP8)
    auto frag = [&](const int8_t* rowp, int row, int ks) -> Frag {
        if constexpr (FP8) {
            const v4i lo = *reinterpret_cast<const v4i*>(rowp + (((4 * ks + lk) ^ swz(row)) << 4));
            const v4i hi = *reinterpret_cast<const v4i*>(rowp + (((4 * ks + 2 + lk) ^ swz(row)) << 4));
            return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
            return *reinterpret_cast<const v4i*>(rowp + (((2 * ks + lk) ^ swz(row)) << 4));
        }
    };
    auto fload = [&](int stage, int ks, int slot) {
        const int8_t* As = lds + stage * STAGE;
        const int8_t* Bs = As + BM * BK;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WTM + i * 32 + lrow;
            af[slot][i] = frag(As + row * BK, row, ks);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * WTN + j * 32 + lrow;
            bf[slot][j] = frag(Bs + row * BK, row, ks);
        }
    };
    auto mfmas = [&](int slot) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if constexpr (FP8)   // format 0 = E4M3 for both operands; no block scales
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[slot][j], af[slot][i], acc[i][j],
                                                                                0, 0, 0, 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[slot][j], af[slot][i], acc[i][j], 0, 0, 0);
            }
    };

    // Tile order: [partial tail], 0, 1, ..., nfull-1.  Tile j lives in stage j % 2.
    const int nfull = K / BK;
    const bool has_tail = (K % BK) != 0;
    const int nk = nfull + (has_tail ? 1 : 0);
    auto kofs = [&](int j) { return (has_tail ? (j == 0 ? nfull : j - 1) : j) * BK; };
    // LLM.int8() side operands: 8 consecutive outlier columns from tk on, zero past the count.
    // Activations come from the panel Xo [M x ldo]; weights straight from the fp16 weight's
    // rows, at the outlier columns col[e] = sidx[tk + e].
    auto side_frag = [&](const _Float16* p, bool ok, int tk) {
        h8 v{};
        if (ok) {
            if (tk + 8 <= side_cnt) v = *reinterpret_cast<const h8*>(p + tk);
            else
                for (int e = 0; e < 8; ++e) v[e] = tk + e < side_cnt ? p[tk + e] : (_Float16)0.0f;
        }
        return v;
    };
    auto wside_frag = [&](const _Float16* row, bool ok, const int* col, int tk) {
        h8 v{};
        if (ok)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = tk + e < side_cnt ? row[col[e]] : (_Float16)0.0f;
        return v;
    };
    // The tile's side operands for the first 16 outlier columns are read in the prologue, so
    // that their latency (scattered 2-byte reads of the fp16 weight) overlaps the first K
    // tile's, and kept in LDS for the epilogue: thread t holds 8 columns (8 (t % 2) on) of
    // tile row t / 2 and of tile column t / 2.
    static_assert(!SIDE || (2 * BM <= NT && 2 * BN <= NT), "one side chunk per thread");
    __shared__ __attribute__((aligned(16))) _Float16 sxo[SIDE ? BM : 1][16], swo[SIDE ? BN : 1][16];
    const int so_r = tid >> 1, so_c = 8 * (tid & 1);
    // With panel rows and an outlier list of at least 16 entries (the usual case) the loads are
    // issued unconditionally, in one batch, and the values past the count (or of rows past M,
    // N) are zeroed when they are stored; columns past the count read column 0 of the weight
    // row and the panel's unused columns.  Otherwise guarded per-element loads.
    const bool side_fast = SIDE && ldo >= 16 && K >= 16;
    h8 xo_v{}, wo_v{};
    const int so_row = m0 + (so_r < BM ? so_r : 0), so_col = n0 + (so_r < BN ? so_r : 0);
    const bool xo_ok = SIDE && so_r < BM && so_row < M, wo_ok = SIDE && so_r < BN && so_col < N;
    const _Float16* xo_p = SIDE ? Xo + (int64_t)(so_row < M ? so_row : 0) * ldo : nullptr;
    const _Float16* wo_p = SIDE ? W16 + (int64_t)(so_col < N ? so_col : 0) * K : nullptr;
    _Float16 wo_r[8];
    // The first K tile's DMA goes out first.
    if (has_tail) tail_tile(0, kofs(0));
    else dma(0, kofs(0));
    if constexpr (SIDE) {
        if (side_fast) {
            // The outlier list through scalar loads (uniform addresses; they wait on their own
            // counter, not behind the DMA), then the weight columns and the panel row.
            int cl[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) cl[e] = __builtin_amdgcn_readfirstlane(sidx[e]);
            const int hmask = -(tid & 1);   // all ones for the upper 8 columns
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = cl[e] ^ ((cl[e] ^ cl[8 + e]) & hmask);   // a select, kept out of array indexing
                wo_r[e] = wo_p[so_c + e < side_cnt ? c : 0];
            }
            xo_v = *reinterpret_cast<const h8*>(xo_p + so_c);
        }
    }
    // Dequantization scales of the tile's rows and columns: thread t loads row t's and
    // column t's, all in one batch with the loads above, so that the prologue waits once for
    // everything; the prologue barrier publishes them.
    static_assert(BM <= NT && BN <= NT, "one row and one column scale per thread");
    float xs_v = 0.0f, ws_v = 0.0f, b_v = -0.0f;   // x + (-0.0) == x for every x: no bias
    int xz_v = 0, rs_v = 0;                         // zero-point activations: zero point, weight row sum
    if (tid < BM) {
        xs_v = xs[m0 + tid < M ? m0 + tid : M - 1];
        if constexpr (ASYM) xz_v = xz[m0 + tid < M ? m0 + tid : M - 1];
    }
    if (tid < BN) {
        const int n = n0 + tid < N ? n0 + tid : N - 1;
        ws_v = ws[(int64_t)n * ws_stride];
        if (bias != nullptr) b_v = bias[n];
        if constexpr (ASYM) rs_v = wrs[n];
    }
    __shared__ float sxs[BM], sws[BN], sbias[BN];
    __shared__ int szq[ASYM ? BM : 1], srs[ASYM ? BN : 1];
    if (tid < BM) sxs[tid] = xs_v;
    if (tid < BN) {
        sws[tid] = ws_v;
        sbias[tid] = b_v;
    }
    if constexpr (ASYM) {
        if (tid < BM) szq[tid] = xz_v;
        if (tid < BN) srs[tid] = rs_v;
    }
    if constexpr (SIDE) {
        if (side_fast) {   // zero the values past the count and of rows past M, N
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool live = so_c + e < side_cnt;
                xo_v[e] = xo_ok && live ? xo_v[e] : (_Float16)0.0f;
                wo_v[e] = wo_ok && live ? wo_r[e] : (_Float16)0.0f;
            }
            if (so_r < BM) *reinterpret_cast<h8*>(&sxo[so_r][so_c]) = xo_v;
            if (so_r < BN) *reinterpret_cast<h8*>(&swo[so_r][so_c]) = wo_v;
        } else {   // guarded per-element loads, last, so that no other code waits behind them
            if (xo_ok) xo_v = side_frag(xo_p, side_cnt > 0, so_c);
            if (wo_ok) {
                int col[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) col[e] = so_c + e < side_cnt ? sidx[so_c + e] : 0;
                wo_v = wside_frag(wo_p, side_cnt > 0, col, so_c);
            }
            if (so_r < BM) *reinterpret_cast<h8*>(&sxo[so_r][so_c]) = xo_v;
            if (so_r < BN) *reinterpret_cast<h8*>(&swo[so_r][so_c]) = wo_v;
        }
    }
    // The epilogue's kernel arguments go to registers now: scalar loads still in
    // flight when the loop starts would make the compiler's fragment waits in it
    // conservative (it cannot order them against the LDS reads).
    asm volatile("" ::"s"(Yv), "s"(acc_out), "s"(ws_stride));
    // The 256-column tiles keep two K tiles in flight: the second one's DMA goes out here,
    // and the wait leaves exactly those L loads (the youngest) outstanding.
    constexpr bool EARLY = BN == 256;
    if (EARLY && nk > 1) {
        dma(1, kofs(1));
        wait_loads_but<L>();
    } else {
        wait_all_loads();
    }
    block_barrier();
    fload(0, 0, 0);

    // Scheduling fence between k-steps (fragment reads, then the MFMAs of the step
    // before): measured faster for the 256-column tile, while the compiler's own
    // interleaving is faster for the others.
    auto fence = [] {
        if constexpr (BN == 256) __builtin_amdgcn_sched_barrier(0);
    };
    auto steps = [&](int st) {   // k-steps 0 .. KS-2 of the tile in stage st
#pragma unroll
        for (int ks = 0; ks + 1 < KS; ++ks) {
            fload(st, ks + 1, (ks + 1) & 1);
            fence();
            mfmas(ks & 1);
            fence();
        }
    };
    // One fragment (q < TM: A fragment q, else B fragment q - TM), one MFMA, one DMA
    // instruction: the pieces of the hand-interleaved k-step below.
    auto frag_one = [&](int stage, int ks, int slot, int q) {
        const int8_t* As = lds + stage * STAGE;
        const int8_t* Bs = As + BM * BK;
        if (q < TM) {
            const int row = wm * WTM + q * 32 + lrow;
            af[slot][q] = frag(As + row * BK, row, ks);
        } else {
            const int row = wn * WTN + (q - TM) * 32 + lrow;
            bf[slot][q - TM] = frag(Bs + row * BK, row, ks);
        }
    };
    auto mfma_one = [&](int slot, int i, int jj) {
        if constexpr (FP8)
            acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[slot][jj], af[slot][i], acc[i][jj], 0, 0, 0,
                                                                         0, 0, 0);
        else
            acc[i][jj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[slot][jj], af[slot][i], acc[i][jj], 0, 0, 0);
    };
    auto dma_one = [&](int stage, int k0, int i) {
        dma_to_lds(wave + NW * i < BM / 8 ? rA : rB, __builtin_amdgcn_readfirstlane(lds_base + stage * STAGE + ldsoff[i]),
                   voff[i], k0);
    };
    if constexpr (EARLY) {
        // Tile j+1 was issued one barrier earlier (or in the prologue).  Every tile but the
        // last ends in the barrier; the last runs after the loop.
        for (int j = 0; j + 1 < nk; ++j) {
            const int st = j & 1;
            steps(st);
            // tile j+1 landed for every wave, and tile j's last fragments are in registers
            wait_all_loads();
            block_barrier();
            // so stage st is free: tile j+2 goes into it (after the last tile, the last tile's
            // bytes again, into a stage nothing reads any more), spread over the MFMAs of tile
            // j's last k-step after the first fragment reads of tile j+1.  The scheduling
            // barriers keep this order.
            const int k2 = __builtin_amdgcn_readfirstlane(j + 2 < nk ? kofs(j + 2) : kofs(j));
            constexpr int NM = TM * TN, NQ = TM + TN;
            static_assert(NM > NQ, "MFMAs left for the DMA instructions");
            constexpr int PER = (L + NM - NQ - 1) / (NM - NQ);
            int d = 0;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                __builtin_amdgcn_sched_barrier(0);
                mfma_one((KS - 1) & 1, m / TN, m % TN);
                __builtin_amdgcn_sched_barrier(0);
                if (m < NQ) {
                    frag_one(st ^ 1, 0, 0, m);
                } else {
#pragma unroll
                    for (int e = 0; e < PER; ++e)
                        if (d < L) dma_one(st, k2, d++);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    } else
    // Every tile but the last prefetches its successor and ends in the barrier;
    // the last runs after the loop, so the loop body has a single shape.
    for (int j = 0; j + 1 < nk; ++j) {
        const int st = j & 1;
        // the other stage held tile j-1, which every wave finished reading before
        // the previous barrier
        dma(st ^ 1, kofs(j + 1));
        fence();
        steps(st);
        // tile j+1 landed for every wave, and tile j's last fragments are in registers
        wait_all_loads();
        block_barrier();
        fload(st ^ 1, 0, 0);
        fence();
        mfmas((KS - 1) & 1);
        fence();
    }
    steps((nk - 1) & 1);
    mfmas((KS - 1) & 1);

    // ---- epilogue, staged through LDS.
    // With the weight fragment as the instruction's A operand, lane l, register
    // 4a+b of tile (i, j) holds output row  wm*WTM + i*32 + l%32  and column
    // wn*WTN + j*32 + 8a + 4(l/32) + b  (runs of four consecutive columns).
    //   y = ((float)acc * xs[m]) * ws[n] (+ bias[n])   [+ fp16 side product]
    // Each wave writes its y values, already in the output dtype, into an LDS
    // copy of the block tile (16-byte chunks XOR-swizzled by row); the block then
    // writes the tile out with 16-byte stores, row by row.  fp32 output goes in
    // two halves of the tile rows (the LDS ring holds half a 256 x 256 fp32 tile).
    constexpr int OB = OUT_F16 ? 2 : 4;                  // output bytes
    constexpr int HALVES = OUT_F16 ? 1 : 2;
    constexpr int TMH = TM / HALVES;                     // tiles per wave per half
    constexpr int HROWS = BM / HALVES;                   // tile rows per half
    constexpr int RB = BN * OB;                          // LDS bytes per tile row
    constexpr int CH16 = RB / 16;                        // 16-byte chunks per row
    static_assert(HROWS * RB <= S * STAGE, "epilogue tile must fit the LDS ring");
    constexpr int SWM = CH16 % 16 == 0 ? 15 : (CH16 % 8 == 0 ? 7 : (CH16 % 4 == 0 ? 3 : 0));   // XOR mask
    auto lofs = [&](int r, int cbyte) {                  // LDS byte offset of (row, byte in row)
        return r * RB + ((((cbyte >> 4) ^ (r & SWM))) << 4) + (cbyte & 15);
    };

    wait_all_loads();
    block_barrier();                                      // ring no longer read
    // LLM.int8() side operands of this wave's rows and columns for the first 16 outlier
    // columns, from the prologue's LDS copy (more than 16 columns load per chunk below).
    h8 xpre[SIDE ? TM : 1], wpre[SIDE ? TN : 1];
    if constexpr (SIDE) {
#pragma unroll
        for (int i = 0; i < TM; ++i) xpre[i] = *reinterpret_cast<const h8*>(&sxo[wm * WTM + i * 32 + lrow][8 * lk]);
#pragma unroll
        for (int j = 0; j < TN; ++j) wpre[j] = *reinterpret_cast<const h8*>(&swo[wn * WTN + j * 32 + lrow][8 * lk]);
    }

    // This lane's row and column scales for the whole epilogue, read from LDS in
    // one batch (one latency instead of one per accumulator group); the optional
    // bias is read where it is added.
    constexpr bool HOIST = true;
    float xsr[TM];
    v4f wsr[HOIST ? TN : 1][4];
#pragma unroll
    for (int i = 0; i < TM; ++i) xsr[i] = sxs[wm * WTM + i * 32 + lrow];
    if constexpr (HOIST) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                wsr[j][a] = *reinterpret_cast<const v4f*>(&sws[wn * WTN + j * 32 + 8 * a + 4 * lk]);
    }

    // int32 accumulators, when requested (parity checks): straight from the
    // accumulator registers, 16 bytes per lane per group of four columns
    if (acc_out != nullptr) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm * WTM + i * 32 + lrow;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int n = n0 + wn * WTN + j * 32 + 8 * a + 4 * lk;
                    int iv[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(iv[b]) : "a"(acc[i][j][4 * a + b]));
                    if constexpr (ASYM) {   // the corrected accumulator: acc - zq * rowsum (int32, wraps like int64 when it fits)
                        const int zq = szq[wm * WTM + i * 32 + lrow];
                        const v4i r4 = *reinterpret_cast<const v4i*>(&srs[wn * WTN + j * 32 + 8 * a + 4 * lk]);
#pragma unroll
                        for (int b = 0; b < 4; ++b) iv[b] -= zq * r4[b];
                    }
                    if (m < M)
                        for (int b = 0; b < 4; ++b)
                            if (n + b < N) acc_out[(int64_t)m * ldy + n + b] = iv[b];
                }
        }
    }

#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
        // write phase: branch-free per accumulator tile (the bias add is unconditional,
        // the int32 accumulator output has its own pass)
#pragma unroll
        for (int ii = 0; ii < TMH; ++ii) {
            const int i = h * TMH + ii;
            const int lr = wm * (TMH * 32) + ii * 32 + lrow;      // LDS row
            const int mloc = wm * WTM + i * 32 + lrow;           // tile row
            const float xsv = xsr[i];
            const int zq = ASYM ? szq[mloc] : 0;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                v16f y;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int nloc = wn * WTN + j * 32 + 8 * a + 4 * lk;
                    const v4f w4 = HOIST ? wsr[HOIST ? j : 0][a] : *reinterpret_cast<const v4f*>(&sws[nloc]);
                    const v4f b4 = *reinterpret_cast<const v4f*>(&sbias[nloc]);
                    v4i r4{};
                    if constexpr (ASYM) r4 = *reinterpret_cast<const v4i*>(&srs[nloc]);
                    int iv[4];
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        // read the accumulator register directly, one value at a time
                        asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(iv[b]) : "a"(acc[i][j][4 * a + b]));
                        if constexpr (ASYM) iv[b] -= zq * r4[b];
                        float v = FP8 ? __builtin_bit_cast(float, iv[b]) : (float)iv[b];
                        v = v * xsv;
                        v = v * w4[b];
                        v = v + b4[b];      // -0.0 without a bias: an exact identity
                        y[4 * a + b] = v;
                    }
                }
                if constexpr (SIDE) {
                    // fp16 side product over the gathered outlier columns, same operand roles
                    const int arow = m0 + mloc;
                    const int bcol = n0 + wn * WTN + j * 32 + lrow;
                    if (side_cnt > 0) y = __builtin_amdgcn_mfma_f32_32x32x16_f16(wpre[j], xpre[i], y, 0, 0, 0);
                    for (int t0 = 16; t0 < side_cnt; t0 += 16) {
                        const int tk = t0 + 8 * lk;   // this lane's 8 k-slots
                        int col[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) col[e] = tk + e < side_cnt ? sidx[tk + e] : 0;
                        const h8 xa = side_frag(Xo + (int64_t)(arow < M ? arow : 0) * ldo, arow < M, tk);
                        const h8 wb = wside_frag(W16 + (int64_t)(bcol < N ? bcol : 0) * K, bcol < N, col, tk);
                        y = __builtin_amdgcn_mfma_f32_32x32x16_f16(wb, xa, y, 0, 0, 0);
                    }
                }
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int cb = (wn * WTN + j * 32 + 8 * a + 4 * lk) * OB;
                    if constexpr (OUT_F16) {
                        // two round-to-nearest-even pair conversions (v_cvt_pk_f16_f32), stored as two dwords
                        typedef float f2 __attribute__((ext_vector_type(2)));
                        typedef _Float16 hf2 __attribute__((ext_vector_type(2)));
                        typedef uint32_t u2 __attribute__((ext_vector_type(2)));
                        const hf2 lo = __builtin_convertvector(f2{y[4 * a], y[4 * a + 1]}, hf2);
                        const hf2 hi = __builtin_convertvector(f2{y[4 * a + 2], y[4 * a + 3]}, hf2);
                        *reinterpret_cast<u2*>(lds + lofs(lr, cb)) =
                            u2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
                    } else {
                        *reinterpret_cast<v4f*>(lds + lofs(lr, cb)) = v4f{y[4 * a], y[4 * a + 1], y[4 * a + 2], y[4 * a + 3]};
                    }
                }
            }
        }
        wait_lds();
        block_barrier();
        // copy phase: 16-byte chunks, consecutive threads along a row; a thread
        // issues its LDS reads in batches of up to 8 before the batch's stores
        constexpr int NQ = HROWS * CH16 / NT;
        static_assert(NQ * NT == HROWS * CH16, "copy phase must split evenly over the threads");
        constexpr int QB = [] {   // largest divisor of NQ up to 8
            for (int d = 8; d > 1; --d)
                if (NQ % d == 0) return d;
            return 1;
        }();
        static_assert(NQ % QB == 0, "copy batches must split evenly");
        const bool vec = (ldy * OB) % 16 == 0;
#pragma unroll
        for (int k0 = 0; k0 < NQ; k0 += QB) {
            v4i cv[QB];
#pragma unroll
            for (int k = 0; k < QB; ++k) {
                const int q = tid + (k0 + k) * NT;
                cv[k] = *reinterpret_cast<const v4i*>(lds + lofs(q / CH16, (q % CH16) * 16));
            }
#pragma unroll
            for (int k = 0; k < QB; ++k) {
                const int q = tid + (k0 + k) * NT;
                const int lr = q / CH16, c = q % CH16;
                const int wmq = lr / (TMH * 32), rem = lr % (TMH * 32);
                const int m = m0 + wmq * WTM + (h * TMH + rem / 32) * 32 + rem % 32;
                if (m < M) {
                    const int n = n0 + c * (16 / OB);
                    char* dst = reinterpret_cast<char*>(Yv) + ((int64_t)m * ldy + n) * OB;
                    if (vec && n + 16 / OB <= N) {
                        *reinterpret_cast<v4i*>(dst) = cv[k];
                    } else {
                        // ragged edge or unaligned rows: element stores (constant indices keep
                        // the chunk in registers)
#pragma unroll
                        for (int e = 0; e < 16 / OB; ++e) {
                            if (n + e >= N) continue;
                            if constexpr (OB == 4)
                                reinterpret_cast<uint32_t*>(dst)[e] = (uint32_t)cv[k][e];
                            else
                                reinterpret_cast<uint16_t*>(dst)[e] = (uint16_t)((uint32_t)cv[k][e / 2] >> (16 * (e % 2)));
                        }
                    }
                }
            }
        }
        if (h + 1 < HALVES) {
            wait_lds();
            block_barrier();
        }
    }
}

template <int BM, int BN, int WM, int WN, bool OUT_F16, bool SIDE, bool FP8, bool ASYM = false>
hipError_t run(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
               const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int64_t ldy, int32_t* acc_out,
               const SideArgs* side, hipStream_t st, const AsymArgs* asym = nullptr) {
    const int tm = (int)((M + BM - 1) / BM), tn = (int)((N + BN - 1) / BN);
    const _Float16* Xo = side ? side->Xo : nullptr;
    const _Float16* W16 = side ? side->W16 : nullptr;
    const int32_t* sidx = side ? side->idx : nullptr;
    const int32_t* cnt = side ? side->count : nullptr;
    const int64_t ldo = side ? side->ldo : 0;
    const int32_t* xz = asym ? asym->xz : nullptr;
    const int32_t* wrs = asym ? asym->wrs : nullptr;
    SQ_LAUNCH((gemm_i8_kernel<BM, BN, WM, WN, OUT_F16, SIDE, FP8, ASYM>), dim3((unsigned)(tm * tn)),
                       dim3(64 * WM * WN), 0, st, Xq, xs, Wq, ws, ws_stride, bias, (int)M, (int)N, (int)K, Y, acc_out,
                       Xo, W16, sidx, cnt, ldo, ldy, tm, tn, xz, wrs);
    return hipSuccess;
}

template <int BM, int BN, int WM, int WN>
hipError_t dispatch(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
                    const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int64_t ldy, int ydt,
                    int32_t* acc_out, const SideArgs* side, bool fp8, hipStream_t st, const AsymArgs* asym) {
    if (asym) {   // zero-point activations: plain int8 products, fp16 or fp32 output
        if (fp8 || side) return hipErrorInvalidValue;
        if (ydt == SQ_F16)
            return run<BM, BN, WM, WN, true, false, false, true>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy,
                                                                 acc_out, nullptr, st, asym);
        return run<BM, BN, WM, WN, false, false, false, true>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy,
                                                              acc_out, nullptr, st, asym);
    }
    if (fp8) {
        if constexpr (BN == 256) {
            return hipErrorInvalidValue;   // the FP8 fragments do not fit beside 256 x 256 accumulators
        } else {
            if (side) return hipErrorInvalidValue;
            if (ydt == SQ_F16)
                return run<BM, BN, WM, WN, true, false, true>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy,
                                                              acc_out, side, st);
            return run<BM, BN, WM, WN, false, false, true>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy,
                                                           acc_out, side, st);
        }
    }
    if (ydt == SQ_F16) {
        if (side)
            return run<BM, BN, WM, WN, true, true, false>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy, acc_out,
                                                          side, st);
        return run<BM, BN, WM, WN, true, false, false>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy, acc_out,
                                                       side, st);
    }
    // The LLM.int8() side product comes with fp16 output only (int8_outlier_matmul writes fp16).
    if (side) return hipErrorInvalidValue;
    return run<BM, BN, WM, WN, false, false, false>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy, acc_out, side,
                                                    st);
}

// Output columns [0, N) of a product whose output rows are ldy elements apart.
// Tile shape: the least estimated time, rounds * (area per CU) / rate with
// rounds = ceil(tiles / tile slots); a 256-row tile takes a whole CU, 128 x 128
// tiles run two per CU at about three quarters of the per-CU rate (measured on
// the 530B-slice shape).  When large tiles would leave a partial last round, the
// full rounds take the leading tile columns and the remaining columns go out as
// a second launch that picks its own tiles, if that is estimated faster.
hipError_t launch_cols(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
                       const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int64_t ldy, int ydt,
                       int32_t* acc_out, const SideArgs* side, bool fp8, hipStream_t st, bool may_split,
                       const AsymArgs* asym = nullptr) {
    const int64_t cus = dev_info().cus;
    struct Cand { int bm, bn, per_cu; double rate; };
    // (FP8 starts at the second candidate: its fragments do not fit beside 256 x 256 accumulators)
    constexpr Cand cands[] = {{256, 256, 1, 1.0}, {256, 192, 1, 1.0}, {128, 128, 2, 0.75}};
    auto cost_of = [&](const Cand& c, int64_t n) {
        const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((n + c.bn - 1) / c.bn);
        const int64_t slots = cus * c.per_cu;
        return (double)((tiles + slots - 1) / slots) * c.per_cu * c.bm * c.bn / c.rate;
    };
    int best = 0;
    double best_cost = 1e300;
    for (int c = fp8 ? 1 : 0; c < 3; ++c) {
        const double cost = cost_of(cands[c], N);
        if (cost < best_cost * 0.999) {
            best_cost = cost;
            best = c;
        }
    }
    const Cand& b = cands[best];
    const int64_t tm = (M + b.bm - 1) / b.bm, tn = (N + b.bn - 1) / b.bn;
    const int64_t full = (tm * tn) / (cus * b.per_cu);            // full rounds
    const int64_t tn_main = full * cus * b.per_cu / tm;            // tile columns they cover
    if (may_split && full >= 1 && tn_main >= 1 && tn_main < tn) {
        const int64_t n_main = tn_main * b.bn;
        double tail_cost = 1e300;
        for (int c = fp8 ? 1 : 0; c < 3; ++c) tail_cost = std::min(tail_cost, cost_of(cands[c], N - n_main));
        if (full * b.per_cu * b.bm * b.bn / b.rate + tail_cost < 0.95 * best_cost) {
            const hipError_t e = launch_cols(Xq, xs, Wq, ws, ws_stride, bias, M, n_main, K, Y, ldy, ydt, acc_out,
                                             side, fp8, st, false, asym);
            if (e != hipSuccess) return e;
            AsymArgs asym2{};
            if (asym) asym2 = AsymArgs{asym->xz, asym->wrs + n_main};   // row sums of the remaining columns
            SideArgs side2{};
            if (side) {
                side2 = *side;
                side2.W16 = side->W16 + n_main * K;           // weight rows of the remaining columns
            }
            return launch_cols(Xq, xs, Wq + n_main * K, ws + n_main * ws_stride, ws_stride,
                               bias ? bias + n_main : nullptr, M, N - n_main, K,
                               static_cast<char*>(Y) + n_main * (ydt == SQ_F16 ? 2 : 4), ldy, ydt,
                               acc_out ? acc_out + n_main : nullptr, side ? &side2 : nullptr, fp8, st, false,
                               asym ? &asym2 : nullptr);
        }
    }
    if (best == 0)
        return dispatch<256, 256, SQ_W256_WM, SQ_W256_WN>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy, ydt,
                                                          acc_out, side, fp8, st, asym);
    if (best == 1)
        return dispatch<256, 192, SQ_W192_WM, SQ_W192_WN>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy, ydt,
                                                          acc_out, side, fp8, st, asym);
    return dispatch<128, 128, 2, 2>(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, ldy, ydt, acc_out, side, fp8, st,
                                    asym);
}

}  // namespace

hipError_t launch_gemm(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
                       const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int ydt, int32_t* acc_out,
                       const SideArgs* side, hipStream_t st) {
    return launch_cols(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, N, ydt, acc_out, side, false, st, true);
}

hipError_t launch_gemm_asym(const int8_t* Xq, const float* xs, const int32_t* xz, const int8_t* Wq, const float* ws,
                            int ws_stride, const int32_t* wrs, const float* bias, int64_t M, int64_t N, int64_t K,
                            void* Y, int ydt, int32_t* acc_out, hipStream_t st) {
    const AsymArgs asym{xz, wrs};
    return launch_cols(Xq, xs, Wq, ws, ws_stride, bias, M, N, K, Y, N, ydt, acc_out, nullptr, false, st, true, &asym);
}

hipError_t launch_gemm_fp8(const uint8_t* Xq, const float* xs, const uint8_t* Wq, const float* ws, int ws_stride,
                           const float* bias, int64_t M, int64_t N, int64_t K, void* Y, int ydt, float* acc_out,
                           hipStream_t st) {
    return launch_cols(reinterpret_cast<const int8_t*>(Xq), xs, reinterpret_cast<const int8_t*>(Wq), ws, ws_stride,
                       bias, M, N, K, Y, N, ydt, reinterpret_cast<int32_t*>(acc_out), nullptr, true, st, true);
}

}  // namespace sq
