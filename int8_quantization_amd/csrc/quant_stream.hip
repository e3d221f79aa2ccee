// Streaming per-token quantizer for fp16 activations on gfx950: the prefill
// shapes' hot path of the fused smoothing + per-token quantization
// ["量化基础与INT8", 量化流程示例: per-row absmax scale, round, clamp;
// "SmoothQuant量化实战", sections 3.3-3.4: X' = X / s before quantizing], and
// its LLM.int8() variant ["LLM.int8()技术解析", section 3.1: the columns whose
// absolute maximum exceeds the threshold leave the int8 part and are multiplied
// in fp16].  In that variant every block also turns the column maxima into the
// ascending outlier slots (a block-wide scan; block 0 writes the list and the
// count) and copies the outlier values of its rows out for the fp16 product, so
// the bookkeeping needs no launch of its own.
//
// Rows of up to 4096 values without outlier columns take quant_wave_kernel (one wave
// per row, below) instead of the streaming kernel.
//
// Persistent blocks (NT threads: two 512-thread blocks per CU, or one of 1024 for
// rows over 8192 values) walk steps of G consecutive rows (G row groups of NT/G
// threads).  Input rows reach LDS by DMA (buffer_load ... lds, no registers),
// through a ring of R slots: while a step is computed, the next R-1 steps are in
// flight, which keeps enough bytes moving to stream at HBM rate.  Per step:
//   wait for this wave's DMA of the step (s_waitcnt vmcnt with the exact count
//   of vector-memory instructions issued after it), barrier;
//   pass 1: x' = fl32(x / s_j) from LDS (x_j without smoothing), kept in
//   registers, |x'| maximum over the group's waves (shuffles, then LDS), barrier;
//   xs = fl32(max / 127);  pass 2: q = rne(fl32(x' / xs)) packed 4 per dword and
//   stored through a buffer resource; then the DMA of step + R into the slot the
//   step used.
// Counting: every wave issues exactly L DMA and CH code-store instructions per
// step (tail chunks, rows past M and steps past the block's last store to
// offsets outside the buffer range, which drops them, or read zeros), so after
// a step's DMA exactly (R-1)(CH+L) such instructions follow before its wait.
// Vector memory instructions complete in issue order, and any other load or
// store only adds to the count after the DMA, so waiting for at most that many
// outstanding guarantees the step's data.
//
// Arithmetic (identical to the register-resident kernel in quant.hip):
//  - x / s_j and x' / xs are RN32(RN64(a * rcp64(b))), which equals the IEEE
//    binary32 quotient in the normal range (proof at div_rcp64); an x / s_j
//    below it takes the IEEE division (possible only when s_j >= 2^100);
//  - rne of the fp32 quotient v comes from one fp32 addition: v + 1.5 * 2^23
//    rounds to the integer 1.5 * 2^23 + rne(v) for |v| < 2^22 (the sum lies in
//    [2^23, 2^24), where the spacing is 1, and 1.5 * 2^23 is even, so ties go to
//    even), and the low byte of its bit pattern is the two's-complement code.
//    A normal xs needs no clamp: |x'| <= max gives |v| <= 127 (1 + 2^-23), which
//    rounds to at most 127.  A subnormal xs (only with smoothing factors of 2^100 and
//    more, whose quotients x / s_j are subnormal) can be coarse enough for |v| > 127.5,
//    and such rows clamp v to [-128, 127] first.
#include <type_traits>

#include "sq_internal.h"

namespace sq {

namespace {

// NT threads per block: 512 (two blocks per CU, whose phases drift apart, so one
// computes while the other waits) for rows of up to 8192 values, 1024 (one block per
// CU) for longer rows, which need the whole block to keep a row in registers.
template <int NT, int CH> struct Ring {
    static constexpr int NW = NT / 64;                            // waves
    static constexpr int L = (CH + 1) / 2;                        // DMA instructions per wave per step
    static constexpr int SLOT = L * NW * 1024;                    // bytes per slot: NW waves x L x 1 KB
    static constexpr int LDS = NT == 1024 ? 144 * 1024 : 72 * 1024;   // ring bytes per block
    static constexpr int R = (LDS / SLOT) < 8 ? (LDS / SLOT) : 8;      // slots
    // vector-memory instructions counted after the DMA of step j before its wait:
    // (R-1) L + min(j, R-1) CH (see the kernel)
    static constexpr int AHEAD = (R - 1) * (CH + L);
    static_assert(R >= 3, "ring of at least three slots");
    static_assert(AHEAD <= 63, "vmcnt holds at most 63");
};

// s_waitcnt vmcnt(N) with the exp/lgkm counts unconstrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N> __device__ __forceinline__ void wait_vm() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}
// vmcnt(BASE + STEP * k) for a wave-uniform k in [0, KMAX] (a chain of scalar branches).
template <int BASE, int STEP, int KMAX> __device__ __forceinline__ void wait_vm_k(int k) {
    if constexpr (KMAX > 0) {
        if (k >= KMAX) {
            wait_vm<BASE + STEP * KMAX>();
            return;
        }
        wait_vm_k<BASE, STEP, KMAX - 1>(k);
    } else {
        wait_vm<BASE>();
    }
}
__device__ __forceinline__ void barrier_lds() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS accesses are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Code byte of rne(v) for |v| < 2^22, in the low byte of the result.
__device__ __forceinline__ uint32_t code_bits(float v) { return __float_as_uint(v + 12582912.0f); }

template <int NT, int CH, bool SMOOTH, bool OUTL>
__global__ __launch_bounds__(NT, NT == 1024 ? 1 : 2) void quant_stream_kernel(const _Float16* __restrict__ X, int M, int K,
                                                                   const float* __restrict__ s,
                                                                   int8_t* __restrict__ Xq, float* __restrict__ scale,
                                                                   OutlierSplit os, int G, int steps) {
    using RG = Ring<NT, CH>;
    constexpr int R = RG::R, L = RG::L, SLOT = RG::SLOT, NW = RG::NW;
    constexpr bool COLS = SMOOTH || OUTL;         // per-column constants to stage
    __shared__ __attribute__((aligned(1024))) int8_t ring[R * SLOT];
    __shared__ __attribute__((aligned(16))) float red[2][NW];
    constexpr int CPT_MAX = NT == 512 ? 16 : 20;  // K / NT: outlier-compaction columns per thread
    __shared__ int ocnt[OUTL ? CPT_MAX * NW : 1];   // per-(q, wave) counts, then their exclusive scan
    _Float16* __restrict__ Xo = os.Xo;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int tpg = NT / G;                       // threads per row group (>= 64)
    const int g = tid / tpg, t = tid - g * tpg;
    const int w0 = (g * tpg) >> 6, nwg = tpg >> 6;
    const int nch = K >> 2;                       // 4-value chunks per row
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const uint32_t step_bytes = (uint32_t)G * row_bytes;
    const uint32_t nblk = (step_bytes + 1023u) >> 10;   // 1 KB DMA blocks holding the step
    const uint32_t x_bytes = (uint32_t)M * row_bytes;
    const v4i rX = buffer_desc(X, x_bytes);
    const __amdgpu_buffer_rsrc_t rQ = __builtin_amdgcn_make_buffer_rsrc(Xq, 0, M * K, 0x00020000);
    const uint32_t lds_base = (uint32_t)(uintptr_t)ring;
    const int nb = gridDim.x;
    constexpr uint32_t OOB = 0x80000000u;         // beyond every record range: dropped / zeros

    // DMA of the block's step j (rows (j * nb + blockIdx.x) * G + [0, G)) into slot j % R
    auto dma_step = [&](int j) {
        const uint64_t src = (uint64_t)((uint32_t)j * (uint32_t)nb + blockIdx.x) * step_bytes;
        const uint32_t src0 = src < x_bytes ? (uint32_t)src : OOB;
        const uint32_t slot = (uint32_t)(j % R) * SLOT;
#pragma unroll
        for (int l = 0; l < L; ++l) {
            const uint32_t b = (uint32_t)(wave + NW * l);
            const uint32_t voff = (b < nblk && src0 != OOB) ? src0 + b * 1024u + (uint32_t)lane * 16u : OOB;
            dma_to_lds(rX, __builtin_amdgcn_readfirstlane(lds_base + slot + b * 1024u), voff, 0);
        }
    };

    // Prologue.  The per-column array (s, or the column maxima) is DMA'd into the last NP
    // slots of the ring, the first R - NP steps into the others; once the array has landed
    // the constants are computed while those steps are in flight, then the remaining steps
    // are requested.  Every wave issues the same instructions, so the counts below hold
    // for each wave.
    const int NP = COLS ? (int)(((uint32_t)K * 4u + SLOT - 1) / SLOT) : 0;   // 1 .. R-1 slots
    if constexpr (COLS) {
        const v4i rP = buffer_desc(SMOOTH ? (const void*)s : (const void*)os.cmax, (uint32_t)K * 4u);
        const uint32_t pbase = lds_base + (uint32_t)(R - NP) * SLOT;
        // K * 4 <= 16 bytes x NT x CH: at most CH 1 KB blocks per wave; blocks past the array read
        // zeros, and none is written past the NP slots (a wave-uniform condition; the count
        // waited for below is of the instructions issued after these)
        for (int l = 0; l < CH; ++l) {
            const uint32_t b = (uint32_t)(wave + NW * l);
            if (b * 1024u < (uint32_t)NP * SLOT)
                dma_to_lds(rP, __builtin_amdgcn_readfirstlane(pbase + b * 1024u), b * 1024u + (uint32_t)lane * 16u, 0);
        }
    }
    for (int j = 0; j < R - NP; ++j) dma_step(j);

    bool valid[CH];
    double rs[SMOOTH ? CH : 1][4];
    unsigned omask[OUTL ? CH : 1];
    int opos[OUTL ? CH : 1][4];
    unsigned ochunks = 0;                         // bit i: some lane of this wave has an outlier in chunk i
    bool guard = false;                           // some x / s_j may fall below the fp32 normal range
    // LLM.int8() outlier columns c = tid + NT q (q < cpt) of this thread
    const int cpt = (K + NT - 1) / NT;
    unsigned oflags = 0;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below this one
#pragma unroll
    for (int i = 0; i < CH; ++i) valid[i] = t + i * tpg < nch;
    if constexpr (COLS) {
        wait_vm_k<0, L, R - 1>(R - NP);           // the array landed (R - NP steps' DMA issued after it)
        barrier_lds();
        int8_t* P = ring + (R - NP) * SLOT;
        if constexpr (OUTL) {
            // Compaction, in every block: column c is an outlier when its maximum exceeds the
            // threshold, and slots ascend with c.  Columns are visited as c = tid + NT q, so
            // every LDS access is conflict-free; the slot of c counts the flagged columns of
            // the rows q' < q and of the waves w' < w in row q (an exclusive scan of the
            // per-(q, wave) counts, done by wave 0) plus the flagged lanes below in its wave.
            // The slots replace the maxima in LDS; block 0 also writes the ascending column
            // list and the count for the later kernels.
            int* cnt = ocnt;
#pragma unroll
            for (int q = 0; q < CPT_MAX; ++q) {
                const int c = tid + NT * q;
                const bool f = q < cpt && c < K &&
                               __uint_as_float(*reinterpret_cast<const uint32_t*>(P + 4 * c)) > os.threshold;
                oflags |= (unsigned)f << q;
                const uint64_t m = __builtin_amdgcn_ballot_w64(f);
                if (lane == 0 && q < cpt) cnt[q * NW + wave] = __builtin_popcountll(m);
            }
            barrier_lds();
            if (wave == 0) {                      // exclusive scan of the cpt * NW counts, E per lane
                constexpr int E = (CPT_MAX * NW + 63) / 64;
                const int n = cpt * NW;
                int a[E], sum = 0;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    a[e] = E * lane + e < n ? cnt[E * lane + e] : 0;
                    sum += a[e];
                }
                int incl = sum;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int u = __shfl_up(incl, off, 64);
                    if (lane >= off) incl += u;
                }
                int ex = incl - sum;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (E * lane + e < n) cnt[E * lane + e] = ex;
                    ex += a[e];
                }
                if (lane == 63 && blockIdx.x == 0) {
                    *os.count = incl;
                    if (os.user_count) *os.user_count = incl;
                }
            }
            barrier_lds();
#pragma unroll
            for (int q = 0; q < CPT_MAX; ++q) {
                const int c = tid + NT * q;
                if (q < cpt && c < K) {
                    const bool f = (oflags >> q) & 1u;
                    const uint64_t m = __builtin_amdgcn_ballot_w64(f);
                    const int slot = cnt[q * NW + wave] + __builtin_popcountll(m & below);
                    *reinterpret_cast<int32_t*>(P + 4 * c) = f ? slot : -1;
                    if (f && blockIdx.x == 0) {
                        os.idx[slot] = c;
                        if (os.user_idx) os.user_idx[slot] = c;
                    }
                }
            }
            barrier_lds();                        // every slot is in LDS
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            const int cc = valid[i] ? t + i * tpg : 0;
            if constexpr (SMOOTH) {
                const v4f sv = *reinterpret_cast<const v4f*>(P + 16 * cc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rs[i][e] = rcp64((double)sv[e]);
                    guard = guard || !(sv[e] < 0x1p100f);
                }
            }
            if constexpr (OUTL) {
                const v4i pq = *reinterpret_cast<const v4i*>(P + 16 * cc);
                omask[i] = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    opos[i][e] = pq[e];
                    if (valid[i] && pq[e] >= 0) omask[i] |= 1u << e;
                }
                if (__builtin_amdgcn_ballot_w64(omask[i] != 0) != 0) ochunks |= 1u << i;
            }
        }
        barrier_lds();                            // the array's slots are free again
        for (int j = R - NP; j < R; ++j) dma_step(j);
    }
    const bool guard_wave = __builtin_amdgcn_ballot_w64(guard) != 0;
    bool clamp_rows = false;                      // this wave saw a row with a subnormal xs

    for (int j = 0; j < steps; ++j) {
        // After this wave's DMA of step j it issued (R-1) L DMA instructions (later steps)
        // and CH code stores for each of the min(j, R-1) steps before j; any other memory
        // instruction only adds to that.
        wait_vm_k<(R - 1) * L, CH, R - 1>(j);
        barrier_lds();                            // every wave's part of step j landed
        const int row = (j * nb + (int)blockIdx.x) * G + g;
        const bool live = row < M;
        const int8_t* rowp = ring + (j % R) * SLOT + g * (int)row_bytes;

        float xv[CH][4];
        float amax = 0.0f;
        auto pass1 = [&](auto guarded) {
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int c = t + i * tpg;
                const h4 hv = *reinterpret_cast<const h4*>(rowp + 8 * c);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = (float)hv[e];
                    if constexpr (SMOOTH) {
                        float q = (float)((double)x * rs[i][e]);
                        if constexpr (decltype(guarded)::value)
                            if (__builtin_fabsf(q) < 1.17549435e-38f && x != 0.0f && valid[i]) q = x / s[4 * c + e];
                        x = q;
                    }
                    // only the last chunk can lie past the row (CH = ceil(chunks / tpg)); its values
                    // there are zeroed, which leaves the maximum unchanged
                    if (i == CH - 1) x = valid[i] ? x : 0.0f;
                    xv[i][e] = x;
                }
                if constexpr (OUTL) {
                    if ((ochunks >> i) & 1u) {    // wave-uniform: some lane holds an outlier column here
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const bool o = (omask[i] >> e) & 1u;
                            if (o && live) Xo[(int64_t)row * K + opos[i][e]] = hv[e];
                            xv[i][e] = o ? 0.0f : xv[i][e];     // out of the maximum; code 0 below
                        }
                    }
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(xv[i][e]));
            }
        };
        // the IEEE-division check runs only in waves with some s_j >= 2^100 (a uniform branch)
        if (SMOOTH && guard_wave) pass1(std::true_type{});
        else pass1(std::false_type{});
        amax = wave_max(amax);
        if (lane == 0) red[j & 1][wave] = amax;
        barrier_lds();                            // also: every wave is done reading the step's slot
        float a = red[j & 1][w0];
        if (nwg >= 4) {                           // the group's wave maxima, 16 bytes per read
            for (int w = 0; w < nwg; w += 4) {
                const v4f r4 = *reinterpret_cast<const v4f*>(&red[j & 1][w0 + w]);
                a = __builtin_fmaxf(a, __builtin_fmaxf(__builtin_fmaxf(r4[0], r4[1]), __builtin_fmaxf(r4[2], r4[3])));
            }
        } else {
            for (int w = 1; w < nwg; ++w) a = __builtin_fmaxf(a, red[j & 1][w0 + w]);
        }
        // xs = fl32(a / 127) as RN32(RN64(a * RN64(1/127))), exact for a normal-range
        // quotient (the argument at div_rcp64); a quotient below it takes the division
        float xs = (float)((double)a * (1.0 / 127.0));
        if (xs < 1.17549435e-38f && a != 0.0f) xs = a / 127.0f;
        if (live && t == 0) scale[row] = xs;
        const double rx = xs != 0.0f ? rcp64((double)xs) : 0.0;   // xs == 0: every x' is 0, codes 0

        // A normal xs keeps |x' / xs| < 127.5.  With smoothing factors of 2^100 and more,
        // max |x'| can be so small that xs is a coarse subnormal and the quotient exceeds
        // the code range: such rows are noted here and get clamped codes after the loop.
        if (SMOOTH && live && xs < 1.17549435e-38f) clamp_rows = true;
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            uint32_t b[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) b[e] = code_bits((float)((double)xv[i][e] * rx));
            const uint32_t w = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                                     __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u), 0x05040100u);
            const int c = t + i * tpg;
            const uint32_t off = (live && valid[i]) ? (uint32_t)row * (uint32_t)K + 4u * (uint32_t)c : OOB;
            __builtin_amdgcn_raw_buffer_store_b32(w, rQ, (int)off, 0, 0);
        }
        dma_step(j + R);                          // into the slot this step used
    }
    if (SMOOTH && clamp_rows) {
        // Rows whose xs is subnormal (see above; a wave-uniform flag, so normal data only
        // pays this test).  The wave waits for its own stores, then for each of its rows
        // recomputes the row maximum over all K columns (x / s_j as in pass 1) and, where xs
        // is subnormal, rewrites its threads' chunks with clamped codes.  Each chunk is only
        // ever written by its own thread, so no other wave is involved.
        __builtin_amdgcn_s_waitcnt(0);
        auto xprime = [&](float x, int col) {
            float q = (float)((double)x * rcp64((double)s[col]));
            if (__builtin_fabsf(q) < 1.17549435e-38f && x != 0.0f) q = x / s[col];
            return q;
        };
        for (int j = 0; j < steps; ++j) {
            const int row = (j * nb + (int)blockIdx.x) * G + g;
            if (row >= M) continue;                  // uniform: a wave lies in one group
            const _Float16* xr = X + (int64_t)row * K;
            float amax = 0.0f;
            for (int col = lane; col < K; col += 64) amax = __builtin_fmaxf(amax, __builtin_fabsf(xprime((float)xr[col], col)));
            amax = wave_max(amax);
            const float xs = amax / 127.0f;
            if (!(xs < 1.17549435e-38f) || xs == 0.0f) continue;
            const double rx = rcp64((double)xs);
#pragma unroll
            for (int i = 0; i < CH; ++i) {
                const int c = t + i * tpg;
                if (!valid[i]) continue;
                uint32_t w = 0;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float v = __builtin_amdgcn_fmed3f((float)((double)xprime((float)xr[4 * c + e], 4 * c + e) * rx),
                                                            -128.0f, 127.0f);
                    w |= (code_bits(v) & 0xffu) << (8 * e);
                }
                *reinterpret_cast<uint32_t*>(Xq + (int64_t)row * K + 4 * c) = w;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// One wave per row, for rows of up to 4096 values with at least four rows per CU (the
// 7B-class prefill activations), with the same arithmetic as the streaming kernel.
// Lane l holds the 16-byte chunks l, l + 64, ... of its row (read through a per-row
// buffer resource: a row past M has 0 records, so its reads return zeros and its
// stores are dropped), converts them to x' in registers, and the row maximum is a DPP
// reduction inside the wave, so there is no block barrier in the row loop and no LDS
// round trip per row.  With smoothing, the block keeps RN64(1/s_j) of every column in
// LDS (computed once, while the first rows are in flight).  The next row's loads go out
// as soon as the current row is converted.
//
// Without a column s_j >= 2^100 (or NaN), x / s_j never falls below the fp32 normal
// range (|x| >= 2^-24 for a non-zero binary16), so RN32(RN64(x * RN64(1/s_j))) is the
// quotient, every non-zero |x'| is at least 2^-124, xs = fl32(max / 127) is within
// 2^-18 relative of max / 127, and |fl32(x' / xs)| < 127.5: the codes need no clamp.  If
// some column has s_j >= 2^100, every wave takes a plain two-pass loop per row instead
// (the IEEE division for quotients below the normal range, and the clamp), which reads
// the row again for the codes.
template <int CPL, bool SMOOTH, int FMT>
__global__ __launch_bounds__(256) void quant_wave_kernel(const _Float16* __restrict__ X, int M, int K,
                                                         const float* __restrict__ s, int8_t* __restrict__ Xq,
                                                         float* __restrict__ scale) {
    constexpr int kThreads = 256, kWaves = kThreads / 64;
    constexpr int FPT = (CPL + 1) / 2;           // s vectors (4 floats) per thread: K / 4 <= 128 CPL
    extern __shared__ double srcp[];             // SMOOTH: RN64(1 / s_j), 4 * kThreads * FPT slots
    __shared__ int hflag[kWaves];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nchunk = K / 8;
    const int nv4 = K / 4;
    const int nwv = (int)gridDim.x * kWaves;
    int m = (int)blockIdx.x * kWaves + wave;
    auto row_rsrc = [&](const void* base, int row, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, row < M ? bytes : 0, 0x00020000);
    };
    auto load = [&](int row, v4i* r) {
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(X + (int64_t)(row < M ? row : 0) * K, row, 2 * K);
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            r[i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (lane + 64 * i), 0, 0));
    };
    // prologue: the s loads, then the first row's loads, then the reciprocals into LDS (the
    // LDS writes wait for the s loads only); the slots past K are slack, never read
    v4f sv[SMOOTH ? FPT : 1];
    if constexpr (SMOOTH) {
#pragma unroll
        for (int i = 0; i < FPT; ++i) {
            const int j = (int)threadIdx.x + kThreads * i;
            sv[i] = reinterpret_cast<const v4f*>(s)[j < nv4 ? j : nv4 - 1];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    v4i cur[CPL];
    load(m, cur);
    __builtin_amdgcn_sched_barrier(0);
    bool huge = false;
    if constexpr (SMOOTH) {
#pragma unroll
        for (int i = 0; i < FPT; ++i) {
            const int j = (int)threadIdx.x + kThreads * i;
            double r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                r[e] = rcp64((double)sv[i][e]);
                huge = huge || (j < nv4 && !(sv[i][e] < 0x1p100f));
            }
            reinterpret_cast<v4f*>(srcp)[2 * j] = __builtin_bit_cast(v4f, (double __attribute__((ext_vector_type(2)))){r[0], r[1]});
            reinterpret_cast<v4f*>(srcp)[2 * j + 1] = __builtin_bit_cast(v4f, (double __attribute__((ext_vector_type(2)))){r[2], r[3]});
        }
    }
    if (lane == 0) hflag[wave] = __builtin_amdgcn_ballot_w64(huge) != 0;
    barrier_lds();
    const bool slow = SMOOTH && (hflag[0] | hflag[1] | hflag[2] | hflag[3]) != 0;
    const v4f* sr = reinterpret_cast<const v4f*>(srcp);

    if (slow) {
        // some s_j >= 2^100: per element div_rcp64 semantics (the IEEE division below the
        // normal range) and clamped codes, the row read twice
        for (; m < M; m += nwv) {
            const _Float16* xr = X + (int64_t)m * K;
            auto xprime = [&](_Float16 h, int j) {
                const float x = (float)h;
                float q = (float)((double)x * srcp[j]);
                if (__builtin_fabsf(q) < 1.17549435e-38f && x != 0.0f) q = x / s[j];
                return q;
            };
            float amax = 0.0f;
            for (int c = lane; c < nchunk; c += 64) {
                const h8 hv = *reinterpret_cast<const h8*>(xr + 8 * c);
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(xprime(hv[e], 8 * c + e)));
            }
            amax = wave_max(amax);
            const float xs = amax / (FMT == 0 ? 127.0f : 448.0f);
            if (lane == 0) scale[m] = xs;
            const double rx = xs != 0.0f ? rcp64((double)xs) : 0.0;
            for (int c = lane; c < nchunk; c += 64) {
                const h8 hv = *reinterpret_cast<const h8*>(xr + 8 * c);
                uint32_t w[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = xs == 0.0f ? 0.0f : (float)((double)xprime(hv[4 * h + e], 8 * c + 4 * h + e) * rx);
                    if constexpr (FMT == 0) {
                        uint32_t b = 0;
#pragma unroll
                        for (int e = 0; e < 4; ++e) b |= (uint32_t)(code_of(v[e]) & 0xff) << (8 * e);
                        w[h] = b;
                    } else {
                        w[h] = fp8x4(fp8_clamp(v[0]), fp8_clamp(v[1]), fp8_clamp(v[2]), fp8_clamp(v[3]));
                    }
                }
                *reinterpret_cast<uint2*>(Xq + (int64_t)m * K + 8 * c) = make_uint2(w[0], w[1]);
            }
        }
        return;
    }

    // the first row's pass runs on every wave (a wave without a row reads zeros, and its
    // stores are dropped), so that its loads stay ahead of the barrier above
    uint32_t lbase = 0;                            // LDS offset, re-read per row (see below)
    do {
        // an opaque zero: keeps the compiler from hoisting the reciprocal reads out of the
        // row loop into registers (128 of them, which would halve the waves per SIMD)
        asm volatile("" : "+s"(lbase));
        float xk[CPL][8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int c = lane + 64 * i;
            v4f r4[4];
            if constexpr (SMOOTH) {
                const int cc = (c < nchunk ? c : 0) + (int)lbase;   // chunks past the row hold zeros
#pragma unroll
                for (int u = 0; u < 4; ++u) r4[u] = sr[4 * cc + u];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float x = (float)__builtin_bit_cast(_Float16, (uint16_t)((uint32_t)cur[i][e >> 1] >> (16 * (e & 1))));
                if constexpr (SMOOTH) {
                    const double r = __builtin_bit_cast(double, (uint64_t)__float_as_uint(r4[e >> 1][2 * (e & 1)]) |
                                                                    ((uint64_t)__float_as_uint(r4[e >> 1][2 * (e & 1) + 1]) << 32));
                    x = (float)((double)x * r);
                }
                xk[i][e] = x;
            }
            float a = __builtin_fmaxf(__builtin_fabsf(xk[i][0]), __builtin_fabsf(xk[i][1]));
#pragma unroll
            for (int e = 2; e < 8; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(xk[i][e]));
            amax = __builtin_fmaxf(amax, a);
        }
        load(m + nwv, cur);                        // next row, in flight from here
        amax = wave_max(amax);
        const float xs = amax / (FMT == 0 ? 127.0f : 448.0f);
        if (lane == 0 && m < M) scale[m] = xs;
        const double rx = xs != 0.0f ? rcp64((double)xs) : 0.0;   // xs == 0: every x' is 0, codes 0
        const __amdgpu_buffer_rsrc_t rq = row_rsrc(Xq + (int64_t)m * K, m, K);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            uint32_t lo, hi;
            if constexpr (FMT == 0) {
                uint32_t b[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) b[e] = code_bits((float)((double)xk[i][e] * rx));
                lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u),
                                           __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u), 0x05040100u);
                hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u),
                                           __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u), 0x05040100u);
            } else {
                // E4M3 codes of fl32(x' / xs) clamped to [-448, 448] (a subnormal xs can leave the
                // quotient above 448; xs == 0 gives rx = 0 and code 0)
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = fp8_clamp((float)((double)xk[i][e] * rx));
                lo = fp8x4(v[0], v[1], v[2], v[3]);
                hi = fp8x4(v[4], v[5], v[6], v[7]);
            }
            __builtin_amdgcn_raw_buffer_store_b64((unsigned int __attribute__((ext_vector_type(2)))){lo, hi}, rq,
                                                  8 * (lane + 64 * i), 0, 0);
        }
        m += nwv;
    } while (m < M);
}

template <int CPL, bool SMOOTH, int FMT>
hipError_t launch_wave(const _Float16* X, int M, int K, const float* s, int8_t* Xq, float* scale, hipStream_t st) {
    constexpr int kWaves = 4;
    const int64_t blocks = ((int64_t)M + kWaves - 1) / kWaves;
    const int64_t cap = (int64_t)dev_info().cus * 8;
    const size_t lds = SMOOTH ? (size_t)256 * ((CPL + 1) / 2) * 4 * sizeof(double) : 0;
    SQ_LAUNCH((quant_wave_kernel<CPL, SMOOTH, FMT>), dim3((unsigned)(blocks < cap ? blocks : cap)), dim3(64 * kWaves), lds,
              st, X, M, K, s, Xq, scale);
    return hipSuccess;
}

template <bool SMOOTH, int FMT>
hipError_t launch_wave_k(const _Float16* X, int M, int K, const float* s, int8_t* Xq, float* scale, hipStream_t st) {
    if (K <= 512) return launch_wave<1, SMOOTH, FMT>(X, M, K, s, Xq, scale, st);
    if (K <= 1024) return launch_wave<2, SMOOTH, FMT>(X, M, K, s, Xq, scale, st);
    if (K <= 2048) return launch_wave<4, SMOOTH, FMT>(X, M, K, s, Xq, scale, st);
    return launch_wave<8, SMOOTH, FMT>(X, M, K, s, Xq, scale, st);
}

template <int NT, int CH, bool SMOOTH, bool OUTL>
hipError_t launch_ch(const _Float16* X, int M, int K, const float* s, int8_t* Xq, float* scale, const OutlierSplit& os,
                     int G, hipStream_t st) {
    const int64_t total = ((int64_t)M + G - 1) / G;               // steps over all blocks
    const int64_t slots = (int64_t)dev_info().cus * (NT == 1024 ? 1 : 2);
    const int nb = (int)(total < slots ? total : slots);
    const int steps = (int)((total + nb - 1) / nb);
    SQ_LAUNCH((quant_stream_kernel<NT, CH, SMOOTH, OUTL>), dim3((unsigned)nb), dim3(NT), 0, st, X, M, K, s, Xq, scale,
              os, G, steps);
    return hipSuccess;
}

template <bool SMOOTH, bool OUTL>
hipError_t launch_mode(const _Float16* X, int M, int K, const float* s, int8_t* Xq, float* scale, const OutlierSplit& os,
                       int nt, int G, int ch, hipStream_t st) {
    if (nt == 512) {
        switch (ch) {
            case 1: return launch_ch<512, 1, SMOOTH, OUTL>(X, M, K, s, Xq, scale, os, G, st);
            case 2: return launch_ch<512, 2, SMOOTH, OUTL>(X, M, K, s, Xq, scale, os, G, st);
            case 3: return launch_ch<512, 3, SMOOTH, OUTL>(X, M, K, s, Xq, scale, os, G, st);
            default: return launch_ch<512, 4, SMOOTH, OUTL>(X, M, K, s, Xq, scale, os, G, st);
        }
    }
    switch (ch) {
        case 3: return launch_ch<1024, 3, SMOOTH, OUTL>(X, M, K, s, Xq, scale, os, G, st);
        case 4: return launch_ch<1024, 4, SMOOTH, OUTL>(X, M, K, s, Xq, scale, os, G, st);
        default: return launch_ch<1024, 5, SMOOTH, OUTL>(X, M, K, s, Xq, scale, os, G, st);
    }
}

}  // namespace

bool quant_stream_applies(int64_t M, int64_t K, bool smooth, bool outliers) {
    // rows of up to 5 x 4096 values (longer rows would spill the per-column constants);
    // enough rows for every CU to stream several steps; byte offsets of X (and of the steps
    // past the last) within 31 bits; no smoothing together with outlier columns (LLM.int8()
    // does not smooth)
    return K <= 20480 && M >= 4 * (int64_t)dev_info().cus && (M + 16 * 1024) * K * 2 < ((int64_t)1 << 31) &&
           !(smooth && outliers);
}

hipError_t launch_quant_stream(const _Float16* X, int64_t M, int64_t K, const float* s, int8_t* Xq, float* scale,
                               const OutlierSplit* os, hipStream_t st) {
    // Rows of up to 8192 values: 512-thread blocks, G row groups per step, the most that
    // keep at most 4 chunks per thread (bigger steps spread the per-step reduction and
    // synchronization over more values).  Longer rows: 1024 threads, one row per step,
    // up to 5 chunks per thread.
    if (!os && K <= 4096) {                      // one wave per row
        if (s) return launch_wave_k<true, 0>(X, (int)M, (int)K, s, Xq, scale, st);
        return launch_wave_k<false, 0>(X, (int)M, (int)K, nullptr, Xq, scale, st);
    }
    const int64_t nch = K / 4;
    const int nt = K <= 8192 ? 512 : 1024;
    int G = nt / 64;
    while (G > 1 && (nch + nt / G - 1) / (nt / G) > 4) G /= 2;
    const int ch = (int)((nch + nt / G - 1) / (nt / G));
    const OutlierSplit none{};
    if (s) return launch_mode<true, false>(X, (int)M, (int)K, s, Xq, scale, none, nt, G, ch, st);
    if (os) return launch_mode<false, true>(X, (int)M, (int)K, nullptr, Xq, scale, *os, nt, G, ch, st);
    return launch_mode<false, false>(X, (int)M, (int)K, nullptr, Xq, scale, none, nt, G, ch, st);
}

hipError_t launch_quant_wave_fp8(const _Float16* X, int64_t M, int64_t K, const float* s, int8_t* q, float* scale,
                                 hipStream_t st) {
    if (s) return launch_wave_k<true, 1>(X, (int)M, (int)K, s, q, scale, st);
    return launch_wave_k<false, 1>(X, (int)M, (int)K, nullptr, q, scale, st);
}

}  // namespace sq
