// LLM.int8() outlier bookkeeping for gfx950 ["LLM.int8()技术解析", sections 2.1
// and 3.1: column-wise absolute maximum of the input, a bitmask of the columns
// above the threshold, int8 for the rest and fp16 for these].
//
// The column maxima come from the shared column-absmax kernel.  Here one block
// turns them into the ascending outlier list, a per-column slot (or -1) and the
// count, with a block-wide prefix sum of per-thread counts; the count stays on the device and
// every later kernel reads it, so the host never waits.  (The activation columns
// are gathered by the quantization kernel, which reads every row anyway; the
// GEMM reads the weight's outlier columns in place.)  Rows the streaming
// quantizer takes do the compaction there instead.
#include "sq_internal.h"

namespace sq {

namespace {

// One block; thread t owns 8 consecutive columns of each 8192-column pass (K is a multiple of 16, so
// the 8 are all in range or all out).  Slots: exclusive prefix sum of the per-thread counts (wave
// shuffles, then the 16 wave totals through LDS).
__global__ __launch_bounds__(1024) void outlier_compact_kernel(const uint32_t* __restrict__ cmax_bits, int64_t K,
                                                               float threshold, int32_t* __restrict__ idx,
                                                               int32_t* __restrict__ pos, int32_t* __restrict__ count,
                                                               int32_t* __restrict__ user_count,
                                                               int32_t* __restrict__ user_idx) {
    constexpr int PER = 8;
    __shared__ int wave_tot[16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, nw = blockDim.x >> 6;
    int base = 0;
    for (int64_t j0 = 0; j0 < K; j0 += (int64_t)blockDim.x * PER) {
        const int64_t jb = j0 + (int64_t)tid * PER;
        unsigned flags = 0;
        if (jb < K) {
            const uint4 lo = *reinterpret_cast<const uint4*>(cmax_bits + jb);
            const uint4 hi = *reinterpret_cast<const uint4*>(cmax_bits + jb + 4);
            const uint32_t v[PER] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
            for (int e = 0; e < PER; ++e) flags |= (unsigned)(__uint_as_float(v[e]) > threshold) << e;
        }
        const int cnt = __popc(flags);
        int incl = cnt;                          // inclusive scan within the wave
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(incl, off, 64);
            if (lane >= off) incl += t;
        }
        if (lane == 63) wave_tot[wave] = incl;
        __syncthreads();
        int woff = 0, tot = 0;
        for (int w = 0; w < nw; ++w) {
            const int t = wave_tot[w];
            woff += w < wave ? t : 0;
            tot += t;
        }
        int p = base + woff + incl - cnt;
        if (jb < K) {
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const bool f = (flags >> e) & 1u;
                pos[jb + e] = f ? p : -1;
                if (f) {
                    idx[p] = (int32_t)(jb + e);
                    if (user_idx) user_idx[p] = (int32_t)(jb + e);
                    ++p;
                }
            }
        }
        base += tot;
        __syncthreads();                         // wave_tot is rewritten by the next pass
    }
    if (tid == 0) {
        *count = base;
        if (user_count) *user_count = base;
    }
}

}  // namespace

hipError_t launch_outlier_compact(const uint32_t* cmax_bits, int64_t K, float threshold, int32_t* idx, int32_t* pos,
                                  int32_t* count, int32_t* user_count, int32_t* user_idx, hipStream_t st) {
    SQ_LAUNCH(outlier_compact_kernel, dim3(1), dim3(1024), 0, st, cmax_bits, K, threshold, idx, pos, count,
                       user_count, user_idx);
    return hipSuccess;
}

}  // namespace sq
