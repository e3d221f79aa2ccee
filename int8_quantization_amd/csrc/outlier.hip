// LLM.int8() outlier bookkeeping for gfx950 ["LLM.int8()技术解析", sections 2.1
// and 3.1: column-wise absolute maximum of the input, a bitmask of the columns
// above the threshold, int8 for the rest and fp16 for these].
//
// The column maxima come from the shared column-absmax kernel.  Here one block
// turns them into the ascending outlier list, a per-column slot (or -1) and the
// count, with a ballot/popcount prefix sum; the count stays on the device and
// every later kernel reads it, so the host never waits.  A second kernel
// gathers the weight's outlier columns into a dense [N x count] fp16 panel for
// the side MFMA product (the activation columns are gathered by the
// quantization kernel, which reads every row anyway).
#include "sq_internal.h"

namespace sq {

namespace {

__global__ __launch_bounds__(1024) void outlier_compact_kernel(const uint32_t* __restrict__ cmax_bits, int64_t K,
                                                               float threshold, int32_t* __restrict__ idx,
                                                               int32_t* __restrict__ pos, int32_t* __restrict__ count,
                                                               int32_t* __restrict__ user_count,
                                                               int32_t* __restrict__ user_idx) {
    __shared__ int wave_tot[16];
    __shared__ int wave_off[16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, nw = blockDim.x >> 6;
    int base = 0;
    for (int64_t j0 = 0; j0 < K; j0 += blockDim.x) {
        const int64_t j = j0 + tid;
        const bool flag = j < K && __uint_as_float(cmax_bits[j]) > threshold;
        const unsigned long long mask = __ballot(flag);
        const int before = __popcll(mask & ((1ull << lane) - 1ull));
        if (lane == 0) wave_tot[wave] = __popcll(mask);
        __syncthreads();
        if (tid == 0) {
            int acc = 0;
            for (int w = 0; w < nw; ++w) {
                wave_off[w] = acc;
                acc += wave_tot[w];
            }
            wave_tot[0] = acc;   // block total, read below after the barrier
        }
        __syncthreads();
        const int p = base + wave_off[wave] + before;
        if (j < K) {
            pos[j] = flag ? p : -1;
            if (flag) {
                idx[p] = (int32_t)j;
                if (user_idx) user_idx[p] = (int32_t)j;
            }
        }
        base += wave_tot[0];
        __syncthreads();
    }
    if (tid == 0) {
        *count = base;
        if (user_count) *user_count = base;
    }
}

// Wo[n * ldo + t] = W16[n * K + idx[t]], t < *count; 4 rows per block, 64 lanes per row.
__global__ __launch_bounds__(256) void gather_cols_kernel(const _Float16* __restrict__ W16, int64_t N, int64_t K,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ count,
                                                          _Float16* __restrict__ Wo) {
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (n >= N) return;
    const int c = *count;
    for (int t = lane; t < c; t += 64) Wo[n * K + t] = W16[n * K + idx[t]];
}

}  // namespace

hipError_t launch_outlier_compact(const uint32_t* cmax_bits, int64_t K, float threshold, int32_t* idx, int32_t* pos,
                                  int32_t* count, int32_t* user_count, int32_t* user_idx, hipStream_t st) {
    hipLaunchKernelGGL(outlier_compact_kernel, dim3(1), dim3(1024), 0, st, cmax_bits, K, threshold, idx, pos, count,
                       user_count, user_idx);
    return hipGetLastError();
}

hipError_t launch_gather_cols(const _Float16* W16, int64_t N, int64_t K, const int32_t* idx, const int32_t* count,
                              _Float16* Wo, hipStream_t st) {
    hipLaunchKernelGGL(gather_cols_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, st, W16, N, K, idx, count, Wo);
    return hipGetLastError();
}

}  // namespace sq
