// Decode (skinny-M, M <= 16) int8 GEMM + dequant for gfx950.
//
// At M <= 16 the layer streams N x K int8 weight bytes once and reuses each of
// them at most 16 times, so it is bound by HBM bandwidth, not by the matrix
// cores.  A 256-thread block owns 16 output features; its 4 waves interleave
// over 64-byte k blocks (wave w takes blocks w, w+4, ...), each lane loading 16
// contiguous bytes of one weight row and of one activation row, and one
// v_mfma_i32_16x16x64_i8 per k block folds all M tokens at once (rows >= M are
// zero).  Eight k blocks are in flight per wave.  The four partial int32 tiles
// are summed through LDS and the dequant epilogue
// ["量化基础与INT8", INT8推理流程: acc * x_scale * w_scale] runs on wave 0.
// Result lane l, register i holds D[4*(l/16) + i][l % 16] = (token, feature).
#include "sq_internal.h"

namespace sq {

namespace {

template <bool OUT_F16>
__global__ __launch_bounds__(256) void gemv_i8_kernel(const int8_t* __restrict__ Xq, const float* __restrict__ xs,
                                                      const int8_t* __restrict__ Wq, const float* __restrict__ ws,
                                                      int ws_stride, const float* __restrict__ bias, int M, int N,
                                                      int K, void* __restrict__ Yv, int32_t* __restrict__ acc_out) {
    constexpr int U = 8;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const bool nval = n0 + r < N, mval = r < M;
    const int8_t* wrow = Wq + (int64_t)(nval ? n0 + r : 0) * K;
    const int8_t* xrow = Xq + (int64_t)(mval ? r : 0) * K;
    const int nkb = (K + 63) / 64;

    v4i acc = {0, 0, 0, 0};
    for (int kb0 = wave; kb0 < nkb; kb0 += 4 * U) {
        v4i wv[U], xv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = kb0 + 4 * u;
            const int k = kb * 64 + g * 16;
            const bool kval = kb < nkb && k < K;
            wv[u] = (kval && nval) ? __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow + k))
                                   : v4i{0, 0, 0, 0};
            xv[u] = (kval && mval) ? *reinterpret_cast<const v4i*>(xrow + k) : v4i{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(xv[u], wv[u], acc, 0, 0, 0);
    }

    __shared__ v4i part[4][64];
    part[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    const v4i tot = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    const int n = n0 + r;
    if (n >= N) return;
    const float wsv = ws[(int64_t)n * ws_stride];
    const float bv = bias != nullptr ? bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m >= M) continue;
        float y = (float)tot[i];
        y = y * xs[m];
        y = y * wsv;
        if (bias != nullptr) y = y + bv;
        if constexpr (OUT_F16) reinterpret_cast<_Float16*>(Yv)[(int64_t)m * N + n] = (_Float16)y;
        else reinterpret_cast<float*>(Yv)[(int64_t)m * N + n] = y;
        if (acc_out != nullptr) acc_out[(int64_t)m * N + n] = tot[i];
    }
}

}  // namespace

hipError_t launch_gemv(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int ws_stride,
                       const float* bias, int64_t M, int64_t N, int64_t K, void* Y, sq_dtype ydt, int32_t* acc_out,
                       const SideArgs* side, hipStream_t st) {
    (void)side;
    const unsigned blocks = (unsigned)((N + 15) / 16);
    if (ydt == SQ_F16)
        hipLaunchKernelGGL(gemv_i8_kernel<true>, dim3(blocks), dim3(256), 0, st, Xq, xs, Wq, ws, ws_stride, bias,
                           (int)M, (int)N, (int)K, Y, acc_out);
    else
        hipLaunchKernelGGL(gemv_i8_kernel<false>, dim3(blocks), dim3(256), 0, st, Xq, xs, Wq, ws, ws_stride, bias,
                           (int)M, (int)N, (int)K, Y, acc_out);
    return hipGetLastError();
}

}  // namespace sq
