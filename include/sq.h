/*
 * sq.h -- C ABI of the MI355X (gfx950) quantized INT8 linear layer.
 *
 * The layer computes Y = X W^T for X [M x K] (tokens x in_features) and
 * W [N x K] (out_features x in_features, the PyTorch Linear layout) through
 *   1. SmoothQuant smoothing X diag(s)^-1 and diag(s) W, with
 *      s_j = max|X_j|^alpha / max|W_j|^(1-alpha)
 *      ("SmoothQuant量化实战：W8A8推理部署与单节点530B模型落地", sections 1.3, 2.1, 3.3);
 *   2. symmetric absmax int8 quantization, scale = max|x|/127, q = round(x/scale)
 *      clamped to [-128, 127]: per token (row) for activations, per output
 *      channel or per tensor for weights ("量化基础与INT8", sections 量化粒度 and
 *      量化流程示例);
 *   3. an int8 x int8 -> int32 GEMM ("量化基础与INT8", section INT8推理流程);
 *   4. the dequantizing epilogue Y = acc * x_scale * w_scale (+ bias), stored as
 *      fp16 or fp32 (same section; bias kept in floating point: SmoothQuant page,
 *      section 4.5);
 * and the LLM.int8() variant, where activation columns whose absolute maximum
 * exceeds a threshold bypass int8 and are multiplied in fp16, the two partial
 * products being summed ("LLM.int8()技术解析：8位量化如何优化大语言模型计算",
 * sections 2.1 and 3.1).
 *
 * Numerics, common to all entry points:
 *  - every floating-point step is one IEEE binary32 operation, round to nearest
 *    even; rounding to an integer code is half-to-even; fp16 inputs are widened
 *    exactly; fp16 outputs are rounded to nearest even.
 *  - quantizing divides by the scale; a row (or tensor) whose absolute maximum
 *    is 0 gets scale 0 and all-zero codes.
 *  - int32 accumulation is exact for K <= 131071 (|acc| <= 127^2 K < 2^31).
 *  The int8 codes, the scales and the int32 accumulators are therefore fully
 *  determined by the inputs.
 *
 * Conventions, common to all entry points:
 *  - Ownership: the caller allocates and owns every buffer; the library never
 *    allocates, frees, copies device-to-host or synchronizes.
 *  - Pointers marked "device" are HIP device pointers; all are 16-byte aligned,
 *    dense, row-major, and outputs do not alias inputs.
 *  - Streams: every call enqueues its kernels on `stream` (NULL = the default
 *    stream) and returns without waiting.
 *  - Errors: arguments are validated on the host before anything is enqueued;
 *    on a non-zero status nothing was enqueued, except SQ_ERR_HIP, which
 *    reports a failed launch (kernels enqueued before it may run).  Faults
 *    inside kernels surface at the caller's next synchronization, as in HIP.
 *    Inputs must be finite (NaN/Inf give unspecified codes).
 *  - Sizes: M, N >= 1; 16 <= K <= 131056 and K % 16 == 0.
 *  - Codes: dtype arguments (xdt, wdt, ydt, dt) are int holding an sq_dtype value and
 *    granularity arguments (g) an sq_wgran value; any other value returns SQ_ERR_DTYPE.
 *  - Thread safety: calls are reentrant; calls that share output or workspace
 *    buffers must be ordered by the caller (same stream or events).
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle (the same declaration as in the HIP headers). */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
    SQ_OK = 0,
    SQ_ERR_NULL = 1,      /* a required pointer is NULL */
    SQ_ERR_SHAPE = 2,     /* M, N or K out of range, or K % 16 != 0 */
    SQ_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
    SQ_ERR_DTYPE = 4,     /* unsupported dtype or granularity code */
    SQ_ERR_VALUE = 5,     /* alpha outside [0,1], threshold negative or NaN, eps not finite and > 0,
                             percentile outside (0, 100] */
    SQ_ERR_WORKSPACE = 6, /* workspace missing or smaller than sq_workspace_size() */
    SQ_ERR_HIP = 7        /* a HIP launch or device query failed */
} sq_status;

typedef enum { SQ_F32 = 0, SQ_F16 = 1 } sq_dtype;            /* passed as int */
typedef enum { SQ_PER_CHANNEL = 0, SQ_PER_TENSOR = 1 } sq_wgran;  /* passed as int */
typedef enum { SQ_OP_QUANT_WEIGHT = 0, SQ_OP_OUTLIER = 1, SQ_OP_CALIB_STATIC = 2, SQ_OP_LINEAR = 3 } sq_op;

/* Static, human-readable name of a status code. */
const char* sq_status_string(int st);

/* Bytes of device workspace an entry point needs.
 *   SQ_OP_QUANT_WEIGHT: for sq_quantize_weight (M ignored).
 *   SQ_OP_OUTLIER:      for int8_outlier_matmul; sized for the worst case of
 *                       all K columns being outliers: an M * K * 2 fp16 panel of outlier
 *                       activations, M * K int8 codes, 4 * M scales, 12 * K bytes of
 *                       column data and a 16-byte count, each region rounded up to 256
 *                       bytes (under 2 KB of padding in total).
 *   SQ_OP_CALIB_STATIC: for sq_calibrate_static_scale (N ignored): 8448 bytes.
 *   SQ_OP_LINEAR:       for sq_w8a8_linear: M * K and 4 * M bytes, each rounded up to 256.
 * Returns 0 for an unknown op or sizes out of range. */
size_t sq_workspace_size(int op, int64_t M, int64_t N, int64_t K);

/* Calibration and smoothing factors (offline).
 * [SmoothQuant page, section 3.2: running per-channel max of the activations;
 *  section 3.3: compute_smooth_scale with both maxima floored at 1e-8;
 *  section 2.1: s_j = max|X_j|^alpha / max|W_j|^(1-alpha).]
 *   X_cal   device, [M_cal x K] in xdt; may be NULL when M_cal == 0.
 *   act_max device, float [K], in/out: act_max[j] = max(act_max[j], max_m |X_cal[m,j]|).
 *           Start it at zeros; call once per calibration batch.
 *   W       device, [N x K] in wdt.  If W == NULL only act_max is updated and s may be NULL.
 *   s       device, float [K], out:
 *           s_j = (float)( pow((double)max(act_max_j,1e-8f), alpha)
 *                        / pow((double)max(max_n |W[n,j]|, 1e-8f), 1 - alpha) ),
 *           pow in fp64 (the device and host pow may differ in the last fp32 ulp).
 *   alpha   in [0, 1].
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_VALUE, SQ_ERR_HIP. */
sq_status sq_smooth_scales(const void* X_cal, int xdt, int64_t M_cal,
                           const void* W, int wdt, int64_t N, int64_t K, float alpha,
                           float* act_max, float* s, hipStream_t stream);

/* Fused smoothing + dynamic per-token activation quantization (every forward).
 * [basics notes, 量化流程示例: per-row absmax scale, round, clamp;
 *  SmoothQuant page, sections 3.3-3.4: X' = X / s before quantizing.]
 *   X       device, [M x K] in xdt (fp16 or fp32).
 *   s       device, float [K], or NULL for no smoothing.
 *   Xq      device, int8 [M x K], out: clamp(rne(fl32(x'_j / xs)), -128, 127),
 *           x'_j = fl32(x_j / s_j) (x_j when s == NULL).
 *   x_scale device, float [M], out: xs = fl32(max_j |x'_j| / 127).
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_HIP. */
sq_status sq_quantize_per_token(const void* X, int xdt, int64_t M, int64_t K,
                                const float* s, int8_t* Xq, float* x_scale, hipStream_t stream);

/* Weight smoothing + quantization (offline).
 * [SmoothQuant page, section 3.3: W' = W * s along in_features;
 *  basics notes, 量化粒度: per-tensor or per-output-channel absmax scales.]
 *   W       device, [N x K] in wdt.
 *   s       device, float [K], or NULL for no smoothing: W'[n,j] = fl32(W[n,j] * s_j).
 *   g       SQ_PER_CHANNEL: w_scale[n] = fl32(max_j |W'[n,j]| / 127), float [N];
 *           SQ_PER_TENSOR:  w_scale[0] = fl32(max_{n,j} |W'| / 127), float [1].
 *   Wq      device, int8 [N x K], out: clamp(rne(fl32(W' / w_scale)), -128, 127).
 *   ws      device workspace of ws_bytes >= sq_workspace_size(SQ_OP_QUANT_WEIGHT, 0, N, K)
 *           (only SQ_PER_TENSOR uses it; may be NULL for SQ_PER_CHANNEL).
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_WORKSPACE, SQ_ERR_HIP. */
sq_status sq_quantize_weight(const void* W, int wdt, int64_t N, int64_t K, const float* s,
                             int g, int8_t* Wq, float* w_scale, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* int8 GEMM with fused dequantization.
 * [basics notes, INT8推理流程 and 量化流程示例: int32 accumulation, then
 *  acc * X_scale * W_scale; SmoothQuant page, section 3.4 and 4.5: + bias.]
 *   Xq [M x K] int8, x_scale float [M], Wq [N x K] int8, all device.
 *   w_scale float [N] (SQ_PER_CHANNEL) or [1] (SQ_PER_TENSOR), device.
 *   bias    device float [N], or NULL.
 *   acc[m,n] = sum_k Xq[m,k] * Wq[n,k]            (exact int32)
 *   Y[m,n]   = ((fl32(acc) * x_scale[m]) * w_scale[n or 0]) + bias[n],
 *              each step one fp32 operation, stored as ydt (fp16 rounded to nearest even).
 *   Y       device, [M x N] in ydt.
 *   acc_out device int32 [M x N], or NULL; when given, acc is written too (parity checks).
 * M <= 16 runs a weight-streaming decode kernel; larger M the MFMA tile kernel.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_HIP. */
sq_status w8a8_gemm_dequant(const int8_t* Xq, const float* x_scale, const int8_t* Wq,
                            const float* w_scale, int g, const float* bias,
                            int64_t M, int64_t N, int64_t K, void* Y, int ydt,
                            int32_t* acc_out, hipStream_t stream);

/* The whole W8A8 layer for one activation batch: per-token quantization of X (with the
 * smoothing division) and the GEMM with the dequantizing epilogue, in one call.
 * [SmoothQuant page, section 3.4: the forward of the quantized linear layer, scaling,
 *  quantization, INT8 GEMM and dequantization.]
 *   X, xdt, M, K, s  as for sq_quantize_per_token;  Wq, w_scale, g, bias, N, Y, ydt as
 *                    for w8a8_gemm_dequant.
 *   x_scale  device float [M] or NULL: receives the per-token scales.
 *   ws       device workspace >= sq_workspace_size(SQ_OP_LINEAR, M, N, K) (holds Xq; the
 *            decode case below leaves it untouched).
 * Results are bit-identical to sq_quantize_per_token followed by w8a8_gemm_dequant.
 * With fp16 X, M <= 2 and K <= 8192 (decode) one kernel does both: every block of the
 * weight-streaming kernel quantizes the activation rows in its prologue.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_WORKSPACE, SQ_ERR_HIP. */
sq_status sq_w8a8_linear(const void* X, int xdt, int64_t M, int64_t K, const float* s,
                         const int8_t* Wq, const float* w_scale, int g, const float* bias,
                         int64_t N, void* Y, int ydt, float* x_scale, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/* Limits of sq_w8a8_linear_noalloc's built-in scratch. */
#define SQ_NOALLOC_XQ_BYTES ((size_t)16 << 20) /* int8 activation codes: M * K <= 16 MiB */
#define SQ_NOALLOC_MAX_M 16384                 /* per-token scales held there when x_scale is NULL */

/* sq_w8a8_linear without a workspace, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It calls no allocating routine.  The int8 activation codes (and the per-token scales
 * when x_scale is NULL) go to a fixed array in the library's device memory,
 * SQ_NOALLOC_XQ_BYTES + 4 * SQ_NOALLOC_MAX_M bytes (16.06 MiB), which each GPU the
 * library runs on holds until the process ends.
 *   Arguments and results as for sq_w8a8_linear, without ws and ws_bytes; the outputs are
 *   bit-identical to sq_w8a8_linear's.
 *   Limits: M * K <= SQ_NOALLOC_XQ_BYTES, and M <= SQ_NOALLOC_MAX_M when x_scale is NULL;
 *   larger inputs return SQ_ERR_WORKSPACE before anything is enqueued (use sq_w8a8_linear).
 *   Every call on one GPU shares that GPU's array, which keeps the last call's contents
 *   (nothing in it needs to start at zero): calls that can overlap on one GPU (streams
 *   not ordered against each other, or several host threads) race on it, and the caller
 *   must order them.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_WORKSPACE, SQ_ERR_HIP. */
sq_status sq_w8a8_linear_noalloc(const void* X, int xdt, int64_t M, int64_t K, const float* s,
                                 const int8_t* Wq, const float* w_scale, int g, const float* bias,
                                 int64_t N, void* Y, int ydt, float* x_scale, hipStream_t stream);

/* LLM.int8() linear layer (no smoothing).
 * [LLM.int8() page, section 2.1: column-wise absmax of the input, columns above
 *  the threshold are outliers; section 3.1: bitmask of outlier columns, int8 GEMM
 *  over the normal columns, fp16 GEMM over the outlier columns, results combined.]
 *   X        device fp16 [M x K];  W16 device fp16 [N x K] (the unquantized weight).
 *   Wq, w_scale  device, from sq_quantize_weight(W16, s = NULL, SQ_PER_CHANNEL).
 *   bias     device float [N], or NULL.
 *   threshold >= 0: column j is an outlier iff max_m |X[m,j]| > threshold.
 *   The int8 part quantizes each row over its non-outlier columns only (outlier
 *   columns get code 0 and stay out of the row maximum), then runs the int8 GEMM
 *   and the dequant epilogue (+ bias).  The side part is
 *   side[m,n] = sum over outlier j of X[m,j] * W16[n,j] (fp16 products, fp32 sum).
 *   Y[m,n] = fp16(y_int8[m,n] + side[m,n]).   Y: device fp16 [M x N].
 *   ws, ws_bytes  device workspace >= sq_workspace_size(SQ_OP_OUTLIER, M, N, K).
 *   n_outliers    device int32 [1] or NULL: receives the number of outlier columns.
 *   outlier_idx   device int32 [K] or NULL: receives them in ascending order.
 *   acc_out       device int32 [M x N] or NULL: the int8 part's accumulators.
 * The outlier count stays on the device; no host synchronization happens.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_VALUE, SQ_ERR_WORKSPACE, SQ_ERR_HIP. */
sq_status int8_outlier_matmul(const void* X, const void* W16, const int8_t* Wq,
                              const float* w_scale, const float* bias,
                              int64_t M, int64_t N, int64_t K, float threshold, void* Y,
                              void* ws, size_t ws_bytes, int32_t* n_outliers,
                              int32_t* outlier_idx, int32_t* acc_out, hipStream_t stream);

/* Offline fold of the smoothing into the preceding LayerNorm's weights.
 * [SmoothQuant page, section 2.3: the per-channel division of the activations
 *  can be merged into the previous layer; section 4.2: absorb the scaling into
 *  the preceding operation's output, e.g. the LayerNorm; section 4.5: with the
 *  LayerNorm before the Linear the scaling costs nothing extra.]
 *   gamma, s   device float [K];  beta device float [K] or NULL.
 *   gamma_out  device float [K], out: fl32(gamma[j] / s[j]).
 *   beta_out   device float [K], out: fl32(beta[j] / s[j]); NULL exactly when beta is NULL.
 * LayerNorm(x; gamma_out, beta_out) is then LayerNorm(x; gamma, beta) / s per channel.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE (K as above), SQ_ERR_ALIGN, SQ_ERR_HIP. */
sq_status sq_fold_smoothing_layernorm(const float* gamma, const float* beta, const float* s,
                                      int64_t K, float* gamma_out, float* beta_out,
                                      hipStream_t stream);

/* LayerNorm (folded weights) fused with per-token quantization (every forward):
 * the smoothed activation of step 1 comes straight out of the LayerNorm and is
 * quantized as in sq_quantize_per_token with s = NULL.
 * [SmoothQuant page, sections 2.3, 4.2 and 4.5, as for the fold above.]
 *   X        device, fp16 [M x K] (xdt must be SQ_F16).
 *   gamma    device float [K], beta device float [K] or NULL (from the fold).
 *   eps      finite, > 0.
 *   Row statistics are exact: each x is n * 2^-24 for an integer n, and
 *     mu   = fl64(fl64(S1) / (K 2^24)),  S1 = sum n (exact);
 *     var  = fl64(fl64(K S2 - S1^2) / (K^2 2^48)),  S2 = sum n^2 (exact);
 *     rstd = fl64(1 / fl64(sqrt(fl64(var + eps))));
 *   then per element, in binary32: z = (x - fl32(mu)) * fl32(rstd),
 *   y = z * gamma[j] (+ beta[j]).
 *   Xq       device int8 [M x K], out: clamp(rne(fl32(y / xs)), -128, 127).
 *   x_scale  device float [M], out: xs = fl32(max_j |y_j| / 127) (0 and all-zero codes when y == 0).
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_VALUE, SQ_ERR_HIP. */
sq_status sq_layernorm_quantize_per_token(const void* X, int xdt, int64_t M, int64_t K,
                                          const float* gamma, const float* beta, float eps,
                                          int8_t* Xq, float* x_scale, hipStream_t stream);

/* Static per-tensor activation scale from a calibration batch (offline).
 * [basics notes, 静态量化: activation ranges are precomputed on a calibration
 *  set; the deployment page's calibration flow uses a percentile calibrator
 *  (percentile 99.99) over the collected activations.]
 *   X_cal      device, [M_cal x K] in xdt (M_cal * K < 2^32).
 *   s          device float [K] (smoothing, x' = fl32(x / s_j)) or NULL (x' = x).
 *   percentile in (0, 100]: T = the value at 1-based rank r = ceil(percentile * n / 100)
 *              (fp64 expression, clamped to [1, n]) among the n = M_cal * K values |x'|
 *              in ascending order (nearest rank; 100 gives the maximum).
 *   x_scale    device float [1], out: fl32(T / 127).
 *   ws         device workspace >= sq_workspace_size(SQ_OP_CALIB_STATIC, M_cal, 0, K).
 * The rank is found by an exact radix select on the device (no host synchronization).
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_VALUE, SQ_ERR_WORKSPACE, SQ_ERR_HIP. */
sq_status sq_calibrate_static_scale(const void* X_cal, int xdt, int64_t M_cal, int64_t K,
                                    const float* s, double percentile, float* x_scale,
                                    void* ws, size_t ws_bytes, hipStream_t stream);

/* Activation quantization with a static (calibrated) per-tensor scale (every forward).
 * [basics notes, 静态量化; with the scale fixed there is no per-token maximum to take.]
 *   X        device, [M x K] in xdt;  s device float [K] or NULL, as in sq_quantize_per_token.
 *   x_scale  device float [1]: the calibrated scale xs (e.g. from sq_calibrate_static_scale).
 *   Xq       device int8 [M x K], out: clamp(rne(fl32(x'_j / xs)), -128, 127) (0 when xs == 0);
 *            values beyond the calibrated range saturate.
 *   x_scale_rows  device float [M] or NULL: when given, every entry is set to xs, so the
 *            codes feed w8a8_gemm_dequant unchanged.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_HIP. */
sq_status sq_quantize_static(const void* X, int xdt, int64_t M, int64_t K, const float* s,
                             const float* x_scale, int8_t* Xq, float* x_scale_rows, hipStream_t stream);

/* Zero-point (asymmetric) activation variant.
 * [basics notes, 非对称量化: scale from the range, (max - min) / 255, and a zero point, so
 *  that a range that is not centred on 0 uses all 256 codes; the dequantized value is
 *  scale * (code - zero point).  The page's own formulas mix float and code units; the
 *  reading taken: the row range is widened to contain 0, so the zero point is a code.]
 * Per-token activation codes:
 *   X, s, M, K as for sq_quantize_per_token (x' = fl32(x / s_j) with s, else x).
 *   x_scale  device float [M], out: sc = fl32(fl32(hi - lo) / 255) with lo = min(0, min_j x'_j),
 *            hi = max(0, max_j x'_j) (0 for an all-zero row).
 *   x_zero   device int32 [M], out: z - 128 with z = clamp(rne(fl32(-lo / sc)), 0, 255) (z = 0 when sc == 0).
 *   Xq       device int8 [M x K], out: u - 128 with u = clamp(rne(fl32(x'_j / sc)) + z, 0, 255)
 *            (u = 0 when sc == 0), so x'_j ~ sc * (Xq - x_zero).
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_HIP. */
sq_status sq_quantize_per_token_asym(const void* X, int xdt, int64_t M, int64_t K, const float* s,
                                     int8_t* Xq, float* x_scale, int32_t* x_zero, hipStream_t stream);

/* Row sums of the quantized weight, rowsum[n] = sum_k Wq[n,k] (offline, once per weight):
 * the weight term of the zero-point correction.
 *   Wq      device int8 [N x K];  rowsum  device int32 [N], out.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_HIP. */
sq_status sq_weight_rowsum(const int8_t* Wq, int64_t N, int64_t K, int32_t* rowsum, hipStream_t stream);

/* int8 GEMM with zero-point activations and the dequantizing epilogue (any M):
 *   acc'[m,n] = sum_k Xq[m,k] Wq[n,k] - x_zero[m] * w_rowsum[n]  (= sum_k (Xq - x_zero) Wq),
 *   exact int32 when it fits int32;  y = ((float)acc' * x_scale[m]) * w_scale[n or 0] (+ bias[n]),
 *   fp32 steps, stored as ydt.  x_zero and w_rowsum come from sq_quantize_per_token_asym and
 *   sq_weight_rowsum; other arguments as for w8a8_gemm_dequant; acc_out (device int32
 *   [M x N] or NULL) receives acc'.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_HIP. */
sq_status w8a8_asym_gemm_dequant(const int8_t* Xq, const float* x_scale, const int32_t* x_zero, const int8_t* Wq,
                                 const float* w_scale, int g, const int32_t* w_rowsum, const float* bias, int64_t M,
                                 int64_t N, int64_t K, void* Y, int ydt, int32_t* acc_out, hipStream_t stream);

/* FP8 W8A8 variant: FP8 E4M3 codes (OCP "e4m3fn": bias 7, 3 mantissa bits, largest
 * finite 448, smallest subnormal 2^-9, no infinities; byte = sign | exponent | mantissa).
 * [SmoothQuant page, section 6.1: W8A8 in FP8 is the scheme to prefer on hardware
 *  with FP8 matrix units; the flow is the int8 one with the 8-bit code changed.]
 * Per-token activation codes:
 *   X, s, M, K as for sq_quantize_per_token.
 *   x_scale  device float [M], out: xs = fl32(max_j |x'_j| / 448) (0 for an all-zero row).
 *   Xq       device uint8 [M x K], out: e4m3(clamp(fl32(x'_j / xs), -448, 448)), nearest even
 *            (0x00 when xs == 0; -0 codes as 0x80).
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_HIP. */
sq_status sq_quantize_per_token_fp8(const void* X, int xdt, int64_t M, int64_t K, const float* s,
                                    uint8_t* Xq, float* x_scale, hipStream_t stream);

/* FP8 E4M3 weight codes of W' = fl32(W * s_j) (or W), per output channel (w_scale [N]) or
 * per tensor (w_scale [1], workspace as for sq_quantize_weight): scale = fl32(max|W'| / 448),
 * codes as in sq_quantize_per_token_fp8.  Arguments as for sq_quantize_weight.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_WORKSPACE, SQ_ERR_HIP. */
sq_status sq_quantize_weight_fp8(const void* W, int wdt, int64_t N, int64_t K, const float* s,
                                 int g, uint8_t* Wq, float* w_scale, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* FP8 E4M3 GEMM with the dequantizing epilogue (any M; gfx950 FP8 matrix instructions):
 *   acc[m,n] = sum_k dec(Xq[m,k]) dec(Wq[n,k]), accumulated in fp32 (the products are
 *   exact; the order of the fp32 additions is the hardware's, so acc is within
 *   gamma_K * sum_k |products| of the exact sum, gamma_K = K 2^-24 / (1 - K 2^-24));
 *   y = ((acc * x_scale[m]) * w_scale[n or 0]) (+ bias[n]), fp32 steps, stored as ydt.
 *   Other arguments as for w8a8_gemm_dequant; acc_out (device float [M x N] or NULL)
 *   receives the fp32 accumulators.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_HIP. */
sq_status fp8_gemm_dequant(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                           int g, const float* bias, int64_t M, int64_t N, int64_t K, void* Y,
                           int ydt, float* acc_out, hipStream_t stream);

/* INT8 KV cache, per-head calibration (offline or at cache creation).
 * [SmoothQuant page, section 5.2: the KV cache is stored as int8 with one scale per
 *  attention head, the heads' ranges being different; a scale fixed from calibration
 *  and widened by a safety factor avoids recomputing it while the cache grows.]
 *   KV      device, [T x H x D] in dt (tokens x heads x head_dim), row-major.
 *   T >= 1, H >= 1, 16 <= D, D % 16 == 0, H * D <= 131056.
 *   margin  finite, > 0: the safety factor.
 *   scale   device float [H], out: scale_h = fl32(fl32(margin * max_{t,d} |x[t,h,d]|) / 127)
 *           (0 for a head that is all zero).
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_VALUE, SQ_ERR_HIP. */
sq_status sq_kv_calibrate_per_head(const void* KV, int dt, int64_t T, int64_t H, int64_t D,
                                   float margin, float* scale, hipStream_t stream);

/* INT8 KV cache, quantization with fixed per-head scales (every appended block).
 * [SmoothQuant page, section 5.2.]
 *   KV      device, [T x H x D] in dt; sizes as for sq_kv_calibrate_per_head.
 *   scale   device float [H] (e.g. from sq_kv_calibrate_per_head).
 *   q       device int8 [T x H x D], out: clamp(rne(fl32(x[t,h,d] / scale_h)), -128, 127)
 *           (0 when scale_h == 0); values beyond the calibrated range saturate.
 *   To append T new tokens to a cache of capacity C, pass q + t0 * H * D.
 *   Per-token (per row and head) scales instead: sq_quantize_per_token on the
 *   [T*H x D] view, whose row scales are the per-token-per-head scales.
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_HIP. */
sq_status sq_kv_quantize_per_head(const void* KV, int dt, int64_t T, int64_t H, int64_t D,
                                  const float* scale, int8_t* q, hipStream_t stream);

/* Dequantization of int8 codes with grouped scales (reading an INT8 KV cache back).
 * ["量化基础与INT8", section 量化流程示例: x ~ q * scale.]
 *   q        device int8 [M x K] (16 <= K <= 131056, K % 16 == 0).
 *   scale    device float, 4-byte aligned; element (m, j) uses
 *            scale[m * scale_row_stride + j / group]:
 *              per head of a [T x H*D] cache:  scale_row_stride 0, group D;
 *              one scale per row:              scale_row_stride 1, group K;
 *              per token and head:             scale_row_stride K / group, group D.
 *   group    >= 16, group % 16 == 0, K % group == 0;  0 <= scale_row_stride <= 131056.
 *   Y        device [M x K] in ydt, out: fl32(q * scale) (rounded to nearest even for fp16).
 * Errors: SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_ALIGN, SQ_ERR_DTYPE, SQ_ERR_HIP. */
sq_status sq_dequantize(const int8_t* q, int64_t M, int64_t K, const float* scale, int64_t scale_row_stride,
                        int64_t group, void* Y, int ydt, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SQ_H */
