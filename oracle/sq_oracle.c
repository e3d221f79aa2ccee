/*
 * CPU oracle for the quantized INT8 linear layer.  TEST INFRASTRUCTURE ONLY:
 * the tests, the smoke check and the benchmark's CPU-baseline leg are the only
 * callers.  The product path never links or calls this file; it shares no
 * code, header, table or constant with the HIP library.
 *
 * Plain C99, built with `gcc -O2 -fopenmp -ffp-contract=off` (no fast-math, so
 * no flush-to-zero and no fused multiply-add).  Every floating-point step below
 * is one IEEE-754 binary32 operation with round-to-nearest-even, except where a
 * comment says fp64.  Integer products are accumulated in int64, exactly.
 *
 * Sources (pages are cited by title and section):
 *  - "量化基础与INT8" (quantization basics notes): symmetric mapping
 *    scale = max|x|/127 and q = round(x/scale) clamped to the int8 range;
 *    per-tensor / per-channel / per-token granularity; the INT8 inference
 *    flow (quantize -> int8 GEMM with int32 accumulation -> dequantize as
 *    acc * x_scale * w_scale), sections "量化粒度", "INT8推理流程",
 *    "量化流程示例".
 *  - "SmoothQuant量化实战：W8A8推理部署与单节点530B模型落地": the smoothing
 *    identity (section 1.3), s_j = max|X_j|^a / max|W_j|^(1-a) (section 2.1),
 *    compute_smooth_scale with the 1e-8 floors (section 3.3), the calibration
 *    running max (section 3.2), the W8A8 forward (section 3.4), bias kept in
 *    floating point (section 4.5).
 *  - the same SmoothQuant page, sections 2.3, 4.2 and 4.5: the per-channel
 *    division by s can be absorbed into the preceding LayerNorm's output.
 *  - "LLM.int8()技术解析：8位量化如何优化大语言模型计算": column-wise absmax,
 *    columns above a threshold handled in fp16, the rest in int8, results
 *    combined (sections 2.1 and 3.1).
 *
 * Readings where the pages leave a step open (all listed in the design notes):
 *  rounding is half-to-even (torch.round in every code sample); quantizing
 *  divides by the scale (not multiply by 127/max); clamp to [-128,127]; an
 *  all-zero row/column gets scale 0 and q = 0; the smoothing factor is
 *  evaluated in fp64 and rounded once to fp32, without the optional
 *  normalisation of section 3.3's sample; the LLM.int8() per-token scale uses
 *  the non-outlier columns only; the int8 and fp16 parts are summed.
 *
 * Dtype codes used by this file only: 0 = float32, 1 = float16 (raw bits).
 */
#include <fenv.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_F32 0
#define ORC_F16 1

/* ------------------------------------------------------------------ */
/* fp16 <-> fp32 conversions, written out from the binary16 format.     */
/* ------------------------------------------------------------------ */

/* Exact widening of an IEEE binary16 bit pattern to binary32. */
float orc_half_to_float(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t expo = (uint32_t)(h >> 10) & 0x1fu;
    uint32_t mant = (uint32_t)h & 0x3ffu;
    float v;
    if (expo == 0) {
        v = (float)mant * 0x1p-24f;              /* subnormal (or zero): mant * 2^-24, exact */
    } else if (expo == 31) {
        v = mant ? NAN : INFINITY;
    } else {
        uint32_t bits = ((expo - 15u + 127u) << 23) | (mant << 13);
        memcpy(&v, &bits, 4);
    }
    return sign ? -v : v;
}

/* binary32 -> binary16, round to nearest, ties to even. */
uint16_t orc_float_to_half(float f)
{
    uint32_t x;
    memcpy(&x, &f, 4);
    uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
    uint32_t ax = x & 0x7fffffffu;
    if (ax > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);   /* NaN */
    if (ax >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);  /* >= 65520 rounds to inf */
    int e = (int)(ax >> 23) - 127;                               /* unbiased exponent */
    if (e >= -14) {                                              /* normal binary16 */
        uint32_t mant = ax & 0x7fffffu;
        uint32_t h = ((uint32_t)(e + 15) << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1fffu;
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;   /* carry into exponent is correct */
        return (uint16_t)(sign | h);
    }
    if (e < -25) return sign;                                    /* below 2^-25: rounds to zero */
    /* subnormal binary16: the result is round(value * 2^24) */
    uint32_t sig = (ax & 0x7fffffu) | 0x800000u;                 /* value = sig * 2^(e-23) */
    int shift = -(e + 1);                                        /* value*2^24 = sig >> shift */
    uint32_t q = sig >> shift;
    uint32_t rem = sig & ((1u << shift) - 1u);
    uint32_t half = 1u << (shift - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
    return (uint16_t)(sign | q);
}

void orc_half_to_float_array(const uint16_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_half_to_float(in[i]);
}

void orc_float_to_half_array(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_float_to_half(in[i]);
}

static float load_elem(const void* p, int dt, int64_t i)
{
    if (dt == ORC_F16) return orc_half_to_float(((const uint16_t*)p)[i]);
    return ((const float*)p)[i];
}

/* round half to even, then clamp to the int8 range */
static int8_t quant_code(float v)
{
    float r = rintf(v);            /* default rounding mode: nearest, ties to even */
    if (r > 127.0f) r = 127.0f;
    if (r < -128.0f) r = -128.0f;
    return (int8_t)r;
}

/* Rounding mode.  Every step above and below assumes round-to-nearest-even, the
 * IEEE default; a caller could have left its thread in another mode.  The Python
 * wrapper brackets every call into this file with these two functions: the first
 * sets nearest-even on the calling thread and on every thread of the OpenMP team
 * and returns the caller's mode, the second restores that mode. */
int orc_rounding_enter(void)
{
    int prev = fegetround();
    fesetround(FE_TONEAREST);
#ifdef _OPENMP
#pragma omp parallel
    fesetround(FE_TONEAREST);
#endif
    return prev;
}

void orc_rounding_leave(int prev)
{
    fesetround(prev);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count for the OpenMP loops that follow (timing only; results do not depend on it). */
void orc_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ */
/* Calibration statistic and smoothing factors (SmoothQuant page,       */
/* sections 2.1, 3.2, 3.3).                                             */
/* ------------------------------------------------------------------ */

/* amax[j] = max(amax[j], max_m |X[m,j]|): the per-input-channel running
 * maximum that the calibration hook accumulates across batches. */
void orc_col_absmax(const void* X, int dt, int64_t M, int64_t K, float* amax)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < K; ++j) {
        float a = amax[j];
        for (int64_t m = 0; m < M; ++m) {
            float v = fabsf(load_elem(X, dt, m * K + j));
            if (v > a) a = v;
        }
        amax[j] = a;
    }
}

/* s_j = max(a_j,1e-8)^alpha / max(w_j,1e-8)^(1-alpha), both powers in fp64,
 * the ratio rounded once to fp32. */
void orc_smooth_from_maxima(const float* act_max, const float* w_max, int64_t K,
                            float alpha, float* s)
{
    double al = (double)alpha;
    for (int64_t j = 0; j < K; ++j) {
        float a = act_max[j] > 1e-8f ? act_max[j] : 1e-8f;
        float w = w_max[j] > 1e-8f ? w_max[j] : 1e-8f;
        s[j] = (float)(pow((double)a, al) / pow((double)w, 1.0 - al));
    }
}

/* Full step a1+a2: update the running activation maximum with a calibration
 * batch (X_cal may be NULL when M_cal == 0), take the column maxima of W over
 * its output rows, and form s. */
void orc_smooth_scales(const void* X_cal, int xdt, int64_t M_cal,
                       const void* W, int wdt, int64_t N, int64_t K,
                       float alpha, float* act_max, float* s)
{
    if (X_cal && M_cal > 0) orc_col_absmax(X_cal, xdt, M_cal, K, act_max);
    float* w_max = (float*)calloc((size_t)K, sizeof(float));
    orc_col_absmax(W, wdt, N, K, w_max);
    orc_smooth_from_maxima(act_max, w_max, K, alpha, s);
    free(w_max);
}

/* ------------------------------------------------------------------ */
/* Weight smoothing and quantization (SmoothQuant page 3.3-3.4; basics  */
/* notes "量化粒度").  gran: 0 = one scale per output row (channel),     */
/* 1 = one scale for the whole tensor.                                  */
/* ------------------------------------------------------------------ */
void orc_quantize_weight(const void* W, int dt, int64_t N, int64_t K, const float* s,
                         int gran, int8_t* Wq, float* w_scale)
{
    float* Ws = (float*)malloc((size_t)(N * K) * sizeof(float));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K; ++j) {
            float w = load_elem(W, dt, n * K + j);
            Ws[n * K + j] = s ? w * s[j] : w;          /* W' = W diag(s): scales input channels */
        }

    if (gran == 0) {
#pragma omp parallel for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            float m = 0.0f;
            for (int64_t j = 0; j < K; ++j) {
                float v = fabsf(Ws[n * K + j]);
                if (v > m) m = v;
            }
            float sc = m / 127.0f;
            w_scale[n] = sc;
            for (int64_t j = 0; j < K; ++j)
                Wq[n * K + j] = sc == 0.0f ? 0 : quant_code(Ws[n * K + j] / sc);
        }
    } else {
        float m = 0.0f;
        for (int64_t i = 0; i < N * K; ++i) {
            float v = fabsf(Ws[i]);
            if (v > m) m = v;
        }
        float sc = m / 127.0f;
        w_scale[0] = sc;
#pragma omp parallel for schedule(static)
        for (int64_t i = 0; i < N * K; ++i)
            Wq[i] = sc == 0.0f ? 0 : quant_code(Ws[i] / sc);
    }
    free(Ws);
}

/* ------------------------------------------------------------------ */
/* Per-token activation quantization with optional smoothing (basics    */
/* notes "量化流程示例"; SmoothQuant page 3.4).  skip (may be NULL) marks */
/* columns excluded from the int8 part (LLM.int8() outliers): they get  */
/* q = 0 and do not enter the row maximum.                              */
/* ------------------------------------------------------------------ */
void orc_quantize_per_token(const void* X, int dt, int64_t M, int64_t K, const float* s,
                            const uint8_t* skip, int8_t* Xq, float* x_scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            if (skip && skip[j]) continue;
            float x = load_elem(X, dt, m * K + j);
            if (s) x = x / s[j];                        /* X' = X diag(s)^-1 */
            float v = fabsf(x);
            if (v > a) a = v;
        }
        float sc = a / 127.0f;
        x_scale[m] = sc;
        for (int64_t j = 0; j < K; ++j) {
            if ((skip && skip[j]) || sc == 0.0f) {
                Xq[m * K + j] = 0;
                continue;
            }
            float x = load_elem(X, dt, m * K + j);
            if (s) x = x / s[j];
            Xq[m * K + j] = quant_code(x / sc);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Asymmetric (zero-point) per-token activation quantization (basics    */
/* notes, 非对称量化: scale = (max - min) / 255, a zero point, codes     */
/* round(x / scale) shifted by it, x ~ scale * (code - zero point)).     */
/*                                                                      */
/* Reading (the page's own formulas mix float and code units): the row  */
/* range is widened to contain 0, lo = min(0, min x'), hi = max(0, max  */
/* x'), so the zero point is a code; scale = fl32(fl32(hi - lo) / 255);  */
/* z = clamp(rne(fl32(-lo / scale)), 0, 255); code u = clamp(rne(fl32(  */
/* x' / scale)) + z, 0, 255).  Stored as int8 q = u - 128 with zero     */
/* point zq = z - 128, so x' ~ scale * (q - zq).  An all-zero row (scale */
/* 0) gets u = z = 0.  x' = fl32(x / s_j) with smoothing, as above.     */
/* ------------------------------------------------------------------ */
void orc_quantize_per_token_asym(const void* X, int dt, int64_t M, int64_t K, const float* s, int8_t* Xq,
                                 float* x_scale, int32_t* x_zero)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float lo = 0.0f, hi = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float x = load_elem(X, dt, m * K + j);
            if (s) x = x / s[j];
            if (x < lo) lo = x;
            if (x > hi) hi = x;
        }
        float sc = (hi - lo) / 255.0f;
        int z = 0;
        if (sc != 0.0f) {
            float zf = rintf(-lo / sc);
            z = zf < 0.0f ? 0 : (zf > 255.0f ? 255 : (int)zf);
        }
        x_scale[m] = sc;
        x_zero[m] = z - 128;
        for (int64_t j = 0; j < K; ++j) {
            int u = 0;
            if (sc != 0.0f) {
                float x = load_elem(X, dt, m * K + j);
                if (s) x = x / s[j];
                u = (int)rintf(x / sc) + z;
                u = u < 0 ? 0 : (u > 255 ? 255 : u);
            }
            Xq[m * K + j] = (int8_t)(u - 128);
        }
    }
}

/* rowsum[n] = sum_k Wq[n,k]: the weight term of the zero-point correction, once per weight. */
void orc_weight_rowsum(const int8_t* Wq, int64_t N, int64_t K, int32_t* rowsum)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        int64_t t = 0;
        for (int64_t k = 0; k < K; ++k) t += Wq[n * K + k];
        rowsum[n] = (int32_t)t;
    }
}

/* The corrected accumulator acc'[m,n] = acc[m,n] - zq[m] * rowsum[n] (the sum of
 * (q - zq) * w over k), in int64 and checked to fit int32 (returns the number that do
 * not), then dequantized like the symmetric accumulator:
 * y = ((float)acc' * x_scale[m]) * w_scale[n or 0] (+ bias[n]).  acc_corr may be NULL. */
int64_t orc_dequant_asym(const int32_t* acc, const float* x_scale, const int32_t* x_zero, const float* w_scale,
                         int wgran, const int32_t* rowsum, const float* bias, int64_t M, int64_t N, float* y,
                         int32_t* acc_corr)
{
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t a = (int64_t)acc[m * N + n] - (int64_t)x_zero[m] * (int64_t)rowsum[n];
            if (a > INT32_MAX || a < INT32_MIN) ++bad;
            if (acc_corr) acc_corr[m * N + n] = (int32_t)a;
            float v = (float)(int32_t)a;
            v = v * x_scale[m];
            v = v * w_scale[wgran == 0 ? n : 0];
            if (bias) v = v + bias[n];
            y[m * N + n] = v;
        }
    return bad;
}

/* ------------------------------------------------------------------ */
/* int8 x int8 -> int32 GEMM, "NT": acc[m,n] = sum_k A[m,k] * B[n,k],  */
/* accumulated in int64 and checked to fit int32 (basics notes          */
/* "INT8推理流程").  Returns the number of results that did not fit.      */
/* ------------------------------------------------------------------ */
int64_t orc_gemm_i8(const int8_t* A, const int8_t* B, int64_t M, int64_t N, int64_t K,
                    int32_t* acc)
{
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t t = 0;
            for (int64_t k = 0; k < K; ++k) t += (int64_t)A[m * K + k] * (int64_t)B[n * K + k];
            if (t > INT32_MAX || t < INT32_MIN) ++bad;
            acc[m * N + n] = (int32_t)t;
        }
    return bad;
}

/* The same dot products at nsamp given (row, col) positions. */
int64_t orc_gemm_i8_sampled(const int8_t* A, const int8_t* B, int64_t K, const int64_t* rows,
                            const int64_t* cols, int64_t nsamp, int32_t* out)
{
    int64_t bad = 0;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i < nsamp; ++i) {
        int64_t t = 0;
        const int8_t* a = A + rows[i] * K;
        const int8_t* b = B + cols[i] * K;
        for (int64_t k = 0; k < K; ++k) t += (int64_t)a[k] * (int64_t)b[k];
        if (t > INT32_MAX || t < INT32_MIN) ++bad;
        out[i] = (int32_t)t;
    }
    return bad;
}

/* ------------------------------------------------------------------ */
/* Dequantization: y = ((float)acc * x_scale[m]) * w_scale[n or 0],    */
/* left to right, then + bias[n] (bias stays floating point, SmoothQuant */
/* page 4.5).  Writes fp32.                                              */
/* ------------------------------------------------------------------ */
static float dequant_one(int32_t acc, float xs, float ws, const float* bias, int64_t n)
{
    float y = (float)acc;          /* int32 -> fp32, nearest-even (exact below 2^24) */
    y = y * xs;
    y = y * ws;
    if (bias) y = y + bias[n];
    return y;
}

void orc_dequant(const int32_t* acc, const float* x_scale, const float* w_scale, int wgran,
                 const float* bias, int64_t M, int64_t N, float* y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = dequant_one(acc[m * N + n], x_scale[m], w_scale[wgran == 0 ? n : 0], bias, n);
}

void orc_dequant_sampled(const int32_t* acc, const float* x_scale, const float* w_scale, int wgran,
                         const float* bias, const int64_t* rows, const int64_t* cols, int64_t nsamp,
                         float* y)
{
    for (int64_t i = 0; i < nsamp; ++i)
        y[i] = dequant_one(acc[i], x_scale[rows[i]], w_scale[wgran == 0 ? cols[i] : 0], bias, cols[i]);
}

/* ------------------------------------------------------------------ */
/* LLM.int8() pieces (LLM.int8() page, sections 2.1 and 3.1).           */
/* ------------------------------------------------------------------ */

/* Column j is an outlier when max_m |X[m,j]| > threshold (strictly).
 * Writes mask[K] (0/1), the ascending index list idx[0..count) and returns count. */
int64_t orc_outlier_columns(const uint16_t* X16, int64_t M, int64_t K, float threshold,
                            uint8_t* mask, int32_t* idx)
{
    float* cmax = (float*)calloc((size_t)K, sizeof(float));
    orc_col_absmax(X16, ORC_F16, M, K, cmax);
    int64_t count = 0;
    for (int64_t j = 0; j < K; ++j) {
        mask[j] = cmax[j] > threshold ? 1 : 0;
        if (mask[j]) idx[count++] = (int32_t)j;
    }
    free(cmax);
    return count;
}

/* side[i] = sum over the listed columns t of X[row,t] * W16[col,t], in fp64,
 * at the given (row, col) positions (pass rows/cols covering a full matrix for
 * a dense result). */
void orc_side_product_sampled(const uint16_t* X16, const uint16_t* W16, int64_t K,
                              const int32_t* idx, int64_t count, const int64_t* rows,
                              const int64_t* cols, int64_t nsamp, double* side)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nsamp; ++i) {
        double t = 0.0;
        for (int64_t c = 0; c < count; ++c) {
            int64_t j = idx[c];
            t += (double)orc_half_to_float(X16[rows[i] * K + j]) *
                 (double)orc_half_to_float(W16[cols[i] * K + j]);
        }
        side[i] = t;
    }
}

/* out = fp16( fp32( (double)y_int8 + side ) ) */
void orc_combine_to_half(const float* y_int8, const double* side, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_float_to_half((float)((double)y_int8[i] + side[i]));
}

/* ------------------------------------------------------------------ */
/* LayerNorm with the smoothing folded in, then per-token quantization  */
/* (SmoothQuant page, sections 2.3, 4.2 and 4.5: the per-channel        */
/* division X/s is absorbed into the preceding LayerNorm's output).     */
/*                                                                      */
/* Reading (the pages give no LayerNorm precision): binary16 inputs     */
/* only.  Each finite x is n * 2^-24 with an integer n (|n| < 2^40), so  */
/* the row sums S1 = sum n and S2 = sum n^2 are exact integers and the   */
/* statistics do not depend on summation order:                         */
/*   mu   = fl64( fl64(S1) / (K * 2^24) )                               */
/*   var  = fl64( fl64(K*S2 - S1^2) / (K^2 * 2^48) )   (population var) */
/*   rstd = fl64( 1 / fl64(sqrt( fl64(var + eps) )) )                    */
/*   z_j  = fl32( fl32(x_j - fl32(mu)) * fl32(rstd) )                    */
/*   y_j  = fl32( fl32(z_j * g_j) + b_j )   (no add when there is no b)  */
/* with g = gamma/s and b = beta/s folded offline, each one fl32 divide. */
/* ------------------------------------------------------------------ */

/* the integer n with x = n * 2^-24 for a finite binary16 x */
static int64_t half_to_int24(uint16_t h)
{
    int64_t e = (h >> 10) & 0x1f, m = h & 0x3ff;
    int64_t n = e ? (1024 + m) << (e - 1) : m;
    return (h & 0x8000u) ? -n : n;
}

void orc_layernorm_stats(const uint16_t* X, int64_t M, int64_t K, float eps, float* mu32, float* rstd32,
                         double* mu64, double* var64)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        int64_t s1 = 0;
        __int128 s2 = 0;
        for (int64_t j = 0; j < K; ++j) {
            int64_t n = half_to_int24(X[m * K + j]);
            s1 += n;
            s2 += (__int128)n * n;
        }
        __int128 v = (__int128)K * s2 - (__int128)s1 * s1;        /* K^2 times the variance, scaled */
        double mu = (double)s1 / ((double)K * 0x1p24);
        double var = (double)v / (((double)K * (double)K) * 0x1p48);
        double rstd = 1.0 / sqrt(var + (double)eps);
        mu32[m] = (float)mu;
        rstd32[m] = (float)rstd;
        if (mu64) mu64[m] = mu;
        if (var64) var64[m] = var;
    }
}

/* y = LayerNorm output with the folded weights, fp32 [M x K]; beta may be NULL */
void orc_layernorm(const uint16_t* X, int64_t M, int64_t K, const float* gamma, const float* beta, float eps,
                   float* Y)
{
    float* mu = (float*)malloc((size_t)M * sizeof(float));
    float* r = (float*)malloc((size_t)M * sizeof(float));
    orc_layernorm_stats(X, M, K, eps, mu, r, NULL, NULL);
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < K; ++j) {
            float x = orc_half_to_float(X[m * K + j]);
            float z = (x - mu[m]) * r[m];
            float y = z * gamma[j];
            if (beta) y = y + beta[j];
            Y[m * K + j] = y;
        }
    free(mu);
    free(r);
}

/* The fused step: LayerNorm (folded weights), then per-token quantization of
 * its fp32 output with no smoothing (the smoothing is inside gamma and beta). */
void orc_layernorm_quantize(const uint16_t* X, int64_t M, int64_t K, const float* gamma, const float* beta,
                            float eps, int8_t* Xq, float* x_scale)
{
    float* Y = (float*)malloc((size_t)(M * K) * sizeof(float));
    orc_layernorm(X, M, K, gamma, beta, eps, Y);
    orc_quantize_per_token(Y, ORC_F32, M, K, NULL, NULL, Xq, x_scale);
    free(Y);
}

/* Offline fold: gamma' = fl32(gamma / s), beta' = fl32(beta / s) per input channel. */
void orc_fold_layernorm(const float* gamma, const float* beta, const float* s, int64_t K, float* gamma_out,
                        float* beta_out)
{
    for (int64_t j = 0; j < K; ++j) {
        gamma_out[j] = gamma[j] / s[j];
        if (beta) beta_out[j] = beta[j] / s[j];
    }
}

/* ------------------------------------------------------------------ */
/* Static per-tensor activation scale from calibration data, and        */
/* quantization with it (basics notes, 静态量化: activation ranges are  */
/* precomputed on a calibration set; the deployment page's calibrator  */
/* takes a percentile (99.99) of the activation distribution).          */
/*                                                                      */
/* Reading: the statistic is the nearest-rank percentile of |x'| over   */
/* every calibration element, x' = fl32(x / s_j) (or x without s): the  */
/* value at 1-based rank r = ceil(p * n / 100) (fp64 expression,        */
/* clamped to [1, n]) in ascending order, so p = 100 is the maximum.    */
/* The scale is fl32(T / 127); quantizing divides by it and clamps, so  */
/* values beyond T saturate at 127 / -128.                              */
/* ------------------------------------------------------------------ */
static int cmp_float(const void* a, const void* b)
{
    float x = *(const float*)a, y = *(const float*)b;
    return (x > y) - (x < y);
}

int64_t orc_percentile_rank(int64_t n, double p)
{
    int64_t r = (int64_t)ceil(p * (double)n / 100.0);
    if (r < 1) r = 1;
    if (r > n) r = n;
    return r;
}

float orc_abs_percentile(const void* X, int dt, int64_t M, int64_t K, const float* s, double p)
{
    int64_t n = M * K;
    float* v = (float*)malloc((size_t)n * sizeof(float));
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < K; ++j) {
            float x = load_elem(X, dt, m * K + j);
            if (s) x = x / s[j];
            v[m * K + j] = fabsf(x);
        }
    qsort(v, (size_t)n, sizeof(float), cmp_float);
    float t = v[orc_percentile_rank(n, p) - 1];
    free(v);
    return t;
}

float orc_static_scale(const void* X, int dt, int64_t M, int64_t K, const float* s, double p)
{
    return orc_abs_percentile(X, dt, M, K, s, p) / 127.0f;
}

void orc_quantize_static(const void* X, int dt, int64_t M, int64_t K, const float* s, float xs, int8_t* Xq)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < K; ++j) {
            float x = load_elem(X, dt, m * K + j);
            if (s) x = x / s[j];
            Xq[m * K + j] = xs == 0.0f ? 0 : quant_code(x / xs);
        }
}

/* ------------------------------------------------------------------ */
/* INT8 KV cache with per-head scales (SmoothQuant page, section 5.2:  */
/* the KV cache is quantized to INT8 with one scale per head, since the */
/* heads' distributions differ; as the cache grows, a scale from the    */
/* calibration stage with a safety factor avoids recomputing it).       */
/*                                                                      */
/* Layout [T x H x D] row-major (tokens, heads, head dim).              */
/*   scale_h = fl32( fl32(margin * max_{t,d} |x[t,h,d]|) / 127 )         */
/*   q = clamp(rne(fl32(x / scale_h)), -128, 127)   (0 when scale_h = 0) */
/* Dequantization, general: y[m,j] = fl32(q[m,j] * scale[m*rs + j/g])     */
/* (rs = 0, g = D: per head over [T x H*D]; rs = 1, g = K: per row).     */
/* ------------------------------------------------------------------ */
void orc_kv_calibrate_per_head(const void* KV, int dt, int64_t T, int64_t H, int64_t D, float margin,
                               float* scale)
{
    for (int64_t h = 0; h < H; ++h) {
        float m = 0.0f;
        for (int64_t t = 0; t < T; ++t)
            for (int64_t d = 0; d < D; ++d) {
                float v = fabsf(load_elem(KV, dt, (t * H + h) * D + d));
                if (v > m) m = v;
            }
        scale[h] = (margin * m) / 127.0f;
    }
}

void orc_kv_quantize_per_head(const void* KV, int dt, int64_t T, int64_t H, int64_t D, const float* scale,
                              int8_t* q)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d) {
                int64_t i = (t * H + h) * D + d;
                float x = load_elem(KV, dt, i);
                q[i] = scale[h] == 0.0f ? 0 : quant_code(x / scale[h]);
            }
}

/* y = fl32(q * scale[m*row_stride + j/group]), fp32 out (the caller rounds to fp16) */
void orc_dequantize(const int8_t* q, int64_t M, int64_t K, const float* scale, int64_t row_stride,
                    int64_t group, float* y)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < K; ++j)
            y[m * K + j] = (float)q[m * K + j] * scale[m * row_stride + j / group];
}

/* ------------------------------------------------------------------ */
/* FP8 W8A8 variant (SmoothQuant page, section 6.1: W8A8 in FP8 on      */
/* hardware with FP8 matrix units).  The same flow with the 8-bit code  */
/* switched from int8 to FP8 E4M3 (OCP "e4m3fn": 1 sign bit, 4 exponent */
/* bits with bias 7, 3 mantissa bits, no infinities; largest finite     */
/* value 448, smallest subnormal 2^-9):                                 */
/*   scale = fl32(max|x'| / 448); code = e4m3(clamp(fl32(x' / scale),   */
/*   -448, 448)), rounded to nearest, ties to even; scale 0 -> code 0.  */
/* ------------------------------------------------------------------ */

/* binary32 -> e4m3fn, round to nearest even; |v| above 448 saturates to 448
 * (the quantizer's clamp).  Finite inputs only. */
uint8_t orc_fp8_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80u : 0x00u;
    double a = fabs((double)v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7eu);              /* 448 = 1.110b * 2^8 */
    if (a < 0x1p-6) {
        /* subnormal range: multiples of 2^-9; code = the multiple (8 = 2^-6 is the
         * first normal, whose code is also 8) */
        double q = nearbyint(a * 512.0);                         /* exact scaling; ties to even */
        return (uint8_t)(sign | (uint8_t)q);
    }
    int e;
    double f = frexp(a, &e);                                     /* a = f * 2^e, f in [0.5, 1) */
    int E = e - 1;                                               /* a = (2f) * 2^E, 2f in [1, 2) */
    double r = nearbyint((2.0 * f - 1.0) * 8.0);                 /* 3-bit mantissa, ties to even */
    if (r == 8.0) {
        r = 0.0;
        E += 1;
    }
    return (uint8_t)(sign | (uint8_t)(((E + 7) << 3) | (int)r));
}

float orc_fp8_decode(uint8_t c)
{
    int s = c >> 7, E = (c >> 3) & 15, m = c & 7;
    float v;
    if (E == 15 && m == 7) v = NAN;
    else if (E == 0) v = (float)m * 0x1p-9f;
    else v = ldexpf(1.0f + (float)m / 8.0f, E - 7);
    return s ? -v : v;
}

void orc_fp8_encode_array(const float* in, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_encode(in[i]);
}

void orc_fp8_decode_array(const uint8_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_fp8_decode(in[i]);
}

static uint8_t fp8_code_of(float x, float sc)
{
    if (sc == 0.0f) return 0;
    float v = x / sc;
    if (v > 448.0f) v = 448.0f;
    if (v < -448.0f) v = -448.0f;
    return orc_fp8_encode(v);
}

/* Per-row FP8 quantization of X [M x K]: mode 0 x' = x, mode 1 x' = fl32(x / s_j)
 * (activations, smoothing), mode 2 x' = fl32(x * s_j) (weight rows, smoothed). */
void orc_fp8_quantize_rows(const void* X, int dt, int64_t M, int64_t K, const float* s, int mode,
                           uint8_t* q, float* scale)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float a = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float x = load_elem(X, dt, m * K + j);
            if (mode == 1) x = x / s[j];
            if (mode == 2) x = x * s[j];
            float v = fabsf(x);
            if (v > a) a = v;
        }
        float sc = a / 448.0f;
        scale[m] = sc;
        for (int64_t j = 0; j < K; ++j) {
            float x = load_elem(X, dt, m * K + j);
            if (mode == 1) x = x / s[j];
            if (mode == 2) x = x * s[j];
            q[m * K + j] = fp8_code_of(x, sc);
        }
    }
}

/* Per-tensor FP8 weight quantization: one scale fl32(max|W'| / 448). */
void orc_fp8_quantize_tensor(const void* W, int dt, int64_t N, int64_t K, const float* s, uint8_t* q,
                             float* scale)
{
    float a = 0.0f;
    for (int64_t i = 0; i < N * K; ++i) {
        float w = load_elem(W, dt, i);
        if (s) w = w * s[i % K];
        float v = fabsf(w);
        if (v > a) a = v;
    }
    float sc = a / 448.0f;
    scale[0] = sc;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < N * K; ++i) {
        float w = load_elem(W, dt, i);
        if (s) w = w * s[i % K];
        q[i] = fp8_code_of(w, sc);
    }
}

/* Every finite e4m3 value is an integer multiple of 2^-9 with |n| <= 448 * 2^9 < 2^18,
 * so a product is n_a n_b 2^-18 with |n_a n_b| < 2^36, and a sum of K <= 131071 such
 * products is an integer below 2^53: accumulated in int64 it is exact, and so is its
 * conversion to fp64. */
static int64_t fp8_units(uint8_t c)
{
    int E = (c >> 3) & 15, m = c & 7;
    int64_t n = E == 0 ? m : (int64_t)(8 + m) << (E - 1);      /* value * 2^9 */
    return (c & 0x80u) ? -n : n;
}

/* Exact FP8 "NT" GEMM: acc[m,n] = sum_k A[m,k] B[n,k] (fp64, exact); abs_sum (may be
 * NULL) receives sum_k |A[m,k] B[n,k]|, for error bounds of inexact accumulations. */
void orc_gemm_fp8(const uint8_t* A, const uint8_t* B, int64_t M, int64_t N, int64_t K, double* acc,
                  double* abs_sum)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t t = 0, u = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t p = fp8_units(A[m * K + k]) * fp8_units(B[n * K + k]);
                t += p;
                u += p < 0 ? -p : p;
            }
            acc[m * N + n] = ldexp((double)t, -18);
            if (abs_sum) abs_sum[m * N + n] = ldexp((double)u, -18);
        }
}

void orc_gemm_fp8_sampled(const uint8_t* A, const uint8_t* B, int64_t K, const int64_t* rows,
                          const int64_t* cols, int64_t nsamp, double* acc, double* abs_sum)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nsamp; ++i) {
        int64_t t = 0, u = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t p = fp8_units(A[rows[i] * K + k]) * fp8_units(B[cols[i] * K + k]);
            t += p;
            u += p < 0 ? -p : p;
        }
        acc[i] = ldexp((double)t, -18);
        if (abs_sum) abs_sum[i] = ldexp((double)u, -18);
    }
}

/* FP8 dequantization: y = ((float)acc * x_scale[m]) * w_scale[n or 0] (+ bias[n]), with
 * the exact accumulator rounded once to fp32 (a matrix unit accumulates in fp32). */
void orc_fp8_dequant(const double* acc, const float* x_scale, const float* w_scale, int wgran,
                     const float* bias, const int64_t* rows, const int64_t* cols, int64_t nsamp, float* y)
{
    for (int64_t i = 0; i < nsamp; ++i) {
        float v = (float)acc[i];
        v = v * x_scale[rows[i]];
        v = v * w_scale[wgran == 0 ? cols[i] : 0];
        if (bias) v = v + bias[cols[i]];
        y[i] = v;
    }
}
