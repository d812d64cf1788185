/*
 * qw_oracle.c -- CPU oracle for the weight-quantized decode linear (W4A8 and W8A16).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow statement of what the
 * GPU path must compute.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no source, header, table or helper with
 * the HIP library, and the HIP library never calls it.
 *
 * Sources (cited by page title and section):
 *  [P1] "Jetson Orin AGX 上的 INT4 量化推理实践：从 9 tok/s 到 19.6 tok/s"
 *       - section 当前实现方式 (current implementation): weights are quantized row-wise
 *         to INT4 at load time, one scale per row, weight ~= int4 * weight_scale;
 *         before every linear the activation is quantized dynamically to INT8,
 *         activation ~= int8 * activation_scale; the output is
 *         int32_accumulate * weight_scale * activation_scale.
 *       - section 正确方向 (the right direction): int8 x int8 products accumulated
 *         in int32 (the DP4A dot); INT4 values widened to int8 lanes.
 *       - section 问题原因 (cause of the problem): the unpack step sign-extends the
 *         nibble, so nibbles hold two's-complement values.
 *  [P3] IntAttention (CSDN summary of the MLSys 2026 paper): IndexSoftmax, section
 *       基准/方法设计 (clipping, LUT exponent, integer normalisation) and section
 *       方法细节 (the all-integer attention data flow).
 *  [P2] ChatGLM2-6B W8A16 deployment on BM1684X (TPU-MLIR write-up)
 *       - section 2 量化方案 (quantization scheme): linear weights stored per-channel
 *         as INT8 and dequantized back to F16 at compute time.
 *       - section 3 TPU-MLIR实现: the scale vector is stored as f16.
 *       - section 4 后端性能提升原理: the W8A16 matmul loads INT8, casts to F16,
 *         multiplies by the scale (dequantize), then multiplies with the activation.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - "row" is an output row n of W[N][K] (the [out, in] layout of a linear layer).
 *  - INT4 scale = maxabs/7 and INT8 scale = maxabs/127, symmetric, fp32 division,
 *    round half to even (rintf under the default rounding mode), then clamp to
 *    +-7 / +-127.  A row whose scale is 0 gets all-zero codes.
 *  - Canonical INT4 packing: byte j of a row = low nibble k=2j, high nibble k=2j+1.
 *  - The activation scale is per row m of X (per vector).
 *  - Epilogue order: ((float)acc * w_scale[n]) * a_scale[m].
 *  - Group-wise INT4 (listed by [P1] 后续优化方向 as future work, with no formula):
 *    one fp32 scale per output row and group of g consecutive k, the row-wise
 *    rule inside each group; per-group int32 dots scaled and summed in fp32 in
 *    group order, then multiplied by the activation scale.
 *  - W8A16: the fp32 scale is rounded to an f16 scale, and the codes are computed
 *    against that stored f16 scale.
 *
 * Compile with gcc -O2 -fno-fast-math -ffp-contract=off (SSE arithmetic, no x87).
 * Precision: the quantization decisions are taken in fp32 (the precision of the
 * kernel); the W8A16 reference product is taken in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { QWO_OK = 0, QWO_ERR_ARG = 1, QWO_ERR_NONFINITE = 2 };

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32, written from the format's definition          */
/* (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits).             */
/* gcc 11 on x86 has no _Float16, so the conversion is spelled out here.     */
/* ------------------------------------------------------------------------ */

float qwo_f32_from_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                  /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);      /* (1 + f/1024) * 2^(e-15) */
    return (float)(sign ? -v : v);
}

uint16_t qwo_f16_from_f32(float x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs((double)x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7e00u);
    /* The largest finite half is 65504; the midpoint to the next binade step is
       65520, and a tie there rounds to the even neighbour, which is infinity. */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00u);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = m * 2^-24, m rounded half to even.  m == 1024
           is the smallest normal, whose bit pattern is 0x0400 = 1024. */
        double m = nearbyint(a / ldexp(1.0, -24));
        return (uint16_t)(sign | (uint16_t)m);
    }
    int e;
    frexp(a, &e);               /* a = fr * 2^e, fr in [0.5, 1): a in [2^(e-1), 2^e) */
    int ue = e - 1;             /* unbiased exponent, -14 .. 15 */
    double m = nearbyint(a / ldexp(1.0, ue - 10));   /* 1024 .. 2048 */
    if (m == 2048.0) {
        m = 1024.0;
        ue += 1;
    }
    if (ue > 15)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)((ue + 15) << 10) | (uint16_t)(m - 1024.0));
}

/* Bulk helpers for the tests (exhaustive checks of the two conversions). */
void qwo_f16_from_f32_n(const float* x, int64_t n, uint16_t* h)
{
    for (int64_t i = 0; i < n; ++i)
        h[i] = qwo_f16_from_f32(x[i]);
}

void qwo_f32_from_f16_n(const uint16_t* h, int64_t n, float* x)
{
    for (int64_t i = 0; i < n; ++i)
        x[i] = qwo_f32_from_f16(h[i]);
}

/* ------------------------------------------------------------------------ */
/* Symmetric quantization of one vector                                     */
/* ------------------------------------------------------------------------ */

static float maxabs_f32(const float* v, int64_t n)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > m)
            m = a;
    }
    return m;
}

static int all_finite(const float* v, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(v[i]))
            return 0;
    return 1;
}

/* code = clamp(rint(v / scale), -qmax, qmax); scale == 0 gives 0. */
static int8_t quant_one(float v, float scale, int qmax)
{
    if (scale == 0.0f)
        return 0;
    float t = v / scale;          /* correctly rounded fp32 division */
    float r = rintf(t);           /* round half to even */
    if (r > (float)qmax)
        r = (float)qmax;
    if (r < (float)-qmax)
        r = (float)-qmax;
    return (int8_t)r;
}

/* ------------------------------------------------------------------------ */
/* [P1] 当前实现方式: row-wise INT4 weight quantization at load time.         */
/* W is [N][K] fp32; q receives [N][K] int8 codes in -7..7; s receives [N].   */
/* ------------------------------------------------------------------------ */
int qwo_quant_w4(const float* W, int64_t N, int64_t K, int8_t* q, float* s)
{
    if (N < 0 || K < 0)
        return QWO_ERR_ARG;
    for (int64_t n = 0; n < N; ++n) {
        const float* row = W + n * K;
        if (!all_finite(row, K))
            return QWO_ERR_NONFINITE;
        float sc = maxabs_f32(row, K) / 7.0f;
        s[n] = sc;
        for (int64_t k = 0; k < K; ++k)
            q[n * K + k] = quant_one(row[k], sc, 7);
    }
    return QWO_OK;
}

/* Canonical INT4 packing: two 4-bit two's-complement codes per byte, the even k
   in the low nibble.  K must be even.  packed is [N][K/2]. */
int qwo_pack_w4(const int8_t* q, int64_t N, int64_t K, uint8_t* packed)
{
    if (N < 0 || K < 0 || (K & 1))
        return QWO_ERR_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t lo = (uint8_t)(q[n * K + 2 * j] & 0x0f);
            uint8_t hi = (uint8_t)(q[n * K + 2 * j + 1] & 0x0f);
            packed[n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
    return QWO_OK;
}

/* Inverse of qwo_pack_w4: nibbles are sign-extended ([P1] 问题原因 lists the
   sign extension among the per-weight unpack steps). */
int qwo_unpack_w4(const uint8_t* packed, int64_t N, int64_t K, int8_t* q)
{
    if (N < 0 || K < 0 || (K & 1))
        return QWO_ERR_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            uint8_t b = packed[n * (K / 2) + j];
            int lo = b & 0x0f;
            int hi = (b >> 4) & 0x0f;
            q[n * K + 2 * j] = (int8_t)(lo >= 8 ? lo - 16 : lo);
            q[n * K + 2 * j + 1] = (int8_t)(hi >= 8 ? hi - 16 : hi);
        }
    return QWO_OK;
}

/* ------------------------------------------------------------------------ */
/* [P1] 当前实现方式: dynamic INT8 activation quantization before each linear. */
/* X is [M][K] fp32; xq receives [M][K] int8 in -127..127; a receives [M].    */
/* ------------------------------------------------------------------------ */
int qwo_quant_act_i8(const float* X, int64_t M, int64_t K, int8_t* xq, float* a)
{
    if (M < 0 || K < 0)
        return QWO_ERR_ARG;
    for (int64_t m = 0; m < M; ++m) {
        const float* row = X + m * K;
        if (!all_finite(row, K))
            return QWO_ERR_NONFINITE;
        float sc = maxabs_f32(row, K) / 127.0f;
        a[m] = sc;
        for (int64_t k = 0; k < K; ++k)
            xq[m * K + k] = quant_one(row[k], sc, 127);
    }
    return QWO_OK;
}

/* ------------------------------------------------------------------------ */
/* [P1] 正确方向 + 当前实现方式: W4A8 linear.                                 */
/*   xq, a  = quant_act_i8(X)                                               */
/*   acc[m][n] = sum_k q[n][k] * xq[m][k]          (int32, exact)            */
/*   Y[m][n]   = ((float)acc * s[n]) * a[m]                                  */
/* q is the [N][K] int8 code matrix (unpacked).  acc may be NULL.            */
/* nthreads > 1 spreads output elements over threads; every element's sum    */
/* is sequential over k, so the result does not depend on the thread count. */
/* ------------------------------------------------------------------------ */
int qwo_gemv_w4a8(const float* X, const int8_t* q, const float* s, int64_t M, int64_t N,
                  int64_t K, float* Y, int32_t* acc, int8_t* xq, float* a, int nthreads)
{
    int st = qwo_quant_act_i8(X, M, K, xq, a);
    if (st != QWO_OK)
        return st;
    if (nthreads < 1)
        nthreads = 1;
    int64_t total = M * N;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        int32_t sum = 0;
        for (int64_t k = 0; k < K; ++k)
            sum += (int32_t)q[n * K + k] * (int32_t)xq[m * K + k];
        if (acc)
            acc[m * N + n] = sum;
        Y[m * N + n] = ((float)sum * s[n]) * a[m];
    }
    return QWO_OK;
}

/* ------------------------------------------------------------------------ */
/* [P1] 后续优化方向 (follow-up work) lists trying a group-wise scale.  Reading  */
/* (the page gives no formula): one fp32 scale per output row n and per group */
/* t of g consecutive k (K a multiple of g), the row-wise rule applied inside */
/* each group:                                                                */
/*   s[n][t] = maxabs(W[n][t*g .. t*g+g-1]) / 7                               */
/*   q[n][k] = clamp(rint(W[n][k] / s[n][k / g]), -7, 7)                      */
/* s is [N][K/g].  With g == K this is qwo_quant_w4.                          */
/* ------------------------------------------------------------------------ */
int qwo_quant_w4g(const float* W, int64_t N, int64_t K, int64_t g, int8_t* q, float* s)
{
    if (N < 0 || K < 0 || g <= 0 || K % g != 0)
        return QWO_ERR_ARG;
    const int64_t G = K / g;
    for (int64_t n = 0; n < N; ++n) {
        const float* row = W + n * K;
        if (!all_finite(row, K))
            return QWO_ERR_NONFINITE;
        for (int64_t t = 0; t < G; ++t) {
            float sc = maxabs_f32(row + t * g, g) / 7.0f;
            s[n * G + t] = sc;
            for (int64_t k = t * g; k < (t + 1) * g; ++k)
                q[n * K + k] = quant_one(row[k], sc, 7);
        }
    }
    return QWO_OK;
}

/* ------------------------------------------------------------------------ */
/* Group-wise W4A8 linear (the same reading): the activation quantization of  */
/* [P1] 当前实现方式, an exact int32 dot per group,                            */
/*   acc[m][n][t] = sum_{k in group t} q[n][k] * xq[m][k],                     */
/* each scaled by its group scale and added in fp32, group by group:          */
/*   y = 0;  for t = 0 .. G-1:  y = y + (float)acc[m][n][t] * s[n][t]         */
/*   Y[m][n] = y * a[m]                                                        */
/* With one group (g == K), 0 + x == x makes this qwo_gemv_w4a8 bit for bit.  */
/* accg ([M][N][K/g]) may be NULL.  Each output element is summed in order on */
/* one thread, so the result does not depend on the thread count.             */
/* ------------------------------------------------------------------------ */
int qwo_gemv_w4a8g(const float* X, const int8_t* q, const float* s, int64_t M, int64_t N,
                   int64_t K, int64_t g, float* Y, int32_t* accg, int8_t* xq, float* a,
                   int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || g <= 0 || K % g != 0)
        return QWO_ERR_ARG;
    int st = qwo_quant_act_i8(X, M, K, xq, a);
    if (st != QWO_OK)
        return st;
    if (nthreads < 1)
        nthreads = 1;
    const int64_t G = K / g;
    int64_t total = M * N;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        float y = 0.0f;
        for (int64_t t = 0; t < G; ++t) {
            int32_t sum = 0;
            for (int64_t k = t * g; k < (t + 1) * g; ++k)
                sum += (int32_t)q[n * K + k] * (int32_t)xq[m * K + k];
            if (accg)
                accg[(m * N + n) * G + t] = sum;
            y = y + (float)sum * s[n * G + t];
        }
        Y[m * N + n] = y * a[m];
    }
    return QWO_OK;
}

/* ------------------------------------------------------------------------ */
/* [P2] 2 量化方案 / 3 TPU-MLIR实现: per-output-channel INT8 weights with an  */
/* f16 scale vector.  s32 = maxabs/127 (fp32), s16 = f16(s32); codes are      */
/* taken against the stored f16 scale so that weight ~= q * s16 is exactly   */
/* what the matmul uses.  A row whose s16 is 0 gets all-zero codes; a row    */
/* whose s16 overflows f16 is rejected.                                      */
/* ------------------------------------------------------------------------ */
int qwo_quant_w8(const float* W, int64_t N, int64_t K, int8_t* q, uint16_t* s16)
{
    if (N < 0 || K < 0)
        return QWO_ERR_ARG;
    for (int64_t n = 0; n < N; ++n) {
        const float* row = W + n * K;
        if (!all_finite(row, K))
            return QWO_ERR_NONFINITE;
        float s32 = maxabs_f32(row, K) / 127.0f;
        uint16_t h = qwo_f16_from_f32(s32);
        float sf = qwo_f32_from_f16(h);
        if (isinf(sf))
            return QWO_ERR_NONFINITE;
        s16[n] = h;
        for (int64_t k = 0; k < K; ++k)
            q[n * K + k] = quant_one(row[k], sf, 127);
    }
    return QWO_OK;
}

/* ------------------------------------------------------------------------ */
/* [P2] 4 后端性能提升原理: W8A16 matmul, taken literally in fp64:            */
/*   cast the INT8 weight, multiply by its scale (dequantize), then multiply */
/*   with the f16 activation and accumulate.                                 */
/*   Y64[m][n] = sum_k (q[n][k] * s16[n]) * x16[m][k]                        */
/* X16 is [M][K] f16 bits, q [N][K] int8, s16 [N] f16 bits; Y64 [M][N].       */
/* ------------------------------------------------------------------------ */
int qwo_gemv_w8a16_ref64(const uint16_t* X16, const int8_t* q, const uint16_t* s16, int64_t M,
                         int64_t N, int64_t K, double* Y64, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return QWO_ERR_ARG;
    if (nthreads < 1)
        nthreads = 1;
    int64_t total = M * N;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        double sn = (double)qwo_f32_from_f16(s16[n]);
        double sum = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double w = (double)q[n * K + k] * sn;                 /* dequantize */
            sum += w * (double)qwo_f32_from_f16(X16[m * K + k]);  /* matmul */
        }
        Y64[m * N + n] = sum;
    }
    return QWO_OK;
}

/* ------------------------------------------------------------------------ */
/* [P1] 速度结果 (speed results) times an FP16 baseline and a weight-only INT4  */
/* path beside W4A8.  The two ablations, as this library reads them:           */
/*                                                                            */
/* FP16 GEMV: weights and activations in f16, no quantization, as an fp64      */
/*   value: Y64[m][n] = sum_k (double)w16[n][k] * (double)x16[m][k].            */
/* ------------------------------------------------------------------------ */
int qwo_gemv_f16_ref64(const uint16_t* X16, const uint16_t* W16, int64_t M, int64_t N,
                       int64_t K, double* Y64, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return QWO_ERR_ARG;
    if (nthreads < 1)
        nthreads = 1;
    int64_t total = M * N;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        double sum = 0.0;
        for (int64_t k = 0; k < K; ++k)
            sum += (double)qwo_f32_from_f16(W16[n * K + k]) * (double)qwo_f32_from_f16(X16[m * K + k]);
        Y64[m * N + n] = sum;
    }
    return QWO_OK;
}

/* Weight-only INT4 with float activations ([P1] 最初的问题 and 问题原因: the INT4   */
/* weight is unpacked in the kernel, sign-extended, converted to float and used  */
/* in a float FMA; the activation stays float).  Row-wise INT4 codes and scales  */
/* as qwo_quant_w4; the row scale multiplies the finished sum (it factors out):  */
/*   y = 0;  for k: y = fmaf((float)q[n][k], x[m][k], y);   Y[m][n] = y * s[n]  */
/* and Y64[m][n] = sum_k ((double)q[n][k] * s[n]) * x[m][k] in fp64.  Y64 may be  */
/* NULL.                                                                         */
int qwo_gemv_w4f32(const float* X, const int8_t* q, const float* s, int64_t M, int64_t N,
                   int64_t K, float* Y, double* Y64, int nthreads)
{
    if (M < 0 || N < 0 || K < 0)
        return QWO_ERR_ARG;
    if (nthreads < 1)
        nthreads = 1;
    int64_t total = M * N;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t i = 0; i < total; ++i) {
        int64_t m = i / N, n = i % N;
        float y = 0.0f;
        double y64 = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            y = fmaf((float)q[n * K + k], X[m * K + k], y);
            y64 += ((double)q[n * K + k] * (double)s[n]) * (double)X[m * K + k];
        }
        Y[m * N + n] = y * s[n];
        if (Y64)
            Y64[m * N + n] = y64;
    }
    return QWO_OK;
}

/* ------------------------------------------------------------------------ */
/* [P3] IntAttention (CSDN summary of the MLSys 2026 paper), 基准/方法设计:      */
/* IndexSoftmax, an integer replacement of softmax over int32 logits, in three */
/* steps per row of the logit matrix A (int32, from an INT8 QK^T):             */
/*  1. clipping (机制一):  D = rowMax(A) - A;  D' = min(D, c_int), with          */
/*     c_int = round(c * sqrt(d) / (s_Q * s_K)) fixed per tensor pair;          */
/*  2. LUT exponent (机制二):  idx = round(D' * (2^b - 1) / c_int);             */
/*     E = LUT[idx], LUT[i] = round(255 * exp(-c * i / (2^b - 1))), the last     */
/*     entry forced to 0 (a 2^b-entry UINT8 table; (b, c) = (5, 6.6));          */
/*  3. integer normalisation (机制三):  rowSum = sum E (32-bit);                 */
/*     P = round(255 * E / rowSum), UINT8.                                       */
/* Readings (the page writes the rounding as a bracket only): every rounding of */
/* a non-negative ratio is half up, done in integers: round(x / y) =            */
/* (2x + y) / (2y); the table rounds to nearest (round()).  c_int must be >= 1. */
/* ------------------------------------------------------------------------ */
int qwo_index_lut(int b, double c, uint8_t* lut)
{
    if (b < 1 || b > 8 || !(c > 0.0))
        return QWO_ERR_ARG;
    const int n = (1 << b) - 1;
    for (int i = 0; i < n; ++i)
        lut[i] = (uint8_t)round(255.0 * exp(-c * (double)i / (double)n));
    lut[n] = 0;
    return QWO_OK;
}

int32_t qwo_index_cint(double c, int d, double s_q, double s_k)
{
    return (int32_t)llround(c * sqrt((double)d) / (s_q * s_k));
}

int qwo_index_softmax(const int32_t* A, int64_t rows, int64_t L, int32_t c_int, int b,
                      const uint8_t* lut, uint8_t* P, int32_t* rowsum, int nthreads)
{
    if (rows < 0 || L < 1 || c_int < 1 || b < 1 || b > 8)
        return QWO_ERR_ARG;
    if (nthreads < 1)
        nthreads = 1;
    const int64_t n = (1 << b) - 1;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const int32_t* a = A + r * L;
        int32_t mx = a[0];
        for (int64_t j = 1; j < L; ++j)
            if (a[j] > mx)
                mx = a[j];
        int64_t sum = 0;
        for (int64_t j = 0; j < L; ++j) {
            int64_t dl = (int64_t)mx - (int64_t)a[j];
            if (dl > c_int)
                dl = c_int;
            const int64_t idx = (2 * dl * n + c_int) / (2 * (int64_t)c_int);
            sum += lut[idx];
        }
        if (rowsum)
            rowsum[r] = (int32_t)sum;
        for (int64_t j = 0; j < L; ++j) {
            int64_t dl = (int64_t)mx - (int64_t)a[j];
            if (dl > c_int)
                dl = c_int;
            const int64_t idx = (2 * dl * n + c_int) / (2 * (int64_t)c_int);
            P[r * L + j] = (uint8_t)((2 * 255 * (int64_t)lut[idx] + sum) / (2 * sum));
        }
    }
    return QWO_OK;
}

/* [P3] 方法细节 (the full data flow): per-tensor symmetric INT8 Q, K, V            */
/* (scale = maxabs/127, the activation rule of qwo_quant_act_i8 over the whole   */
/* tensor), A = Qq Kq^T in int32, IndexSoftmax with c_int from the scales and d,  */
/* UINT8 P, O_acc = P Vq in int32, O = O_acc * s_V / 255.  One head: Q [Lq][d],   */
/* K and V [Lk][d].  Outputs A [Lq][Lk], P [Lq][Lk], O [Lq][d]; *c_int_out.        */
int qwo_int_attention(const float* Q, const float* K, const float* V, int64_t Lq, int64_t Lk,
                      int64_t d, int b, double c, int32_t* A, uint8_t* P, float* O,
                      int32_t* c_int_out)
{
    if (Lq < 1 || Lk < 1 || d < 1)
        return QWO_ERR_ARG;
    int8_t* q = (int8_t*)malloc((size_t)(Lq * d));
    int8_t* k = (int8_t*)malloc((size_t)(Lk * d));
    int8_t* v = (int8_t*)malloc((size_t)(Lk * d));
    int st = QWO_ERR_ARG;
    float sq, sk, sv;
    uint8_t lut[256];
    if (!q || !k || !v)
        goto done;
    if ((st = qwo_quant_act_i8(Q, 1, Lq * d, q, &sq)) != QWO_OK ||
        (st = qwo_quant_act_i8(K, 1, Lk * d, k, &sk)) != QWO_OK ||
        (st = qwo_quant_act_i8(V, 1, Lk * d, v, &sv)) != QWO_OK)
        goto done;
    st = QWO_ERR_ARG;
    if (!(sq > 0.0f) || !(sk > 0.0f))
        goto done;
    for (int64_t i = 0; i < Lq; ++i)
        for (int64_t j = 0; j < Lk; ++j) {
            int32_t acc = 0;
            for (int64_t t = 0; t < d; ++t)
                acc += (int32_t)q[i * d + t] * (int32_t)k[j * d + t];
            A[i * Lk + j] = acc;
        }
    const int32_t ci = qwo_index_cint(c, (int)d, sq, sk);
    *c_int_out = ci;
    if (ci < 1 || qwo_index_lut(b, c, lut) != QWO_OK)
        goto done;
    if ((st = qwo_index_softmax(A, Lq, Lk, ci, b, lut, P, NULL, 1)) != QWO_OK)
        goto done;
    for (int64_t i = 0; i < Lq; ++i)
        for (int64_t t = 0; t < d; ++t) {
            int32_t acc = 0;
            for (int64_t j = 0; j < Lk; ++j)
                acc += (int32_t)P[i * Lk + j] * (int32_t)v[j * d + t];
            O[i * d + t] = (float)((double)acc * (double)sv / 255.0);
        }
    st = QWO_OK;
done:
    free(q);
    free(k);
    free(v);
    return st;
}

int qwo_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
