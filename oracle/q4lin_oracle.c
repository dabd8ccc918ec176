/*
 * q4lin_oracle.c -- plain CPU reference for the Q4_G64_FP16 pure Linear op.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no code, header or constant table with the HIP
 * library.
 *
 * What it computes (the plain definition, written out):
 *   Y[n,t] = bf16_rne( sum_k  W[n,k] * X[k,t] )
 * where W[n,k] = (q[n,k] - 8) * scale[n, k/64]  (q a 4-bit code in 0..15),
 * the sum is taken in IEEE binary64 in increasing k, and the result is rounded
 * once, directly from binary64 to bfloat16 with round-to-nearest-even.
 *
 * Sources (the pages' text):
 *  - "q4-linear.md" (NInferEZ-Engine maintainer example), setup table: W is
 *    Q4_G64_FP16 with a row-split layout, 64 weights share one FP16 scale;
 *    the math shape is W[N,K] x X[K,T] -> Y[N,T]; BF16 input and output.
 *  - same page, test paragraph: the check decodes the packed codes and FP16
 *    scales independently and uses an FP64 matrix product as the oracle.
 *  - "linear-benchmark.md", section 4 (theoretical traffic), weight-format
 *    table: a Q4G64_F16S group is 64 weights = 32 code bytes + 2 scale bytes,
 *    34 bytes per group, weight bytes = groups * 34.
 * Readings where the pages are silent (each listed in the design notes):
 *  - code -> value is (q - 8) * scale;
 *  - nibble order: byte j of a row holds k = 2j in its low nibble and
 *    k = 2j+1 in its high nibble;
 *  - planes: codes[N][K/2] row-major, scales[N][K/64] row-major (fp16 bits);
 *  - X and Y are token-major: X(k,t) at x[t*K + k], Y(n,t) at y[t*N + n].
 *
 * Exactness: every weight (q-8)*s has at most 15 significant bits and every
 * activation at most 8, so each product is exact in binary64; the binary64
 * running sum has relative error at most about K * 2^-53, far below one bf16
 * ulp, and the single final rounding is correctly rounded.
 *
 * Parity pins live in the CPU test-suite (hand-worked examples, library
 * special cases, invariants, exact rational brute force).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* IEEE binary16 bits -> binary64, decoded by hand (sign, 5-bit exponent with
 * bias 15, 10-bit fraction, subnormals, Inf/NaN). */
double q4o_fp16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);            /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 bits -> binary64, decoded by hand (sign, 8-bit exponent with bias
 * 127, 7-bit fraction, subnormals, Inf/NaN). */
double q4o_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int m = b & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);           /* subnormal: m * 2^-133 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 128), e - 134); /* (1 + m/128) * 2^(e-127) */
    return sign ? -v : v;
}

/* binary64 -> bfloat16 bits, round to nearest, ties to even, done once from
 * the binary64 value (no pass through binary32, which could round twice).
 * bfloat16 keeps 8 significant bits; its quantum in the binade
 * [2^e, 2^(e+1)) is 2^(e-7) for e >= -126 and 2^-133 below (subnormals).
 * Magnitudes that round to 2^128 or more become Inf; NaN stays NaN. */
uint16_t q4o_double_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    if (isnan(v))
        return 0x7FC0;
    double a = fabs(v);
    if (isinf(a))
        return sign | 0x7F80;
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);                 /* a = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;                /* a in [2^e, 2^(e+1)) */
    int qexp = (e < -126) ? -133 : e - 7;
    double r = ldexp(a, -qexp);    /* a / quantum: exact power-of-two scaling */
    double whole = floor(r);
    double frac = r - whole;       /* exact: r has at most 53 significant bits */
    if (frac > 0.5 || (frac == 0.5 && fmod(whole, 2.0) != 0.0))
        whole += 1.0;
    /* whole is an integer in [0, 256]; the value is whole * 2^qexp */
    if (whole == 0.0)
        return sign;
    int exp_field;
    int frac_field;
    if (qexp == -133 && whole < 128.0) {      /* stays subnormal */
        exp_field = 0;
        frac_field = (int)whole;
    } else {
        int w = (int)whole;
        int ee = qexp + 7;                    /* binade of the rounded value */
        if (w == 256) {                       /* rounding carried into the next binade */
            w = 128;
            ee += 1;
        }
        if (ee > 127)
            return sign | 0x7F80;             /* overflow -> Inf */
        exp_field = ee + 127;
        frac_field = w - 128;
    }
    return (uint16_t)(sign | (exp_field << 7) | frac_field);
}

/* Weight bytes of a Q4_G64_FP16 matrix, the pages' closed form
 * ("linear-benchmark.md", section 4): groups * 34 with groups = N * K / 64
 * (K a multiple of 64; every K used here is also a multiple of 128, so the
 * pages' K_pad equals K). */
int64_t q4o_weight_bytes(int64_t n, int64_t k)
{
    return n * (k / 64) * 34;
}

/* One weight value (q - 8) * scale, exact in binary64. */
static double weight_value(const uint8_t *codes, const uint16_t *scales,
                           int64_t K, int64_t n, int64_t k)
{
    uint8_t byte = codes[n * (K / 2) + k / 2];
    int q = (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
    double s = q4o_fp16_to_double(scales[n * (K / 64) + k / 64]);
    return (double)(q - 8) * s;
}

/* The binary64 sum for one output element, increasing k. */
static double dot_one(const uint8_t *codes, const uint16_t *scales,
                      const uint16_t *x, int64_t K, int64_t n, int64_t t)
{
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += weight_value(codes, scales, K, n, k) * q4o_bf16_to_double(x[t * K + k]);
    return acc;
}

/* Full product.  y[t*N + n] receives bf16 bits; acc (optional, may be NULL)
 * receives the unrounded binary64 sums in the same order.  threads <= 0 uses
 * the OpenMP default.  Rows are independent, so the row loop is split across
 * threads; each sum is still taken sequentially in k. */
void q4o_linear(const uint16_t *x, const uint8_t *codes, const uint16_t *scales,
                uint16_t *y, double *acc, int64_t N, int64_t K, int64_t T,
                int threads)
{
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k)
                w[k] = weight_value(codes, scales, K, n, k);
            for (int64_t t = 0; t < T; ++t) {
                double s = 0.0;
                const uint16_t *xt = x + t * K;
                for (int64_t k = 0; k < K; ++k)
                    s += w[k] * q4o_bf16_to_double(xt[k]);
                y[t * N + n] = q4o_double_to_bf16(s);
                if (acc)
                    acc[t * N + n] = s;
            }
        }
        free(w);
    }
}

/* LinearAdd, the pages' fused variant with a residual ("q4-linear.md" and
 * "linear-benchmark.md" name LinearAdd among the Linear variants without
 * defining it; the plain reading taken here):
 *   Y[n,t] = bf16_rne( sum_k W[n,k] * X[k,t]  +  R[n,t] )
 * with R in bf16, token-major like Y (R(n,t) at r[t*N + n]); the residual
 * (exact in binary64) joins the binary64 sum after the last k, and the
 * result is rounded once. */
void q4o_linear_add(const uint16_t *x, const uint8_t *codes, const uint16_t *scales,
                    const uint16_t *r, uint16_t *y, int64_t N, int64_t K, int64_t T,
                    int threads)
{
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k)
                w[k] = weight_value(codes, scales, K, n, k);
            for (int64_t t = 0; t < T; ++t) {
                double s = 0.0;
                const uint16_t *xt = x + t * K;
                for (int64_t k = 0; k < K; ++k)
                    s += w[k] * q4o_bf16_to_double(xt[k]);
                s += q4o_bf16_to_double(r[t * N + n]);
                y[t * N + n] = q4o_double_to_bf16(s);
            }
        }
        free(w);
    }
}

/* LinearSwiGLU, the pages' fused gate/up variant ("q4-linear.md" and
 * "linear-benchmark.md" name LinearSwiGLU among the Linear variants without
 * defining it; the plain reading taken here, the gated linear unit with the
 * SiLU (swish) gate):
 *   Y[n,t] = bf16_rne( silu(G[n,t]) * U[n,t] ),   silu(g) = g / (1 + e^-g)
 * where G and U are the unrounded binary64 sums of the gate and up weights
 * over the same X (q4o_linear's acc).  The gate, its product with U and the
 * single rounding are all taken in binary64 (exp from the C library).
 * g and u hold `count` sums each; y receives `count` bf16 values. */
void q4o_swiglu(const double *g, const double *u, uint16_t *y, int64_t count)
{
    for (int64_t i = 0; i < count; ++i) {
        const double silu = g[i] / (1.0 + exp(-g[i]));
        y[i] = q4o_double_to_bf16(silu * u[i]);
    }
}

/* Selected output elements only: out[i] = Y[ns[i], ts[i]] (bf16 bits), and
 * acc[i] the binary64 sum (acc may be NULL).  Used where the full product
 * would take too long on the CPU. */
void q4o_linear_at(const uint16_t *x, const uint8_t *codes, const uint16_t *scales,
                   int64_t N, int64_t K, int64_t T,
                   const int64_t *ns, const int64_t *ts, int64_t count,
                   uint16_t *out, double *acc, int threads)
{
    (void)N;
    (void)T;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        double s = dot_one(codes, scales, x, K, ns[i], ts[i]);
        out[i] = q4o_double_to_bf16(s);
        if (acc)
            acc[i] = s;
    }
}

/* ------------------------------------------------------------------------
 * The other weight formats of the same pure Linear.
 *
 * "linear-benchmark.md", section 4 (theoretical traffic), weight-format
 * table: Q5G64_F16S (64 weights per group: 32 low-code bytes + 8 high bytes +
 * a 2-byte scale = 42 bytes), Q6G64_F16S (32 + 16 + 2 = 50 bytes per 64),
 * W8G32_F16S (32 weights per group: 32 code bytes + 2 scale bytes = 34),
 * NVFP4 (16 weights per group: 8 code bytes + one E4M3 scale byte = 9) and
 * BF16_CTRL (plain bf16 weights, 2 N K bytes); section 0 lists the formats
 * the A16 Linear takes.  The pages give byte counts only.  Readings taken
 * (the plainest packing that matches those counts):
 *   Q5: q = low nibble | high bit << 4 in 0..31, weight (q - 16) * scale;
 *       low plane [N][K/2] as in Q4 (even k in the low nibble), high plane
 *       [N][K/8]: bit i of byte b is the high bit of k = 8b + i.
 *   Q6: q = low nibble | high pair << 4 in 0..63, weight (q - 32) * scale;
 *       high plane [N][K/4]: bits 2i, 2i+1 of byte b are the high pair of
 *       k = 4b + i.
 *   W8: a two's-complement byte c per weight, plane [N][K], weight c * scale
 *       with scales [N][K/32].
 *   NVFP4: an E2M1 code per weight (plane [N][K/2], even k in the low
 *       nibble), one E4M3 scale byte per 16 weights (plane [N][K/16]),
 *       weight = E2M1 value * E4M3 value (no further tensor-wide scale: the
 *       table counts none).
 *   BF16_CTRL: the weights themselves, bf16 bits [N][K].
 * Every product of a weight and an activation is exact in binary64 (at most
 * 27 significant bits); sums are taken in binary64 in increasing k and
 * rounded once to bf16, as for Q4.
 * ------------------------------------------------------------------------ */
#define Q4O_FMT_Q4 0
#define Q4O_FMT_Q5 1
#define Q4O_FMT_Q6 2
#define Q4O_FMT_W8 3
#define Q4O_FMT_NVFP4 4
#define Q4O_FMT_BF16 5

/* OCP 8-bit floating point E4M3 (the "fn" variant: exponent bias 7, three
 * fraction bits, subnormals, no infinities, S.1111.111 is NaN), decoded by
 * hand. */
double q4o_e4m3_to_double(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xF;
    int m = b & 0x7;
    double v;
    if (e == 15 && m == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)m, -9);           /* subnormal: m/8 * 2^-6 */
    else
        v = ldexp((double)(m + 8), e - 10); /* (1 + m/8) * 2^(e-7) */
    return sign ? -v : v;
}

/* OCP 4-bit floating point E2M1 (exponent bias 1, one fraction bit,
 * exponent 0 is subnormal): magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double q4o_e2m1_to_double(uint8_t nib)
{
    int sign = (nib >> 3) & 1;
    int e = (nib >> 1) & 3;
    int m = nib & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -v : v;
}

/* Weight bytes of an N x K matrix in each format, the pages' closed forms
 * (section 4 table; K a multiple of 64, so K_pad = K wherever K % 128 == 0
 * and the group count is N * K / group size).  -1 for an unknown format. */
int64_t q4o_fmt_weight_bytes(int fmt, int64_t n, int64_t k)
{
    switch (fmt) {
    case Q4O_FMT_Q4: return n * (k / 64) * 34;
    case Q4O_FMT_Q5: return n * (k / 64) * 42;
    case Q4O_FMT_Q6: return n * (k / 64) * 50;
    case Q4O_FMT_W8: return n * (k / 32) * 34;
    case Q4O_FMT_NVFP4: return n * (k / 16) * 9;
    case Q4O_FMT_BF16: return 2 * n * k;
    default: return -1;
    }
}

static int low_nibble(const uint8_t *lo, int64_t K, int64_t n, int64_t k)
{
    uint8_t byte = lo[n * (K / 2) + k / 2];
    return (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* One weight value W[n,k] of format fmt, exact in binary64.  lo: the code
 * plane (Q4/Q5/Q6/NVFP4 nibbles, W8 bytes, BF16 values); hi: the high plane
 * (Q5, Q6; else unused); sc: the scale plane (fp16 bits, or E4M3 bytes for
 * NVFP4; unused for BF16). */
static double fmt_weight(int fmt, const uint8_t *lo, const uint8_t *hi, const void *sc,
                         int64_t K, int64_t n, int64_t k)
{
    const uint16_t *s16 = (const uint16_t *)sc;
    switch (fmt) {
    case Q4O_FMT_Q4: {
        int q = low_nibble(lo, K, n, k);
        return (double)(q - 8) * q4o_fp16_to_double(s16[n * (K / 64) + k / 64]);
    }
    case Q4O_FMT_Q5: {
        int h = (hi[n * (K / 8) + k / 8] >> (k % 8)) & 1;
        int q = low_nibble(lo, K, n, k) | (h << 4);
        return (double)(q - 16) * q4o_fp16_to_double(s16[n * (K / 64) + k / 64]);
    }
    case Q4O_FMT_Q6: {
        int h = (hi[n * (K / 4) + k / 4] >> (2 * (k % 4))) & 3;
        int q = low_nibble(lo, K, n, k) | (h << 4);
        return (double)(q - 32) * q4o_fp16_to_double(s16[n * (K / 64) + k / 64]);
    }
    case Q4O_FMT_W8: {
        int c = (int)(int8_t)lo[n * K + k];
        return (double)c * q4o_fp16_to_double(s16[n * (K / 32) + k / 32]);
    }
    case Q4O_FMT_NVFP4: {
        const uint8_t *s8 = (const uint8_t *)sc;
        return q4o_e2m1_to_double((uint8_t)low_nibble(lo, K, n, k)) * q4o_e4m3_to_double(s8[n * (K / 16) + k / 16]);
    }
    case Q4O_FMT_BF16: {
        const uint16_t *w = (const uint16_t *)lo;
        return q4o_bf16_to_double(w[n * K + k]);
    }
    default:
        return NAN;
    }
}

/* Full product in format fmt (layouts above; x and y as for q4o_linear):
 * y[t*N + n] = bf16_rne(sum_k W[n,k] X[k,t]), binary64 sum in increasing k;
 * acc (optional) receives the unrounded sums. */
void q4o_linear_fmt(int fmt, const uint16_t *x, const uint8_t *lo, const uint8_t *hi, const void *sc,
                    uint16_t *y, double *acc, int64_t N, int64_t K, int64_t T, int threads)
{
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel
    {
        double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
#pragma omp for schedule(dynamic, 4)
        for (int64_t n = 0; n < N; ++n) {
            for (int64_t k = 0; k < K; ++k)
                w[k] = fmt_weight(fmt, lo, hi, sc, K, n, k);
            for (int64_t t = 0; t < T; ++t) {
                double sum = 0.0;
                const uint16_t *xt = x + t * K;
                for (int64_t k = 0; k < K; ++k)
                    sum += w[k] * q4o_bf16_to_double(xt[k]);
                y[t * N + n] = q4o_double_to_bf16(sum);
                if (acc)
                    acc[t * N + n] = sum;
            }
        }
        free(w);
    }
}

/* Selected elements of the format-fmt product: out[i] = Y[ns[i], ts[i]]. */
void q4o_linear_fmt_at(int fmt, const uint16_t *x, const uint8_t *lo, const uint8_t *hi, const void *sc,
                       int64_t N, int64_t K, int64_t T, const int64_t *ns, const int64_t *ts, int64_t count,
                       uint16_t *out, int threads)
{
    (void)N;
    (void)T;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#else
    (void)threads;
#endif
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i) {
        double sum = 0.0;
        for (int64_t k = 0; k < K; ++k)
            sum += fmt_weight(fmt, lo, hi, sc, K, ns[i], k) * q4o_bf16_to_double(x[ts[i] * K + k]);
        out[i] = q4o_double_to_bf16(sum);
    }
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int q4o_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
