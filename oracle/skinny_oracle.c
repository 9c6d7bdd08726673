/*
 * skinny_oracle.c -- CPU oracle for the small-M GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code with the HIP library.
 *
 * What it computes (the plain definition, nothing faster):
 *
 *   out[m, n] = round_bf16( sum_{k=0}^{K-1} x[m, k] * W[n, k]  (+ bias[n]) )
 *
 * "sglang PR #30117" page, key source snippet (kernel header comment):
 * x[M,K] times the transpose of weight[N,K], plus an optional bias[N];
 * bf16 in and out, accumulation in fp32.  The oracle accumulates in fp64
 * (k ascending) over exactly decoded inputs and rounds once, directly from
 * fp64 to bf16, round-to-nearest-even.  The rounding mode is not stated on
 * the pages; RNE is the reading taken (IEEE default).
 *
 * FP8 modes (the later variant):
 *  - per-tensor: "sglang PR #28333" page, key source snippet
 *    (flashinfer_bmm_fp8 / apply_fp8_linear_bmm_flashinfer): one fp32 scale
 *    for x and one for W; the page's motivation section calls a second
 *    application of the scales a bug, so the product sx*sw is applied
 *    exactly once per output:  out = round_bf16(sx*sw*sum(xq*wq) + bias).
 *  - MX: "sglang PR #34042" page (MXFP8 dense GEMM): block-scaled FP8.  The
 *    block is 32 consecutive K elements of one row, scale = e8m0.
 *    out = round_bf16( sum_b 2^(ex[m,b]-127) * 2^(ew[n,b]-127)
 *                            * sum_{k in block b} xq*wq  + bias ).
 *  FP8 element format: OCP e4m3fn (max 448, S.1111.111 is NaN, no inf).
 *
 * fp32-output variant (router logits, "vllm PR #42562" page, split-K kernel
 * snippet: out dtype fp32): the same sum rounded once from fp64 to fp32.
 *
 * Static activation quantisation ("sglang PR #28333" page, the static FP8
 * quant kernel): with a given per-tensor scale s,
 *     q = e4m3( clamp( x * (1 / s), -448, 448 ) ),
 * evaluated in binary32 as that kernel does (x widened to fp32, one
 * reciprocal, one product, round to the nearest e4m3 value, ties to even).
 * Because these roundings decide integer codes, the oracle takes them in
 * the same precision (binary32), not in fp64.
 *
 * Threads: the (m, n) outputs are independent; OpenMP splits them over
 * threads.  The k order inside one output never changes, so the result is
 * bitwise identical for every thread count.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoders */

/* bf16 is the upper half of an IEEE binary32; widening is exact. */
double oracle_decode_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits.
 * e >= 1: (-1)^s * 2^(e-7) * (1 + m/8);  e == 0: (-1)^s * 2^-6 * (m/8);
 * e == 15 and m == 7: NaN.  No infinities. */
double oracle_decode_e4m3(uint8_t b)
{
    int s = (b >> 7) & 1;
    int e = (b >> 3) & 15;
    int m = b & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);            /* 2^-6 * m/8 */
    else
        v = ldexp(8.0 + (double)m, e - 10);  /* 2^(e-7) * (8+m)/8 */
    return s ? -v : v;
}

/* OCP e8m0: an exponent-only byte, 2^(e-127); 0xFF is NaN. */
double oracle_decode_e8m0(uint8_t b)
{
    if (b == 0xFF)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* ---------------------------------------------------------------- rounding */

/* Round a double to the nearest bf16, ties to even, in one step.
 * bf16: 8 significant bits, exponent range of binary32, subnormals down to
 * 2^-133, largest finite (2 - 2^-7) * 2^127.  The rounding is done on the
 * double itself (never through a float), so there is exactly one rounding. */
uint16_t oracle_round_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);            /* a = f * 2^e2, f in [0.5, 1) -> floor(log2 a) = e2 - 1 */
    int e = e2 - 1;
    if (e < -126)
        e = -126;             /* subnormal range: fixed quantum 2^-133 */
    int q_exp = e - 7;        /* quantum (ulp) of the binade: 2^(e-7) */
    double q = ldexp(a, -q_exp);  /* exact: scaling by a power of two */
    double r = nearbyint(q);      /* default rounding mode: nearest, ties to even */
    double res = ldexp(r, q_exp); /* exact */
    const double max_finite = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (res > max_finite)
        return (uint16_t)(sign | 0x7F80);
    /* res is exactly representable in bf16, hence in binary32: the float
     * conversion below is exact and the upper 16 bits are the bf16 code. */
    float f = (float)res;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFF));
}

/* Round a double to binary32 (RNE): a single conversion. */
float oracle_round_f32(double v)
{
    return (float)v;
}

/* Round a binary32 value to the nearest OCP e4m3fn code, ties to even.
 * Finite inputs must lie in [-448, 448] (the quantiser clamps first); the
 * top binade's quantum is 32, so nothing rounds past 448.  NaN gives the
 * NaN code with the input's sign.  Below 2^-6 the quantum is fixed at 2^-9
 * (subnormals). */
uint8_t oracle_encode_e4m3(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0;
    if (isnan(v))
        return (uint8_t)(sign | 0x7F);
    double a = fabs((double)v);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);
    int e = e2 - 1;            /* floor(log2 a) */
    if (e < -6)
        e = -6;                /* subnormal range */
    int q_exp = e - 3;         /* 3 mantissa bits: quantum 2^(e-3) */
    double r = nearbyint(ldexp(a, -q_exp));  /* exact scaling, RNE */
    double res = ldexp(r, q_exp);
    if (res == 0.0)
        return sign;
    frexp(res, &e2);
    int E = e2 - 1;
    if (E < -6)                /* subnormal: res = m * 2^-9, m = 1..7 */
        return (uint8_t)(sign | (uint8_t)ldexp(res, 9));
    int mant = (int)ldexp(res, 3 - E) - 8;   /* res = 2^E * (8 + mant) / 8 */
    return (uint8_t)(sign | (uint8_t)((E + 7) << 3) | (uint8_t)mant);
}

/* Static per-tensor quantisation of n bf16 values with scale s. */
void oracle_quant_e4m3(const uint16_t *x, long n, float s, uint8_t *q)
{
    const float inv = 1.0f / s;          /* one correctly rounded reciprocal */
    for (long i = 0; i < n; ++i) {
        float v = (float)oracle_decode_bf16(x[i]) * inv;  /* exact widening, one product */
        if (!isnan(v))
            v = v < -448.0f ? -448.0f : (v > 448.0f ? 448.0f : v);
        q[i] = oracle_encode_e4m3(v);
    }
}

/* ---------------------------------------------------------------- GEMMs */

static void set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Writes the final value: bf16 code into out16, or binary32 into out32. */
static void emit(double acc, long idx, uint16_t *out16, float *out32)
{
    if (out32)
        out32[idx] = oracle_round_f32(acc);
    else
        out16[idx] = oracle_round_bf16(acc);
}

/* bf16 x[M,K], W[N,K] (row-major), optional bias[N]; out[M,N]. */
void oracle_gemm_bf16(const uint16_t *x, const uint16_t *w, const uint16_t *bias,
                      uint16_t *out16, float *out32, long M, long N, long K,
                      int nthreads)
{
    set_threads(nthreads);
#pragma omp parallel for collapse(2) schedule(static)
    for (long m = 0; m < M; ++m) {
        for (long n = 0; n < N; ++n) {
            double acc = 0.0;
            for (long k = 0; k < K; ++k)
                acc += oracle_decode_bf16(x[m * K + k]) * oracle_decode_bf16(w[n * K + k]);
            if (bias)
                acc += oracle_decode_bf16(bias[n]);
            emit(acc, m * N + n, out16, out32);
        }
    }
}

/* FP8 e4m3 with one fp32 scale per tensor (sx for x, sw for W). */
void oracle_gemm_fp8_tensor(const uint8_t *xq, const uint8_t *wq, float sx, float sw,
                            const uint16_t *bias, uint16_t *out16, float *out32,
                            long M, long N, long K, int nthreads)
{
    set_threads(nthreads);
    const double scale = (double)sx * (double)sw;
#pragma omp parallel for collapse(2) schedule(static)
    for (long m = 0; m < M; ++m) {
        for (long n = 0; n < N; ++n) {
            double dot = 0.0;
            for (long k = 0; k < K; ++k)
                dot += oracle_decode_e4m3(xq[m * K + k]) * oracle_decode_e4m3(wq[n * K + k]);
            double acc = dot * scale;
            if (bias)
                acc += oracle_decode_bf16(bias[n]);
            emit(acc, m * N + n, out16, out32);
        }
    }
}

/* FP8 e4m3 with one e8m0 scale per 32 consecutive K of every row:
 * xe[M, K/32], we[N, K/32], row-major.  K must be a multiple of 32. */
void oracle_gemm_fp8_mx(const uint8_t *xq, const uint8_t *wq, const uint8_t *xe,
                        const uint8_t *we, const uint16_t *bias, uint16_t *out16,
                        float *out32, long M, long N, long K, int nthreads)
{
    set_threads(nthreads);
    const long KB = K / 32;
#pragma omp parallel for collapse(2) schedule(static)
    for (long m = 0; m < M; ++m) {
        for (long n = 0; n < N; ++n) {
            double acc = 0.0;
            for (long b = 0; b < KB; ++b) {
                double block = 0.0;
                for (long k = b * 32; k < b * 32 + 32; ++k)
                    block += oracle_decode_e4m3(xq[m * K + k]) * oracle_decode_e4m3(wq[n * K + k]);
                acc += oracle_decode_e8m0(xe[m * KB + b]) * oracle_decode_e8m0(we[n * KB + b]) * block;
            }
            if (bias)
                acc += oracle_decode_bf16(bias[n]);
            emit(acc, m * N + n, out16, out32);
        }
    }
}

/* Number of threads an OpenMP region will use with the given request. */
int oracle_threads_used(int nthreads)
{
#ifdef _OPENMP
    int used = 1;
    set_threads(nthreads);
#pragma omp parallel
    {
#pragma omp single
        used = omp_get_num_threads();
    }
    return used;
#else
    (void)nthreads;
    return 1;
#endif
}
