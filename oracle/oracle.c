/*
 * Plain CPU oracle for the tiled dense GEMM.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The GPU product path never calls it, and it shares
 * no code, header or table with the GPU path.
 *
 * What is computed (the definition, not a fast method):
 *
 *   NT:     C[m][n] = R_out( sum_{k=0}^{K-1} A[m][k] * B[n][k] )
 *           A is M x K, B is N x K, both row-major (TileLang SM100 README,
 *           "Code Example": A (M,K), B (N,K), gemm with trans_B=True).
 *   NN:     C[m][n] = R_out( sum_k A[m][k] * B[k][n] )
 *           B is K x N row-major (velog "tilelang", 1.1 Front-End DSL:
 *           B: T.Tensor((K, N)) and T.gemm(A_shared, B_shared, C_local)).
 *   MXFP8:  C[m][n] = R_bf16( sum_k (q(A[m][k]) * 2^(EA[m][k/128]-127))
 *                                 * (q(B[n][k]) * 2^(EB[n][k/128]-127)) )
 *           one e8m0 scale per row per 128 K elements for each operand
 *           (Blackwell TCGEN05 GEMM tutorial, "进阶" (Advanced):
 *           gemm_blockscaled with sf_a_granularity_k = sf_b_granularity_k = 128).
 *
 * Products and the running sum are IEEE binary64, summed in sequential k
 * order k = 0..K-1 with one accumulator per output, and R_out is a single
 * round-to-nearest-even from binary64 to the output type.  The pages' own
 * check rounds an fp32 matmul to the output type once (SM100 README,
 * "Compilation and Usage": ref_c = (a.float @ b.T.float).to(bfloat16));
 * binary64 is the stricter reading.
 *
 * The outer loop over rows m is split across OpenMP threads.  That changes
 * no arithmetic: every output is still one sequential k-ordered sum.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math: the k order of the
 * sum must not be changed by the compiler).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------ */
/* Decoders: bit patterns -> binary64 (exact).                               */
/* ------------------------------------------------------------------------ */

/* bfloat16 is the upper half of an IEEE binary32 word. */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits,
 * no infinities, S.1111.111 is NaN, largest finite 448. */
double oracle_e4m3fn_to_f64(uint8_t b)
{
    int sign = (b >> 7) & 1;
    int e = (b >> 3) & 0xf;
    int f = b & 0x7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -9);                /* f/8 * 2^(1-7) */
    else
        v = ldexp((double)(8 + f), e - 10);      /* (1 + f/8) * 2^(e-7) */
    return sign ? -v : v;
}

/*
 * OCP FP4 E2M1 (the MXFP4 element type): sign, 2 exponent bits (bias 1),
 * 1 mantissa bit; exponent 0 is subnormal (0 or 0.5); no infinities or
 * NaN.  Values: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives.
 */
double oracle_e2m1_to_f64(uint8_t nibble)
{
    int sign = (nibble >> 3) & 1;
    int e = (nibble >> 1) & 3;
    int f = nibble & 1;
    double v = e == 0 ? 0.5 * f : ldexp(1.0 + 0.5 * f, e - 1);
    return sign ? -v : v;
}

/* Element k of a row of packed FP4: byte k / 2, the low nibble for even k. */
static uint8_t fp4_at(const uint8_t *row, int64_t k)
{
    uint8_t b = row[k / 2];
    return (k & 1) ? (uint8_t)(b >> 4) : (uint8_t)(b & 15);
}

/* OCP E8M0 scale: an unsigned biased exponent, value 2^(E-127); 0xFF is NaN. */
double oracle_e8m0_to_f64(uint8_t e)
{
    if (e == 0xff)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* ------------------------------------------------------------------------ */
/* Encoders: binary64 -> nearest representable, ties to even, one rounding.  */
/* ------------------------------------------------------------------------ */

/*
 * Round |x| to a floating-point grid with `p` significant bits, minimum
 * normal exponent `emin` (value 2^emin) and subnormals below it.  Returns the
 * rounded magnitude as a binary64 (exact: p <= 11 here, well inside 53 bits).
 *
 * The quantum (spacing of the grid at |x|) is 2^(floor(log2|x|) - (p-1)) in
 * the normal range and 2^(emin - (p-1)) below it.  |x| / quantum is exact
 * (a power-of-two scaling), and nearbyint() in the default rounding mode
 * rounds halfway cases to the even integer.
 */
static double round_to_grid(double ax, int p, int emin)
{
    int e2;
    (void)frexp(ax, &e2);            /* ax = f * 2^e2, f in [0.5, 1) */
    int ex = e2 - 1;                 /* floor(log2(ax)) for ax > 0 */
    if (ex < emin)
        ex = emin;
    double quantum = ldexp(1.0, ex - (p - 1));
    return nearbyint(ax / quantum) * quantum;
}

/* binary64 -> bfloat16 (8 significant bits, exponent range of binary32). */
uint16_t oracle_f64_to_bf16(double x)
{
    if (isnan(x))
        return 0x7fc0;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (ax == 0.0)
        return sign;
    if (isinf(ax))
        return sign | 0x7f80;
    double r = round_to_grid(ax, 8, -126);
    if (r >= ldexp(1.0, 128))        /* rounded past the largest finite */
        return sign | 0x7f80;
    /* r is a bfloat16 value, hence exactly a binary32 value. */
    float f = (float)r;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)(u >> 16);
}

/* binary64 -> IEEE binary16 (11 significant bits, emin = -14). */
uint16_t oracle_f64_to_f16(double x)
{
    if (isnan(x))
        return 0x7e00;
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    double ax = fabs(x);
    if (ax == 0.0)
        return sign;
    if (isinf(ax))
        return sign | 0x7c00;
    double r = round_to_grid(ax, 11, -14);
    if (r >= 65536.0)                /* largest finite is 65504 */
        return sign | 0x7c00;
    if (r < ldexp(1.0, -14))         /* subnormal: r = f * 2^-24 */
        return sign | (uint16_t)(r * 16777216.0);
    int e2;
    double fr = frexp(r, &e2);       /* r = fr * 2^e2, fr in [0.5, 1) */
    int ex = e2 - 1;                 /* r = (1 + f/1024) * 2^ex */
    uint16_t f = (uint16_t)(fr * 2048.0 - 1024.0);
    return sign | (uint16_t)((ex + 15) << 10) | f;
}

/*
 * binary64 -> OCP FP8 E4M3FN (4 significant bits, emin = -6, bias 7, largest
 * finite 448 = 0x7e; no infinities, 0x7f/0xff are NaN).  For |x| <= 448
 * only, which is all the quantiser below produces.
 */
uint8_t oracle_f64_to_e4m3fn(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0;
    double ax = fabs(x);
    if (ax == 0.0)
        return sign;
    double r = round_to_grid(ax, 4, -6);
    if (r < ldexp(1.0, -6))          /* subnormal: r = m * 2^-9, m in 0..7 */
        return sign | (uint8_t)(r * 512.0);
    int e2;
    double fr = frexp(r, &e2);       /* r = fr * 2^e2, fr in [0.5, 1) */
    int ex = e2 - 1;                 /* r = (1 + m/8) * 2^ex */
    uint8_t m = (uint8_t)(fr * 16.0 - 8.0);
    return sign | (uint8_t)((ex + 7) << 3) | m;
}

/* Elementwise array forms, for the tests. */
void oracle_decode_bf16(int64_t n, const uint16_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(in[i]);
}
void oracle_decode_f16(int64_t n, const uint16_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(in[i]);
}
void oracle_decode_e4m3fn(int64_t n, const uint8_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3fn_to_f64(in[i]);
}
void oracle_decode_e8m0(int64_t n, const uint8_t *in, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e8m0_to_f64(in[i]);
}
void oracle_encode_bf16(int64_t n, const double *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(in[i]);
}
void oracle_encode_f16(int64_t n, const double *in, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16(in[i]);
}
void oracle_encode_e4m3fn(int64_t n, const double *in, uint8_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_e4m3fn(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Block-scale quantiser.                                                    */
/* ------------------------------------------------------------------------ */

/*
 * The step that makes the block-scaled GEMM's operands: binary32 rows x
 * (R x K, row-major) to e4m3fn bytes q (R x K) with one e8m0 scale byte per
 * row per 128 K elements, s (R x ceil(K/128)) -- the granularity of the
 * Blackwell TCGEN05 GEMM tutorial, section "进阶" (Advanced):
 * sf_a_granularity_k = sf_b_granularity_k = 128.  The pages give no rule
 * for choosing a scale; the reading taken is the smallest power of two 2^e
 * with absmax <= 448 * 2^e (448 = largest e4m3fn), e clamped to
 * [-127, 127], e = -127 for an all-zero block, stored as the byte e + 127;
 * each element is x * 2^-e (exact) rounded once to e4m3fn, ties to even.
 * A last block shorter than 128 (K % 128 != 0) takes the maximum over the
 * elements it has.  Inputs must be finite.
 */
void oracle_quantize_mxfp8(int64_t R, int64_t K, const float *x, uint8_t *q, uint8_t *s)
{
    const int64_t KB = (K + 127) / 128;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        for (int64_t b = 0; b < KB; ++b) {
            const int64_t k0 = b * 128, k1 = k0 + 128 < K ? k0 + 128 : K;
            double absmax = 0.0;
            for (int64_t k = k0; k < k1; ++k) {
                double a = fabs((double)x[r * K + k]);
                if (a > absmax)
                    absmax = a;
            }
            int e;
            if (absmax == 0.0) {
                e = -127;
            } else {
                int e2;
                (void)frexp(absmax, &e2);        /* 2^(e2-1) <= absmax < 2^e2 */
                /* 448 * 2^(e2-10) < 2^(e2-1) <= absmax: start below the answer
                   and take the first e that fits. */
                e = e2 - 10;
                while (absmax > ldexp(448.0, e))
                    ++e;
                if (e < -127)
                    e = -127;
                if (e > 127)
                    e = 127;
            }
            s[r * KB + b] = (uint8_t)(e + 127);
            for (int64_t k = k0; k < k1; ++k)
                q[r * K + k] = oracle_f64_to_e4m3fn(ldexp((double)x[r * K + k], -e));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* The GEMMs.                                                                */
/* ------------------------------------------------------------------------ */

/*
 * Every GEMM below writes, for each output, the binary64 sum (out64, may be
 * NULL) and its single rounding to the output type (out, may be NULL).
 */

/* NT, bf16 in, bf16 out:  C = A . B^T  with A (M,K), B (N,K). */
void oracle_gemm_bf16_nt(int64_t M, int64_t N, int64_t K,
                         const uint16_t *A, const uint16_t *B,
                         uint16_t *C, double *C64)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += oracle_bf16_to_f64(A[m * K + k]) *
                       oracle_bf16_to_f64(B[n * K + k]);
            if (C64) C64[m * N + n] = acc;
            if (C) C[m * N + n] = oracle_f64_to_bf16(acc);
        }
    }
}

/* NN, fp16 in, fp16 out:  C = A . B  with A (M,K), B (K,N). */
void oracle_gemm_f16_nn(int64_t M, int64_t N, int64_t K,
                        const uint16_t *A, const uint16_t *B,
                        uint16_t *C, double *C64)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += oracle_f16_to_f64(A[m * K + k]) *
                       oracle_f16_to_f64(B[k * N + n]);
            if (C64) C64[m * N + n] = acc;
            if (C) C[m * N + n] = oracle_f64_to_f16(acc);
        }
    }
}

/* Block-scaled FP8 NT, bf16 out.  qA (M,K) and qB (N,K) are e4m3fn bytes;
 * sA (M, ceil(K/128)) and sB (N, ceil(K/128)) are e8m0 bytes, row-major. */
void oracle_gemm_mxfp8_nt(int64_t M, int64_t N, int64_t K,
                          const uint8_t *qA, const uint8_t *qB,
                          const uint8_t *sA, const uint8_t *sB,
                          uint16_t *C, double *C64)
{
    const int64_t KB = (K + 127) / 128;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = oracle_e4m3fn_to_f64(qA[m * K + k]) *
                           oracle_e8m0_to_f64(sA[m * KB + k / 128]);
                double b = oracle_e4m3fn_to_f64(qB[n * K + k]) *
                           oracle_e8m0_to_f64(sB[n * KB + k / 128]);
                acc += a * b;
            }
            if (C64) C64[m * N + n] = acc;
            if (C) C[m * N + n] = oracle_f64_to_bf16(acc);
        }
    }
}

/*
 * MXFP4 NT: C[m][n] = R_bf16( sum_k (e2m1(A[m][k]) * 2^(EA[m][k/32]-127))
 *                                  * (e2m1(B[n][k]) * 2^(EB[n][k/32]-127)) ).
 * Block-scaled formats other than MXFP8 (Blackwell TCGEN05 GEMM tutorial,
 * section "进阶" (Advanced), names MXFP8 "and other" block-scaled formats);
 * the pages give the FP4 layout and block size of none, so this follows the
 * OCP MX format: E2M1 elements packed two per byte, element 2i in the low
 * nibble of byte i, and one E8M0 scale per 32 consecutive elements along K.
 * A row of qA holds K/2 bytes; sA is M x ceil(K/32).
 */
void oracle_gemm_mxfp4_nt(int64_t M, int64_t N, int64_t K,
                          const uint8_t *qA, const uint8_t *qB,
                          const uint8_t *sA, const uint8_t *sB,
                          uint16_t *C, double *C64)
{
    const int64_t KB = (K + 31) / 32, KH = (K + 1) / 2;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = oracle_e2m1_to_f64(fp4_at(qA + m * KH, k)) *
                           oracle_e8m0_to_f64(sA[m * KB + k / 32]);
                double b = oracle_e2m1_to_f64(fp4_at(qB + n * KH, k)) *
                           oracle_e8m0_to_f64(sB[n * KB + k / 32]);
                acc += a * b;
            }
            if (C64) C64[m * N + n] = acc;
            if (C) C[m * N + n] = oracle_f64_to_bf16(acc);
        }
    }
}

/*
 * Sampled forms: the same sums, for a list of P output positions
 * (rows[p], cols[p]) only, so that full-size problems can be checked
 * one output at a time.  out[p] / out64[p] receive C[rows[p]][cols[p]].
 */
void oracle_gemm_bf16_nt_at(int64_t M, int64_t N, int64_t K,
                            const uint16_t *A, const uint16_t *B,
                            int64_t P, const int64_t *rows, const int64_t *cols,
                            uint16_t *out, double *out64)
{
    (void)M; (void)N;
    #pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; ++p) {
        int64_t m = rows[p], n = cols[p];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += oracle_bf16_to_f64(A[m * K + k]) *
                   oracle_bf16_to_f64(B[n * K + k]);
        if (out64) out64[p] = acc;
        if (out) out[p] = oracle_f64_to_bf16(acc);
    }
}

void oracle_gemm_f16_nn_at(int64_t M, int64_t N, int64_t K,
                           const uint16_t *A, const uint16_t *B,
                           int64_t P, const int64_t *rows, const int64_t *cols,
                           uint16_t *out, double *out64)
{
    (void)M;
    #pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; ++p) {
        int64_t m = rows[p], n = cols[p];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += oracle_f16_to_f64(A[m * K + k]) *
                   oracle_f16_to_f64(B[k * N + n]);
        if (out64) out64[p] = acc;
        if (out) out[p] = oracle_f64_to_f16(acc);
    }
}

void oracle_gemm_mxfp8_nt_at(int64_t M, int64_t N, int64_t K,
                             const uint8_t *qA, const uint8_t *qB,
                             const uint8_t *sA, const uint8_t *sB,
                             int64_t P, const int64_t *rows, const int64_t *cols,
                             uint16_t *out, double *out64)
{
    (void)M; (void)N;
    const int64_t KB = (K + 127) / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; ++p) {
        int64_t m = rows[p], n = cols[p];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = oracle_e4m3fn_to_f64(qA[m * K + k]) *
                       oracle_e8m0_to_f64(sA[m * KB + k / 128]);
            double b = oracle_e4m3fn_to_f64(qB[n * K + k]) *
                       oracle_e8m0_to_f64(sB[n * KB + k / 128]);
            acc += a * b;
        }
        if (out64) out64[p] = acc;
        if (out) out[p] = oracle_f64_to_bf16(acc);
    }
}

void oracle_gemm_mxfp4_nt_at(int64_t M, int64_t N, int64_t K,
                             const uint8_t *qA, const uint8_t *qB,
                             const uint8_t *sA, const uint8_t *sB,
                             int64_t P, const int64_t *rows, const int64_t *cols,
                             uint16_t *out, double *out64)
{
    (void)M; (void)N;
    const int64_t KB = (K + 31) / 32, KH = (K + 1) / 2;
    #pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; ++p) {
        int64_t m = rows[p], n = cols[p];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = oracle_e2m1_to_f64(fp4_at(qA + m * KH, k)) *
                       oracle_e8m0_to_f64(sA[m * KB + k / 32]);
            double b = oracle_e2m1_to_f64(fp4_at(qB + n * KH, k)) *
                       oracle_e8m0_to_f64(sB[n * KB + k / 32]);
            acc += a * b;
        }
        if (out64) out64[p] = acc;
        if (out) out[p] = oracle_f64_to_bf16(acc);
    }
}

/* Elementwise FP4 decoding, for the tests. */
void oracle_decode_e2m1(int64_t n, const uint8_t *nibbles, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_e2m1_to_f64(nibbles[i] & 15);
}

/* ------------------------------------------------------------------------ */
/* MXFP6                                                                     */
/* ------------------------------------------------------------------------ */

/*
 * OCP FP6 elements (the MXFP6 element types), from their definitions:
 *   fmt 0, E2M3: sign, 2 exponent bits (bias 1), 3 mantissa bits; max 7.5;
 *   fmt 1, E3M2: sign, 3 exponent bits (bias 3), 2 mantissa bits; max 28.
 * Exponent field 0 is subnormal: mantissa * 2^(1 - bias - mantissa bits).
 * Neither type has infinities or NaN.
 */
double oracle_fp6_to_f64(uint8_t code, int fmt)
{
    const int ebits = fmt == 0 ? 2 : 3, mbits = 5 - ebits, bias = fmt == 0 ? 1 : 3;
    const int sign = (code >> 5) & 1;
    const int e = (code >> mbits) & ((1 << ebits) - 1);
    const int f = code & ((1 << mbits) - 1);
    double v = e == 0 ? ldexp((double)f, 1 - bias - mbits)
                      : ldexp((double)((1 << mbits) + f), e - bias - mbits);
    return sign ? -v : v;
}

/*
 * Element k of a row of packed FP6: bits 6k .. 6k + 5 of the row read as a
 * little-endian bit string (byte b holds bits 8b .. 8b + 7, bit 0 its least
 * significant).  The second byte is read only when the element reaches it.
 */
static uint8_t fp6_at(const uint8_t *row, int64_t k)
{
    const int64_t bit = 6 * k, byte = bit / 8;
    const int sh = (int)(bit % 8);
    unsigned v = row[byte] >> sh;
    if (sh > 2) v |= (unsigned)row[byte + 1] << (8 - sh);
    return (uint8_t)(v & 63u);
}

/*
 * MXFP6 NT: C[m][n] = R_bf16( sum_k (fp6(A[m][k]) * 2^(EA[m][k/32]-127))
 *                                  * (fp6(B[n][k]) * 2^(EB[n][k/32]-127)) ),
 * both operands of element type fmt.  Another of the block-scaled formats
 * the Blackwell TCGEN05 GEMM tutorial (section "进阶" (Advanced)) groups
 * with MXFP8; the pages give no layout, so this follows the OCP MX format
 * (one E8M0 scale per 32 consecutive elements along K) with the elements
 * packed densely: a row of K elements is 3K/4 bytes, element k at bits
 * 6k .. 6k + 5.  K % 4 == 0; sA is M x ceil(K/32).
 */
void oracle_gemm_mxfp6_nt(int64_t M, int64_t N, int64_t K, int fmt,
                          const uint8_t *qA, const uint8_t *qB,
                          const uint8_t *sA, const uint8_t *sB,
                          uint16_t *C, double *C64)
{
    const int64_t KB = (K + 31) / 32, RB = K / 4 * 3;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = oracle_fp6_to_f64(fp6_at(qA + m * RB, k), fmt) *
                           oracle_e8m0_to_f64(sA[m * KB + k / 32]);
                double b = oracle_fp6_to_f64(fp6_at(qB + n * RB, k), fmt) *
                           oracle_e8m0_to_f64(sB[n * KB + k / 32]);
                acc += a * b;
            }
            if (C64) C64[m * N + n] = acc;
            if (C) C[m * N + n] = oracle_f64_to_bf16(acc);
        }
    }
}

/* Chosen outputs C[rows[p]][cols[p]] of oracle_gemm_mxfp6_nt. */
void oracle_gemm_mxfp6_nt_at(int64_t M, int64_t N, int64_t K, int fmt,
                             const uint8_t *qA, const uint8_t *qB,
                             const uint8_t *sA, const uint8_t *sB,
                             int64_t P, const int64_t *rows, const int64_t *cols,
                             uint16_t *out, double *out64)
{
    (void)M; (void)N;
    const int64_t KB = (K + 31) / 32, RB = K / 4 * 3;
    #pragma omp parallel for schedule(static)
    for (int64_t p = 0; p < P; ++p) {
        int64_t m = rows[p], n = cols[p];
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = oracle_fp6_to_f64(fp6_at(qA + m * RB, k), fmt) *
                       oracle_e8m0_to_f64(sA[m * KB + k / 32]);
            double b = oracle_fp6_to_f64(fp6_at(qB + n * RB, k), fmt) *
                       oracle_e8m0_to_f64(sB[n * KB + k / 32]);
            acc += a * b;
        }
        if (out64) out64[p] = acc;
        if (out) out[p] = oracle_f64_to_bf16(acc);
    }
}

/* fp6 codes (one per byte, low 6 bits) -> binary64. */
void oracle_decode_fp6(int64_t n, const uint8_t *codes, int fmt, double *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_fp6_to_f64(codes[i] & 63, fmt);
}

/* Element k of each of n packed FP6 rows of `row_bytes` bytes -> codes (the
 * oracle's unpacking, exposed so a test can check the bit order). */
void oracle_unpack_fp6(int64_t rows, int64_t row_bytes, int64_t K, const uint8_t *q, uint8_t *codes)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) codes[r * K + k] = fp6_at(q + r * row_bytes, k);
}

/* Number of OpenMP threads a parallel region of this library would use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
