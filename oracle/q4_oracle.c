/*
 * q4_oracle.c -- plain, slow, fp64 CPU oracle for the 4-bit block-quantized
 * linear layer  y[M x N] = x[M x K] . dequant(Wq[N x K])^T.
 *
 * TEST INFRASTRUCTURE.  Only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  The product
 * path (the HIP library) shares no code with it and never calls it.
 *
 * What is computed, and where it comes from:
 *   - "Why Continuous Batching Slowed Down My LLM Inference Engine: A Metal
 *     Kernel Investigation", section "Two Rows of Input, Two Different
 *     Kernels": the matrix-vector product dot-products each row of the
 *     (4-bit quantized) weight matrix with the input vector; the
 *     matrix-matrix product does the same for several input rows at once.
 *     Both compute the same mathematical value; only summation order and
 *     dequantization timing differ (section "Same Prompt, Different Story").
 *   - "Why LLM Decoding Is Slow, and Why Batching Is (Almost) Free",
 *     section 2 ("First Attempt: A Faster Chip"): every weight is read once
 *     and used for one multiply and one add per input row.
 *   - The pages do not fix a 4-bit format.  The format used here: blocks of
 *     32 consecutive weights along K share one IEEE binary16 scale d; each
 *     weight has a code q in 0..15; the weight's value is (q - 8) * d.
 *     Packed layout: row n of Wq holds K/2 bytes; byte j holds the code of
 *     k = 2j in bits 0..3 and the code of k = 2j+1 in bits 4..7.  Scales
 *     are row-major [N][K/32].
 *
 * Definition computed (the plain reading):
 *     y[m][n] = sum_{k=0}^{K-1} x[m][k] * (q[n][k] - 8) * d[n][k/32]
 *     A[m][n] = sum_{k=0}^{K-1} | x[m][k] * (q[n][k] - 8) * d[n][k/32] |
 * A is the normaliser of the parity tolerance.
 *
 * Exactness: (q-8)*d needs at most 4 + 11 significant bits, and x (fp16 or
 * bf16) at most 11, so every product is exact in fp64; only the running
 * sum rounds, in ascending k, with error at most about K * 2^-53 * A.
 * OpenMP splits work over n only; every output's summation order is fixed,
 * so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define Q4O_ABI 1

int q4o_abi_version(void) { return Q4O_ABI; }

/* IEEE binary16 bit pattern -> exact double (zero, subnormals, inf, nan). */
double q4o_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1F;
    const int frac = h & 0x3FF;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(0x400 | frac), expo - 25);
    return sign ? -mag : mag;
}

/* bfloat16 bit pattern (top half of an IEEE binary32) -> exact double. */
double q4o_bf16_to_f64(uint16_t b)
{
    const int sign = (b >> 15) & 1;
    const int expo = (b >> 7) & 0xFF;
    const int frac = b & 0x7F;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -133);
    else if (expo == 255)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(0x80 | frac), expo - 134);
    return sign ? -mag : mag;
}

static double x_value(uint16_t bits, int x_is_bf16)
{
    return x_is_bf16 ? q4o_bf16_to_f64(bits) : q4o_f16_to_f64(bits);
}

/* Code of weight (n, k) from the packed rows. */
static int code_at(const uint8_t *wq, int64_t K, int64_t n, int64_t k)
{
    const uint8_t byte = wq[n * (K / 2) + k / 2];
    return (k % 2 == 0) ? (byte & 0x0F) : (byte >> 4);
}

/* Dequantized weight (n, k) = (q - 8) * d[n][k/32], exact in fp64. */
static double weight_at(const uint8_t *wq, const uint16_t *scales,
                        int64_t K, int64_t n, int64_t k)
{
    const int q = code_at(wq, K, n, k);
    const double d = q4o_f16_to_f64(scales[n * (K / 32) + k / 32]);
    return (double)(q - 8) * d;
}

/* Pack: codes u8 [N][K] (low 4 bits used) -> Wq u8 [N][K/2]. */
void q4o_pack(const uint8_t *codes, uint8_t *wq, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t j = 0; j < K / 2; ++j) {
            const uint8_t lo = codes[n * K + 2 * j] & 0x0F;
            const uint8_t hi = codes[n * K + 2 * j + 1] & 0x0F;
            wq[n * (K / 2) + j] = (uint8_t)(lo | (hi << 4));
        }
}

/* Unpack: Wq u8 [N][K/2] -> codes u8 [N][K] in 0..15. */
void q4o_unpack(const uint8_t *wq, uint8_t *codes, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)code_at(wq, K, n, k);
}

/* One output and its normaliser, summing in ascending k. */
static void one_output(const double *xrow, const uint8_t *wq,
                       const uint16_t *scales, int64_t K, int64_t n,
                       double *y_out, double *a_out)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double t = xrow[k] * weight_at(wq, scales, K, n, k);
        acc += t;
        mag += fabs(t);
    }
    *y_out = acc;
    *a_out = mag;
}

static double *decode_x(const uint16_t *x, int x_is_bf16, int64_t M, int64_t K)
{
    double *xd = (double *)malloc(sizeof(double) * (size_t)(M * K));
    if (!xd)
        return NULL;
    for (int64_t i = 0; i < M * K; ++i)
        xd[i] = x_value(x[i], x_is_bf16);
    return xd;
}

/*
 * Full product.  x: u16 bit patterns [M][K] (fp16 if x_is_bf16 == 0, else
 * bf16); wq: u8 [N][K/2]; scales: fp16 bits [N][K/32]; y, a: double [M][N].
 * Returns 0, or -1 if K is not a positive multiple of 32 or memory runs out.
 */
int q4o_linear(const uint16_t *x, int x_is_bf16, const uint8_t *wq,
               const uint16_t *scales, int64_t M, int64_t N, int64_t K,
               double *y, double *a)
{
    if (K <= 0 || K % 32 != 0 || M < 0 || N < 0)
        return -1;
    double *xd = decode_x(x, x_is_bf16, M, K);
    if (!xd && M * K > 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m)
            one_output(xd + m * K, wq, scales, K, n, &y[m * N + n], &a[m * N + n]);
    free(xd);
    return 0;
}

/*
 * Selected outputs only: for i < count, output (ms[i], ns[i]) goes to y[i]
 * and a[i].  Same arithmetic as q4o_linear, for spot checks of products too
 * large to evaluate whole.
 */
int q4o_linear_sampled(const uint16_t *x, int x_is_bf16, const uint8_t *wq,
                       const uint16_t *scales, int64_t M, int64_t N, int64_t K,
                       const int64_t *ms, const int64_t *ns, int64_t count,
                       double *y, double *a)
{
    if (K <= 0 || K % 32 != 0)
        return -1;
    for (int64_t i = 0; i < count; ++i)
        if (ms[i] < 0 || ms[i] >= M || ns[i] < 0 || ns[i] >= N)
            return -1;
    int failed = 0;
#pragma omp parallel reduction(| : failed)
    {
        double *xrow = (double *)malloc(sizeof(double) * (size_t)K);
        if (!xrow)
            failed = 1;
#pragma omp for schedule(static)
        for (int64_t i = 0; i < count; ++i) {
            if (!xrow)
                continue;
            for (int64_t k = 0; k < K; ++k)
                xrow[k] = x_value(x[ms[i] * K + k], x_is_bf16);
            one_output(xrow, wq, scales, K, ns[i], &y[i], &a[i]);
        }
        free(xrow);
    }
    return failed ? -1 : 0;
}
