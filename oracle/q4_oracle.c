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
 *     Canonical packed layout: row n of Wq holds K/2 bytes; byte j holds the
 *     code of k = 2j in bits 0..3 and the code of k = 2j+1 in bits 4..7.
 *     Scales are row-major [N][K/32].
 *   - The library's tiled layout (what its pack produces and its kernels
 *     read): tiles of 16 rows (t = n / 16, c = n % 16) by 4 blocks
 *     (q = b / 4, i = b % 4), ordered [ceil(N/16)][ceil(nb/4)], 1024 code
 *     bytes and 64 scales each.  Inside a code tile, the little-endian
 *     32-bit word at byte 16 * (16 g + c) + 4 i holds the eight codes of
 *     k = 32 b + 8 g + r, r = 0..7, of row n: the code of r sits at bit
 *     4 * (r / 2) + 16 * (r % 2) (even r in the low half-word, odd r in the
 *     high one, each half in ascending r).  The scale of (n, b) is element
 *     4 c + i of its tile's 64.  Positions past N rows or nb blocks are zero.
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

#define Q4O_ABI 3

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

/* Tiled layout: quads of 4 blocks along K, and the byte / scale index of
 * weight (n, k) and block (n, b). */
static int64_t quads_of(int64_t K) { return (K / 32 + 3) / 4; }

/* Word index (in 32-bit words) and bit position of weight (n, k)'s code. */
static int64_t tiled_word_index(int64_t K, int64_t n, int64_t k)
{
    const int64_t b = k / 32, g = (k % 32) / 8;
    const int64_t t = n / 16, c = n % 16, q = b / 4, i = b % 4;
    return ((t * quads_of(K) + q) * 1024 + 16 * (16 * g + c) + 4 * i) / 4;
}

static int tiled_bit(int64_t k)
{
    const int r = (int)(k % 8);
    return 4 * (r / 2) + 16 * (r % 2);
}

static int64_t tiled_scale_index(int64_t K, int64_t n, int64_t b)
{
    const int64_t t = n / 16, c = n % 16, q = b / 4, i = b % 4;
    return (t * quads_of(K) + q) * 64 + 4 * c + i;
}

/* The 32-bit word at word index w of a tiled code buffer (little-endian). */
static uint32_t tiled_word(const uint8_t *wq, int64_t w)
{
    return (uint32_t)wq[4 * w] | ((uint32_t)wq[4 * w + 1] << 8) | ((uint32_t)wq[4 * w + 2] << 16) |
           ((uint32_t)wq[4 * w + 3] << 24);
}

static int tiled_code_at(const uint8_t *wq, int64_t K, int64_t n, int64_t k)
{
    return (int)((tiled_word(wq, tiled_word_index(K, n, k)) >> tiled_bit(k)) & 0x0F);
}

/* Dequantized weight (n, k) = (q - 8) * d[n][k/32], exact in fp64. */
static double weight_at(const uint8_t *wq, const uint16_t *scales,
                        int64_t K, int64_t n, int64_t k, int tiled)
{
    const int q = tiled ? tiled_code_at(wq, K, n, k) : code_at(wq, K, n, k);
    const uint16_t dbits = tiled ? scales[tiled_scale_index(K, n, k / 32)]
                                 : scales[n * (K / 32) + k / 32];
    const double d = q4o_f16_to_f64(dbits);
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

/* Sizes of the tiled layout: code bytes and scale entries. */
int64_t q4o_tiled_code_bytes(int64_t N, int64_t K) { return (N + 15) / 16 * quads_of(K) * 1024; }
int64_t q4o_tiled_scale_count(int64_t N, int64_t K) { return (N + 15) / 16 * quads_of(K) * 64; }

/* Pack into the tiled layout: codes u8 [N][K] (low 4 bits used) and scales
 * fp16 bits [N][K/32] -> tiled codes and tiled scales (padding zeroed). */
void q4o_pack_tiled(const uint8_t *codes, const uint16_t *scales, uint8_t *wq_t,
                    uint16_t *sc_t, int64_t N, int64_t K)
{
    for (int64_t i = 0; i < q4o_tiled_code_bytes(N, K); ++i)
        wq_t[i] = 0;
    for (int64_t i = 0; i < q4o_tiled_scale_count(N, K); ++i)
        sc_t[i] = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const int64_t w = tiled_word_index(K, n, k);
            const int bit = tiled_bit(k);
            const uint8_t code = codes[n * K + k] & 0x0F;
            wq_t[4 * w + bit / 8] |= (uint8_t)(code << (bit % 8));
        }
        for (int64_t b = 0; b < K / 32; ++b)
            sc_t[tiled_scale_index(K, n, b)] = scales[n * (K / 32) + b];
    }
}

/* Inverse of q4o_pack_tiled: -> codes u8 [N][K] in 0..15, scales [N][K/32]. */
void q4o_unpack_tiled(const uint8_t *wq_t, const uint16_t *sc_t, uint8_t *codes,
                      uint16_t *scales, int64_t N, int64_t K)
{
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)tiled_code_at(wq_t, K, n, k);
        for (int64_t b = 0; b < K / 32; ++b)
            scales[n * (K / 32) + b] = sc_t[tiled_scale_index(K, n, b)];
    }
}

/* One output and its normaliser, summing in ascending k. */
static void one_output(const double *xrow, const uint8_t *wq,
                       const uint16_t *scales, int64_t K, int64_t n, int tiled,
                       double *y_out, double *a_out)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        const double t = xrow[k] * weight_at(wq, scales, K, n, k, tiled);
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
 * bf16); wq, scales: canonical ([N][K/2], [N][K/32]) if tiled == 0, else the
 * tiled layout; y, a: double [M][N].  Returns 0, or -1 if K is not a
 * positive multiple of 32 or memory runs out.
 */
int q4o_linear_fmt(const uint16_t *x, int x_is_bf16, const uint8_t *wq,
                   const uint16_t *scales, int64_t M, int64_t N, int64_t K,
                   int tiled, double *y, double *a)
{
    if (K <= 0 || K % 32 != 0 || M < 0 || N < 0)
        return -1;
    double *xd = decode_x(x, x_is_bf16, M, K);
    if (!xd && M * K > 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m)
            one_output(xd + m * K, wq, scales, K, n, tiled, &y[m * N + n], &a[m * N + n]);
    free(xd);
    return 0;
}

int q4o_linear(const uint16_t *x, int x_is_bf16, const uint8_t *wq,
               const uint16_t *scales, int64_t M, int64_t N, int64_t K,
               double *y, double *a)
{
    return q4o_linear_fmt(x, x_is_bf16, wq, scales, M, N, K, 0, y, a);
}

/*
 * Selected outputs only: for i < count, output (ms[i], ns[i]) goes to y[i]
 * and a[i].  Same arithmetic as q4o_linear_fmt (either layout), for spot
 * checks of products too large to evaluate whole.
 */
int q4o_linear_sampled(const uint16_t *x, int x_is_bf16, const uint8_t *wq,
                       const uint16_t *scales, int64_t M, int64_t N, int64_t K,
                       int tiled, const int64_t *ms, const int64_t *ns, int64_t count,
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
            one_output(xrow, wq, scales, K, ns[i], tiled, &y[i], &a[i]);
        }
        free(xrow);
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------- quantizer
 * The step before pack, which the pages never define: how dense weights
 * become codes and scales.  The rule (absmax scaling, the plain reading of
 * a symmetric 4-bit code with offset 8 whose largest magnitude, 7, maps to
 * the block's largest weight), per block of 32 consecutive weights of a row:
 *     d = absmax / 7, rounded once to binary16 (nearest, ties to even);
 *     q = clamp(round_half_even(w / d), -8, 7) + 8, on the exact quotient;
 *     a block whose d rounds to zero gets d = +0 and every code 8.
 * Inputs must be finite with absmax / 7 below the binary16 overflow
 * threshold (65520); other blocks are outside the rule.
 *
 * Exactness here: absmax / 7 is rounded to fp64 and then to binary16, which
 * equals one rounding of the exact quotient (53 >= 2 * 11 + 2 bits); w / d
 * for w of at most 24 significant bits and d of at most 11 cannot land on a
 * half-integer by fp64 rounding unless it is one exactly, so nearbyint of
 * the fp64 quotient is the half-even rounding of the exact quotient.
 */

/* double -> binary16 bits, nearest, ties to even (overflow -> infinity). */
uint16_t q4o_f64_to_f16(double v)
{
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    if (isnan(v))
        return 0x7E00;
    if (a == 0.0)
        return sign;
    int e;
    frexp(a, &e);      /* a = m 2^e, m in [0.5, 1) */
    int E = e - 1;     /* a = (2m) 2^E, 2m in [1, 2) */
    if (E < -14) {     /* subnormal range: quantum 2^-24 */
        const double n = nearbyint(ldexp(a, 24));  /* 0 .. 1024 (1024 = smallest normal) */
        return (uint16_t)(sign | (uint16_t)n);
    }
    double n = nearbyint(ldexp(a, 10 - E));  /* 1024 .. 2048 */
    if (n == 2048.0) {
        n = 1024.0;
        ++E;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)n - 1024));
}

/* One input element as an exact double: kind 0 binary16 bits, 1 bfloat16
 * bits (both uint16), 2 IEEE binary32 (float). */
static double w_value(const void *w, int kind, int64_t i)
{
    if (kind == 2)
        return (double)((const float *)w)[i];
    const uint16_t b = ((const uint16_t *)w)[i];
    return kind == 1 ? q4o_bf16_to_f64(b) : q4o_f16_to_f64(b);
}

/* w [N][K] (kind as above) -> codes uint8 [N][K], scales binary16 bits
 * [N][K/32].  Returns 0, or -1 for a bad shape or kind. */
int q4o_quantize(const void *w, int kind, uint8_t *codes, uint16_t *scales, int64_t N, int64_t K)
{
    if (N < 0 || K <= 0 || K % 32 != 0 || kind < 0 || kind > 2)
        return -1;
    const int64_t nb = K / 32;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t base = n * K + 32 * b;
            double absmax = 0.0;
            for (int k = 0; k < 32; ++k) {
                const double a = fabs(w_value(w, kind, base + k));
                if (a > absmax)
                    absmax = a;
            }
            const uint16_t dbits = q4o_f64_to_f16(absmax / 7.0);
            const double d = q4o_f16_to_f64(dbits);
            scales[n * nb + b] = dbits;
            for (int k = 0; k < 32; ++k) {
                int code = 8;
                if (d != 0.0) {
                    double q = nearbyint(w_value(w, kind, base + k) / d);
                    if (q < -8.0)
                        q = -8.0;
                    if (q > 7.0)
                        q = 7.0;
                    code = (int)q + 8;
                }
                codes[base + k] = (uint8_t)code;
            }
        }
    }
    return 0;
}
