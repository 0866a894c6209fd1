/*
 * w4a16_oracle.c — plain, slow CPU oracle of the W4A16 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg load this library.  It shares no code, header,
 * table or constant with the HIP library, and nothing in the product path
 * calls it.
 *
 * Sources (web pages):
 *   [QUANT] qaqbuyan.com article 126 on LLM quantization, section
 *           "量化的数学基石——从 IEEE 754 到量化误差":
 *           sub-section 1 (FP16 bit layout), sub-section 2 (symmetric
 *           quantization: s = max|x| / (2^(b-1) - 1), x_q = clamp(round(x/s),
 *           -2^(b-1), 2^(b-1) - 1), INT4 range [-8,7]), sub-section 3
 *           (per-group granularity; per-group quantizer / dequantizer
 *           listing: groups along in_features, offset-binary nibbles q+8,
 *           even index in the low nibble, fp32 dequantization s*q).
 *   [INT4]  guijiagi.com tag page "量化", INT4 paragraph (absmax / 7,
 *           round, clamp to [-8, 7]).
 *
 * Everything is computed in IEEE binary64.  fp16 values are carried as
 * their bit patterns and decoded / encoded here from the binary16
 * definition ([QUANT] sub-section 1: 1 sign, 5 exponent, 10 mantissa bits,
 * bias 15, subnormals below 2^-14).
 *
 * Readings where the pages leave a step open:
 *   - "round" is round-half-to-even (the pages' listings use torch.round);
 *   - the scale is stored as fp16, and q is computed against that stored
 *     scale, with the exact quotient w/s;
 *   - a group whose fp16 scale is 0 stores scale 0 and q = 0 everywhere;
 *   - eight nibbles per little-endian uint32, element 8j+i in bits 4i..4i+3;
 *   - asymmetric INT4 (see oracle_quantize_asym): the same rounding, the
 *     scale stored as fp16 and z taken against it, z stored as int16, and
 *     a zero-scale group stored as s = 0, z = 0, q = 0;
 *   - Q4_0 blocks (see oracle_quantize_q4_0): scale d = absmax / 7 as for
 *     the symmetric form, and the dequantizer's adjacent-pair nibble order.
 *
 * Build: cc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 */
#include <math.h>
#include <fenv.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- fp16 */

/* binary16 bits -> exact binary64 value ([QUANT] sub-section 1). */
double oracle_f64_from_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v;
    if (e == 0x1F) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexp((double)m, -24);           /* subnormal: m * 2^-24 */
    } else {
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* binary64 -> binary16 bits, round to nearest, ties to even. */
uint16_t oracle_f16_from_f64(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return (uint16_t)(sign | 0x7E00);
    if (a >= 65520.0) return (uint16_t)(sign | 0x7C00); /* 65504 + half ulp rounds to inf */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: value = r * 2^-24, r integer in [0, 1024] */
        double r = nearbyint(ldexp(a, 24)); /* exact scaling, then RNE */
        return (uint16_t)(sign | (uint16_t)r); /* r == 1024 yields the min normal 0x0400 */
    }
    int ex;
    double fr = frexp(a, &ex);          /* a = fr * 2^ex, fr in [0.5, 1) */
    int e = ex - 1;                     /* a = (2 fr) * 2^e, 2 fr in [1, 2) */
    double r = nearbyint(ldexp(fr, 11)); /* 11 significant bits, RNE */
    if (r == 2048.0) { r = 1024.0; e += 1; }
    if (e > 15) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)((int)r - 1024));
}

/* ------------------------------------------------------------ quantize */

/* Per-group symmetric INT4 quantization of one group of `g` fp16 values.
 * [QUANT] sub-section 2 (equations), sub-section 3 (per-group scale).
 * Writes the fp16 scale bits and the g codes q in [-8, 7]. */
static void quantize_group(const uint16_t* w, int64_t g, uint16_t* scale_bits, int8_t* q)
{
    double a = 0.0;
    for (int64_t i = 0; i < g; i++) {
        double v = fabs(oracle_f64_from_f16(w[i]));
        if (v > a) a = v;
    }
    uint16_t s16 = oracle_f16_from_f64(a / 7.0); /* 2^(4-1) - 1 = 7 */
    double s = oracle_f64_from_f16(s16);
    *scale_bits = s16;
    for (int64_t i = 0; i < g; i++) {
        if (s == 0.0) { q[i] = 0; continue; }
        double r = nearbyint(oracle_f64_from_f16(w[i]) / s); /* RNE in FE_TONEAREST */
        if (r < -8.0) r = -8.0;
        if (r > 7.0) r = 7.0;
        q[i] = (int8_t)r;
    }
}

/* W fp16 [N,K] -> packed uint32 [N, K/8], scales fp16 [N, K/group].
 * group must be a multiple of 8 dividing K.  Returns 0, or -1 on bad sizes. */
int oracle_quantize(const uint16_t* W, int64_t N, int64_t K, int64_t group,
                    uint32_t* packed, uint16_t* scales)
{
    if (N < 0 || K < 0 || group <= 0 || group % 8 != 0 || K % group != 0) return -1;
    if (fegetround() != FE_TONEAREST) return -1;
    int64_t ng = K / group;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        int8_t* q = (int8_t*)malloc((size_t)group);
        for (int64_t gi = 0; gi < ng; gi++) {
            quantize_group(W + n * K + gi * group, group, &scales[n * ng + gi], q);
            for (int64_t j = 0; j < group / 8; j++) {
                uint32_t word = 0;
                for (int i = 0; i < 8; i++) {
                    uint32_t nib = (uint32_t)(q[8 * j + i] + 8) & 0xFu; /* offset binary */
                    word |= nib << (4 * i);
                }
                packed[n * (K / 8) + (gi * group) / 8 + j] = word;
            }
        }
        free(q);
    }
    return 0;
}

/* --------------------------------------------------------- dequantize */

/* Code of element k of row n: nibble (k mod 8) of word k/8, minus 8. */
static int code_at(const uint32_t* row_words, int64_t k)
{
    uint32_t word = row_words[k / 8];
    return (int)((word >> (4 * (k % 8))) & 0xFu) - 8;
}

/* Ŵ[n,k] = s[n, k/group] * q[n,k], exact in binary64 ([QUANT] sub-section 3,
 * dequantizer).  What is [N, K] binary64. */
int oracle_dequantize(const uint32_t* packed, const uint16_t* scales, int64_t N, int64_t K,
                      int64_t group, double* What)
{
    if (N < 0 || K < 0 || group <= 0 || group % 8 != 0 || K % group != 0) return -1;
    int64_t ng = K / group;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            What[n * K + k] = oracle_f64_from_f16(scales[n * ng + k / group]) *
                              (double)code_at(packed + n * (K / 8), k);
    return 0;
}

/* ------------------------------------------------------------- matmul */

/* One output: sum_k x[k] * Ŵ[n,k] in binary64, and sum_k |x[k] * Ŵ[n,k]|.
 * Each product is exact (11-bit x 11-bit x 4-bit significands). */
static void dot_row(const uint16_t* x, const uint32_t* row_words, const uint16_t* row_scales,
                    int64_t K, int64_t group, double* y, double* yabs)
{
    double acc = 0.0, acc_abs = 0.0;
    for (int64_t k = 0; k < K; k++) {
        double w = oracle_f64_from_f16(row_scales[k / group]) * (double)code_at(row_words, k);
        double t = oracle_f64_from_f16(x[k]) * w;
        acc += t;
        acc_abs += fabs(t);
    }
    *y = acc;
    *yabs = acc_abs;
}

/* Y[m,n] = sum_k X[m,k] Ŵ[n,k] (binary64), Yabs[m,n] = sum_k |X[m,k] Ŵ[n,k]|.
 * X fp16 [M,K]; Y, Yabs binary64 [M,N]. */
int oracle_matmul(const uint16_t* X, int64_t M, const uint32_t* packed, const uint16_t* scales,
                  int64_t N, int64_t K, int64_t group, double* Y, double* Yabs)
{
    if (M < 0 || N < 0 || K < 0 || group <= 0 || group % 8 != 0 || K % group != 0) return -1;
    int64_t ng = K / group;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            dot_row(X + m * K, packed + n * (K / 8), scales + n * ng, K, group,
                    &Y[m * N + n], &Yabs[m * N + n]);
    return 0;
}

/* The same for `count` chosen outputs (rows[i], cols[i]) of a large problem. */
int oracle_matmul_sampled(const uint16_t* X, int64_t M, const uint32_t* packed,
                          const uint16_t* scales, int64_t N, int64_t K, int64_t group,
                          const int64_t* rows, const int64_t* cols, int64_t count,
                          double* Y, double* Yabs)
{
    if (M < 0 || N < 0 || K < 0 || group <= 0 || group % 8 != 0 || K % group != 0) return -1;
    for (int64_t i = 0; i < count; i++)
        if (rows[i] < 0 || rows[i] >= M || cols[i] < 0 || cols[i] >= N) return -1;
    int64_t ng = K / group;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++)
        dot_row(X + rows[i] * K, packed + cols[i] * (K / 8), scales + cols[i] * ng, K, group,
                &Y[i], &Yabs[i]);
    return 0;
}

/* ------------------------------------------------ asymmetric INT4 */

/* Per-group asymmetric INT4 quantization ([QUANT] sub-section 2, the
 * asymmetric equations: s = (max - min) / (2^b - 1), z = -round(min / s),
 * x_q = clamp(round(x / s) + z, 0, 2^b - 1), INT4 range [0, 15]):
 *   s is stored as fp16 (RNE of the exact (max - min) / 15; max - min is
 *   exact in binary64, fp16 values being multiples of 2^-24 below 2^16),
 *   z = -round_half_even(min / s) against the stored s (an integer; it lies
 *   in [0, 15] when the group holds both signs and can be far outside for a
 *   one-signed group with a narrow range, |z| <= 15 * 2^11 * (1 + 2^-11)),
 *   q = clamp(round_half_even(w / s) + z, 0, 15);
 *   a group whose fp16 scale is 0 stores s = 0, z = 0 and q = 0.
 * Dequantized: s * (q - z). */
static void quantize_group_asym(const uint16_t* w, int64_t g, uint16_t* scale_bits,
                                int16_t* zero, uint8_t* q)
{
    double mx = -INFINITY, mn = INFINITY;
    for (int64_t i = 0; i < g; i++) {
        double v = oracle_f64_from_f16(w[i]);
        if (v > mx) mx = v;
        if (v < mn) mn = v;
    }
    uint16_t s16 = oracle_f16_from_f64((mx - mn) / 15.0); /* 2^4 - 1 = 15 */
    double s = oracle_f64_from_f16(s16);
    *scale_bits = s16;
    if (s == 0.0) {
        *zero = 0;
        for (int64_t i = 0; i < g; i++) q[i] = 0;
        return;
    }
    double z = -nearbyint(mn / s);                        /* RNE in FE_TONEAREST */
    *zero = (int16_t)z;
    for (int64_t i = 0; i < g; i++) {
        double r = nearbyint(oracle_f64_from_f16(w[i]) / s) + z;
        if (r < 0.0) r = 0.0;
        if (r > 15.0) r = 15.0;
        q[i] = (uint8_t)r;
    }
}

/* W fp16 [N,K] -> packed uint32 [N, K/8] (nibble = q in [0, 15], element
 * 8j+i in bits 4i..4i+3 of word j), scales fp16 [N, K/group], zero points
 * int16 [N, K/group]. */
int oracle_quantize_asym(const uint16_t* W, int64_t N, int64_t K, int64_t group,
                         uint32_t* packed, uint16_t* scales, int16_t* zeros)
{
    if (N < 0 || K < 0 || group <= 0 || group % 8 != 0 || K % group != 0) return -1;
    if (fegetround() != FE_TONEAREST) return -1;
    int64_t ng = K / group;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        uint8_t* q = (uint8_t*)malloc((size_t)group);
        for (int64_t gi = 0; gi < ng; gi++) {
            quantize_group_asym(W + n * K + gi * group, group, &scales[n * ng + gi],
                                &zeros[n * ng + gi], q);
            for (int64_t j = 0; j < group / 8; j++) {
                uint32_t word = 0;
                for (int i = 0; i < 8; i++) word |= ((uint32_t)q[8 * j + i] & 0xFu) << (4 * i);
                packed[n * (K / 8) + (gi * group) / 8 + j] = word;
            }
        }
        free(q);
    }
    return 0;
}

/* Nibble of element k of a row (0..15). */
static int nibble_at(const uint32_t* row_words, int64_t k)
{
    return (int)((row_words[k / 8] >> (4 * (k % 8))) & 0xFu);
}

/* Ŵ[n,k] = s[n, k/group] * (q[n,k] - z[n, k/group]), exact in binary64
 * (an 11-bit significand times an integer below 2^16). */
int oracle_dequantize_asym(const uint32_t* packed, const uint16_t* scales, const int16_t* zeros,
                           int64_t N, int64_t K, int64_t group, double* What)
{
    if (N < 0 || K < 0 || group <= 0 || group % 8 != 0 || K % group != 0) return -1;
    int64_t ng = K / group;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++)
            What[n * K + k] = oracle_f64_from_f16(scales[n * ng + k / group]) *
                              (double)(nibble_at(packed + n * (K / 8), k) -
                                       zeros[n * ng + k / group]);
    return 0;
}

/* Y = X·Ŵᵀ and Yabs = sum |X Ŵ| with the asymmetric Ŵ, binary64 (each
 * product exact: 11-bit x 11-bit x 16-bit significands fit 53 bits). */
int oracle_matmul_asym(const uint16_t* X, int64_t M, const uint32_t* packed,
                       const uint16_t* scales, const int16_t* zeros, int64_t N, int64_t K,
                       int64_t group, double* Y, double* Yabs)
{
    if (M < 0 || N < 0 || K < 0 || group <= 0 || group % 8 != 0 || K % group != 0) return -1;
    int64_t ng = K / group;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double sum = 0.0, sum_abs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                double what = oracle_f64_from_f16(scales[n * ng + k / group]) *
                              (double)(nibble_at(packed + n * (K / 8), k) -
                                       zeros[n * ng + k / group]);
                double prod = oracle_f64_from_f16(X[m * K + k]) * what;
                sum += prod;
                sum_abs += fabs(prod);
            }
            Y[m * N + n] = sum;
            Yabs[m * N + n] = sum_abs;
        }
    return 0;
}

/* ----------------------------------------------------- Q4_0 blocks */

/* Q4_0 block layout ([QUANT] GGUF section: type table, Q4_0 = 32 elements
 * per block, 18 bytes, symmetric with a per-block scale; the section's
 * Q4_0 dequantizer): per row, K/32 consecutive blocks of
 *   bytes 0-1   d, the fp16 scale, little-endian
 *   bytes 2-17  byte 2+i holds element 2i in its low nibble and element
 *               2i+1 in its high nibble, each as q + 8
 * with the symmetric quantizer of this file on groups of 32 (d = RNE(absmax
 * / 7), q = clamp(RNE(w/d), -8, 7)).  Dequantized: d * (nibble - 8). */
#define Q4_0_BLOCK 32
#define Q4_0_BYTES 18

int oracle_quantize_q4_0(const uint16_t* W, int64_t N, int64_t K, uint8_t* blocks)
{
    if (N < 0 || K < 0 || K % Q4_0_BLOCK != 0) return -1;
    if (fegetround() != FE_TONEAREST) return -1;
    const int64_t nb = K / Q4_0_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; n++) {
        int8_t q[Q4_0_BLOCK];
        for (int64_t b = 0; b < nb; b++) {
            uint16_t d;
            quantize_group(W + n * K + b * Q4_0_BLOCK, Q4_0_BLOCK, &d, q);
            uint8_t* blk = blocks + (n * nb + b) * Q4_0_BYTES;
            blk[0] = (uint8_t)(d & 0xFF);
            blk[1] = (uint8_t)(d >> 8);
            for (int i = 0; i < Q4_0_BLOCK / 2; i++)
                blk[2 + i] = (uint8_t)(((q[2 * i] + 8) & 0xF) | (((q[2 * i + 1] + 8) & 0xF) << 4));
        }
    }
    return 0;
}

/* Element k of row n of a Q4_0 matrix, dequantized (exact in binary64). */
static double q4_0_weight(const uint8_t* blocks, int64_t nb, int64_t n, int64_t k)
{
    const uint8_t* blk = blocks + (n * nb + k / Q4_0_BLOCK) * Q4_0_BYTES;
    const uint16_t d = (uint16_t)(blk[0] | (blk[1] << 8));
    const int j = (int)(k % Q4_0_BLOCK);
    const uint8_t byte = blk[2 + j / 2];
    const int nib = (j % 2 == 0) ? (byte & 0xF) : (byte >> 4);
    return oracle_f64_from_f16(d) * (double)(nib - 8);
}

int oracle_dequantize_q4_0(const uint8_t* blocks, int64_t N, int64_t K, double* What)
{
    if (N < 0 || K < 0 || K % Q4_0_BLOCK != 0) return -1;
    const int64_t nb = K / Q4_0_BLOCK;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) What[n * K + k] = q4_0_weight(blocks, nb, n, k);
    return 0;
}

/* Y = X·Ŵᵀ and Yabs = sum |X Ŵ| with Ŵ read from Q4_0 blocks (binary64). */
int oracle_matmul_q4_0(const uint16_t* X, int64_t M, const uint8_t* blocks, int64_t N, int64_t K,
                       double* Y, double* Yabs)
{
    if (M < 0 || N < 0 || K < 0 || K % Q4_0_BLOCK != 0) return -1;
    const int64_t nb = K / Q4_0_BLOCK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++) {
            double total = 0.0, total_abs = 0.0;
            for (int64_t k = 0; k < K; k++) {
                const double term = oracle_f64_from_f16(X[m * K + k]) * q4_0_weight(blocks, nb, n, k);
                total += term;
                total_abs += fabs(term);
            }
            Y[m * N + n] = total;
            Yabs[m * N + n] = total_abs;
        }
    return 0;
}

/* Number of threads the parallel loops above use. */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
