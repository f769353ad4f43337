/*
 * mxfp4_oracle.c -- plain, slow CPU reference for the 4-bit float (MXFP4)
 * variant of the SVDQuant W4A4 linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP implementation.
 *
 * The "Bringing Nunchaku 4-bit inference to Diffusers" blog (sections
 * "Introducing Nunchaku Lite" and the quantization_config listing) gives the
 * svdq_w4a4 kernel family an INT4 and an NVFP4 variant, NVFP4 with group
 * size 16, for GPUs that have FP4 arithmetic; the pages do not define its
 * scale format.  The 4-bit float format with native arithmetic on the
 * target here is MXFP4 of the OCP Microscaling Formats (MX) specification
 * v1.0, which this variant uses instead (different numerics, so it is
 * checked against this oracle only):
 *   - blocks of 32 consecutive values along K share one scale X = 2^e stored
 *     as E8M0 (byte e + 127), e = floor(log2(max |v|)) - 2 (2 = the largest
 *     exponent of E2M1), clamped to [-127, 127];
 *   - each value becomes the E2M1 number nearest to v / X (magnitudes 0, 0.5,
 *     1, 1.5, 2, 3, 4, 6), ties to the even code, magnitudes above 6 to 6;
 *   - codes: sign bit 3, magnitude code 0..7 in bits 0-2; a zero magnitude is
 *     stored as code 0 (never -0) -- a reading, the specification allows
 *     either; an all-zero block gets the scale byte 0;
 *   - packing as the INT4 path: two codes per byte, element 2j in the low
 *     nibble, row-major [rows, K/2]; scales row-major u8 [rows, K/32].
 * The rest of the layer is the INT4 path's: x^ = fl32(x fl32(1/lambda)) is
 * quantized, the residual R is quantized the same way, and
 *   Y = sum_blocks X_a X_w sum_e a_e w_e + xl1 L2 + bias  (then GELU)
 * in fp64 with one rounding to bf16.
 *
 * Build: compiled into the same library as svdq_oracle.c.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MX_BLOCK 32

uint16_t oracle_bf16_rne(double v); /* svdq_oracle.c */
double oracle_gelu(double x);       /* svdq_oracle.c */

static const double mx_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* E2M1 code (0..15) of y, nearest with ties to the even code, saturating. */
int oracle_mx_e2m1_code(double y)
{
    const double a = fabs(y);
    int best = 7;
    if (a < 6.0) {
        best = 0;
        for (int c = 1; c < 8; ++c) {
            const double d = fabs(a - mx_mag[c]), db = fabs(a - mx_mag[best]);
            if (d < db || (d == db && (c & 1) == 0))
                best = c;
        }
    }
    if (best == 0)
        return 0;
    return (y < 0 ? 8 : 0) | best;
}

double oracle_mx_e2m1_value(int code)
{
    const double m = mx_mag[code & 7];
    return (code & 8) ? -m : m;
}

/* E8M0 scale byte of a block whose largest magnitude is amax. */
int oracle_mx_scale_byte(double amax)
{
    if (!(amax > 0.0))
        return 0;
    int e2;
    frexp(amax, &e2);            /* amax = f 2^e2, f in [0.5, 1): floor(log2 amax) = e2 - 1 */
    int e = (e2 - 1) - 2;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    return e + 127;
}

/*
 * Quantize v [rows, K] (fp32) block by block: packed codes [rows, K/2] and
 * E8M0 scale bytes [rows, K/32].
 */
void oracle_mx_quantize(const float *v, int64_t rows, int64_t K, uint8_t *packed, uint8_t *scales)
{
    const int64_t NBK = K / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < NBK; ++b) {
            const float *x = v + r * K + b * MX_BLOCK;
            double amax = 0.0;
            for (int j = 0; j < MX_BLOCK; ++j)
                if (fabs((double)x[j]) > amax)
                    amax = fabs((double)x[j]);
            const int sb = oracle_mx_scale_byte(amax);
            const double X = ldexp(1.0, sb - 127);
            scales[r * NBK + b] = (uint8_t)sb;
            uint8_t *dst = packed + r * (K / 2) + b * (MX_BLOCK / 2);
            for (int j = 0; j < MX_BLOCK / 2; ++j) {
                const int c0 = amax > 0.0 ? oracle_mx_e2m1_code((double)x[2 * j] / X) : 0;
                const int c1 = amax > 0.0 ? oracle_mx_e2m1_code((double)x[2 * j + 1] / X) : 0;
                dst[j] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
}

/* Dequantized values [rows, K] in fp64. */
void oracle_mx_dequant(const uint8_t *packed, const uint8_t *scales, int64_t rows, int64_t K,
                       double *out)
{
    const int64_t NBK = K / MX_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k) {
            const unsigned byte = packed[r * (K / 2) + k / 2];
            const int code = (int)((k & 1) ? (byte >> 4) : (byte & 15u));
            out[r * K + k] = oracle_mx_e2m1_value(code) * ldexp(1.0, scales[r * NBK + k / MX_BLOCK] - 127);
        }
}

/*
 * The layer output for the selected token rows (all when rows == NULL):
 *   acc = sum_b Xa[m][b] Xw[n][b] sum_{k in b} a[m][k] w[n][k]
 *       + sum_i xl1[m][i] L2[i][n] + bias[n], GELU if act == 1,
 * fp64; acc_out / y_out [nrows, N] (either may be NULL; y: bf16 bits).
 */
void oracle_mx_gemm_rows(const uint8_t *qa, const uint8_t *sa, const uint8_t *qw,
                         const uint8_t *sw, const double *xl1, const uint16_t *L2,
                         const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                         int32_t r, const int64_t *rows, int64_t nrows, double *acc_out,
                         uint16_t *y_out)
{
    (void)M;
    const int64_t NBK = K / MX_BLOCK;
    double *wv = (double *)malloc(sizeof(double) * (size_t)(N * K));
    oracle_mx_dequant(qw, sw, N, K, wv);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        const int64_t m = rows ? rows[ri] : ri;
        double *av = (double *)malloc(sizeof(double) * (size_t)K);
        oracle_mx_dequant(qa + m * (K / 2), sa + m * NBK, 1, K, av);
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += av[k] * wv[n * K + k];
            for (int32_t i = 0; i < r; ++i) {
                uint32_t u = (uint32_t)L2[(int64_t)i * N + n] << 16;
                float f;
                memcpy(&f, &u, sizeof f);
                acc += xl1[m * r + i] * (double)f;
            }
            if (bias) {
                uint32_t u = (uint32_t)bias[n] << 16;
                float f;
                memcpy(&f, &u, sizeof f);
                acc += (double)f;
            }
            if (act == 1)
                acc = oracle_gelu(acc);
            if (acc_out)
                acc_out[ri * N + n] = acc;
            if (y_out)
                y_out[ri * N + n] = oracle_bf16_rne(acc);
        }
        free(av);
    }
    free(wv);
}
