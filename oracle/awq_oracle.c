/*
 * awq_oracle.c -- plain, slow CPU reference for the 4-bit-weight,
 * 16-bit-activation linear (W4A16).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP implementation.
 *
 * The "Bringing Nunchaku 4-bit inference to Diffusers" blog, section
 * "Introducing Nunchaku Lite", names a second layer kind besides the W4A4
 * one: awq_w4a16, 4-bit weights with 16-bit activations, used for the
 * adaptive-normalization / modulation projections; its quantization_config
 * listing gives precision int4 and group size 64.  The pages say nothing
 * more about the format.  The readings used here:
 *   - asymmetric round-to-nearest quantization of each group of 64
 *     consecutive weights along K with an fp32 scale s and an integer zero
 *     point z in [0, 15]; codes q in [0, 15]; the weight stands for
 *     (q - z) * s;
 *   - the quantized range always contains zero: lo = min(0, min w),
 *     hi = max(0, max w), s = fl32(fl32(hi - lo) / 15), so that zero (and a
 *     constant group) is represented exactly;
 *   - inv = fl32(1 / s); z = clamp(rint(fl32(-lo * inv)), 0, 15);
 *     q = clamp(rint(fl32(w * inv)) + z, 0, 15), ties to even; a zero scale
 *     or a scale whose reciprocal overflows gives q = z = 0;
 *   - codes packed two per byte, element 2j in the low nibble, unsigned,
 *     row-major [N, K/2]; scales fp32 and zero points u8, row-major [N, K/64];
 *   - the layer is Y = X W^T + bias with X bf16 [M, K]; the product and the
 *     bias are taken in fp64 and Y is ONE correct rounding to bf16.
 *
 * Build: compiled into the same library as svdq_oracle.c
 * (gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define AWQ_GROUP 64

uint16_t oracle_bf16_rne(double v); /* svdq_oracle.c */

static float awq_bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float clamp_code(float c)
{
    if (c < 0.0f)
        return 0.0f;
    if (c > 15.0f)
        return 15.0f;
    return c;
}

/*
 * Quantize the fp32 weight W [N, K] (row n = output feature n) group by
 * group: packed codes [N, K/2], scales [N, K/64], zero points [N, K/64].
 */
void oracle_awq_quantize(const float *W, int64_t N, int64_t K, uint8_t *packed,
                         float *scales, uint8_t *zeros)
{
    const int64_t G = K / AWQ_GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < G; ++g) {
            const float *w = W + n * K + g * AWQ_GROUP;
            float lo = 0.0f, hi = 0.0f;
            for (int j = 0; j < AWQ_GROUP; ++j) {
                if (w[j] < lo)
                    lo = w[j];
                if (w[j] > hi)
                    hi = w[j];
            }
            const float range = hi - lo;
            const float s = range / 15.0f;
            int q[AWQ_GROUP];
            int z = 0;
            int degenerate = 1;
            float inv = 0.0f;
            if (s != 0.0f) {
                inv = 1.0f / s;
                degenerate = !isfinite(inv);
            }
            if (!degenerate) {
                const float zl = -lo * inv;
                z = (int)clamp_code(rintf(zl));
            }
            for (int j = 0; j < AWQ_GROUP; ++j) {
                if (degenerate) {
                    q[j] = 0;
                    continue;
                }
                const float y = w[j] * inv;
                q[j] = (int)clamp_code(rintf(y) + (float)z);
            }
            scales[n * G + g] = s;
            zeros[n * G + g] = (uint8_t)z;
            uint8_t *dst = packed + n * (K / 2) + g * (AWQ_GROUP / 2);
            for (int b = 0; b < AWQ_GROUP / 2; ++b)
                dst[b] = (uint8_t)((unsigned)q[2 * b] | ((unsigned)q[2 * b + 1] << 4));
        }
    }
}

/* Dequantized weight [N, K] in fp64: (q - z) * s. */
void oracle_awq_dequant(const uint8_t *packed, const float *scales, const uint8_t *zeros,
                        int64_t N, int64_t K, double *Wq)
{
    const int64_t G = K / AWQ_GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const unsigned byte = packed[n * (K / 2) + k / 2];
            const int q = (int)((k & 1) ? (byte >> 4) : (byte & 0xFu));
            const int64_t g = k / AWQ_GROUP;
            Wq[n * K + k] = (double)(q - (int)zeros[n * G + g]) * (double)scales[n * G + g];
        }
    }
}

/*
 * Y = X Wq^T + bias for the selected rows of X (all rows when rows == NULL):
 * per output, sum over groups of s * sum_k x * (q - z), in fp64, plus bias,
 * then one rounding to bf16.  acc (fp64) and y (bf16 bits) are
 * [nrows, N].
 */
void oracle_awq_linear_rows(const uint16_t *X, const uint8_t *packed, const float *scales,
                            const uint8_t *zeros, const uint16_t *bias, int64_t M, int64_t N,
                            int64_t K, const int64_t *rows, int64_t nrows, double *acc,
                            uint16_t *y)
{
    const int64_t G = K / AWQ_GROUP;
    (void)M;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        const int64_t m = rows ? rows[i] : i;
        const uint16_t *x = X + m * K;
        for (int64_t n = 0; n < N; ++n) {
            double total = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                const int z = (int)zeros[n * G + g];
                double dot = 0.0;
                for (int j = 0; j < AWQ_GROUP; ++j) {
                    const int64_t k = g * AWQ_GROUP + j;
                    const unsigned byte = packed[n * (K / 2) + k / 2];
                    const int q = (int)((k & 1) ? (byte >> 4) : (byte & 0xFu));
                    dot += (double)awq_bf16_to_float(x[k]) * (double)(q - z);
                }
                total += (double)scales[n * G + g] * dot;
            }
            if (bias)
                total += (double)awq_bf16_to_float(bias[n]);
            acc[i * N + n] = total;
            y[i * N + n] = oracle_bf16_rne(total);
        }
    }
}
