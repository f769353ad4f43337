/*
 * svdq_oracle.c -- plain, slow CPU reference for the SVDQuant W4A4 linear.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP implementation.
 *
 * What it computes (SVDQuant as summarized on the "svdq-int4-flux.1-canny-dev"
 * model card, section "SVDQuant overview", stages 1-3, and on the "Nunchaku
 * 4-bit in Diffusers" blog, section "Background: SVDQuant and Nunchaku"):
 * activation outliers are moved into the weights by a per-channel smoothing
 * factor lambda, the smoothed weight is split into a 16-bit low-rank branch
 * L1 L2 and a residual R, and the residual path runs with 4-bit weights AND
 * 4-bit activations (the blog's "W4A4" kernel family svdq_w4a4):
 *
 *   Y = Q4(X diag(lambda)^-1) Q4(R)^T + (X diag(lambda)^-1 L1) L2 + bias
 *
 * The pages leave the quantizer itself open; the readings used here are:
 *   - groups of 64 consecutive inputs along K, one fp32 scale per
 *     (row, group), scale = max|v| / 7, codes in [-7, 7] (symmetric
 *     round-to-nearest; -8 is never produced);
 *   - the code is rint(fl32(v * fl32(1 / scale))), ties to even; a zero
 *     scale, or a scale whose reciprocal overflows, gives all-zero codes;
 *   - smoothing is one fp32 multiply by fl32(1 / lambda);
 *   - codes are stored 4 bits each, row-major [rows, K/2] bytes; each block
 *     of 16 consecutive codes of a row takes 8 bytes, built as follows.
 *     Code e = 8h + i of the block (h = 0, 1; i = 0..7) becomes the 6-bit
 *     field 2i + h of a 96-bit image (image bits 6f .. 6f + 5 for field f):
 *     |c_e| in the field's bits 0-2, bits 3-4 zero, bit 5 set when c_e < 0
 *     (a zero code has no sign) -- the OCP FP6 E2M3 encoding of c_e / 8.
 *     Every field's bits 3-4 are zero, so image bits 0..63 carry 16 free
 *     bits, and image bits 64..95 are stored in them: bit 64 + o goes to
 *     stored bit o when bit o is a free bit of the first 32, otherwise to
 *     stored bit 32 + o (which is then a free bit).  Stored bits 0..63 are
 *     the block's 8 bytes, bit 8j + b in bit b of byte j -- the layout lets a
 *     GPU hand the codes to an FP6 matrix instruction as exact subnormals;
 *     scales row-major [rows, K/64];
 *   - the rescale, the low-rank products, bias and the erf-form GELU are
 *     taken in fp64, and the output is ONE correct rounding of that fp64
 *     value to bf16 (nearest, ties to even).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * (the float steps must be single IEEE fp32 operations, never contracted).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GROUP 64

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Image field (0..15) of code e (0..15) of a block: code 8h + i -> field
 * 2i + h. */
static int code_field(int e)
{
    return 2 * (e % 8) + e / 8;
}

/* Stored bit (0..63) of image bit p (0..95) of a block.  Bits 3 and 4 of
 * every 6-bit field are zero in the image ("free"); bits 64.. of the image
 * move into free bits at the same offset within a 32-bit word. */
static int is_free_bit(int p)
{
    return p % 6 == 3 || p % 6 == 4;
}
static int stored_bit(int p)
{
    if (p < 64)
        return p;
    const int o = p - 64;
    return is_free_bit(o) ? o : 32 + o;
}

/* Pack the 16 codes of one block into its 8 bytes. */
static void pack_block(const int *blk, uint8_t *dst)
{
    memset(dst, 0, 8);
    for (int e = 0; e < 16; ++e) {
        const unsigned v = (unsigned)abs(blk[e]) | (blk[e] < 0 ? 32u : 0u);
        for (int b = 0; b < 6; ++b)
            if (v >> b & 1u) {   /* bits 3-4 of v are zero */
                const int q = stored_bit(6 * code_field(e) + b);
                dst[q / 8] |= (uint8_t)(1u << (q % 8));
            }
    }
}

/*
 * Round a double to the nearest bf16 value (8 significant bits, fp32's
 * exponent range), ties to even, in a single step.  Returns the bf16 bit
 * pattern.  (Rounding fp64 -> fp32 -> bf16 would round twice and can land
 * one bf16 ulp away, so it is not used.)
 */
uint16_t oracle_bf16_rne(double v)
{
    if (isnan(v))
        return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return sign | 0x7F80;
    int e;
    frexp(a, &e);                  /* a in [2^(e-1), 2^e) */
    int E = e - 1;                 /* floor(log2 a) */
    if (E < -126)
        E = -126;                  /* bf16 subnormals: spacing 2^-133 */
    double q = ldexp(a, 7 - E);    /* exact; in [128, 256) for normals */
    double rq = nearbyint(q);      /* default mode: nearest, ties to even */
    double res = ldexp(rq, E - 7); /* exact */
    if (res >= ldexp(1.0, 128))
        return sign | 0x7F80;      /* rounds past the largest finite bf16 */
    float f = (float)res;          /* exact: res is a bf16 value */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return sign | (uint16_t)((u >> 16) & 0x7FFF);
}

/* GELU, erf form: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)), in fp64. */
double oracle_gelu(double x)
{
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

/*
 * Smoothing (stage 2 of the SVDQuant overview: outliers migrate from the
 * activations into the weights).  xh[m][k] = fl32(float(X[m][k]) * fl32(1/lam[k])).
 */
void oracle_smooth(const uint16_t *X, const float *lam, int64_t M, int64_t K, float *xh)
{
    float *inv = (float *)malloc((size_t)K * sizeof(float));
    for (int64_t k = 0; k < K; ++k)
        inv[k] = 1.0f / lam[k];
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            xh[m * K + k] = bf16_to_float(X[m * K + k]) * inv[k];
    free(inv);
}

/*
 * Group-wise symmetric 4-bit quantization of a row-major [rows, K] fp32
 * matrix (the 4-bit path of the W4A4 layer; used for the smoothed
 * activations and, offline, for the residual weight).  Writes packed codes
 * [rows, K/2] and scales [rows, K/64].
 */
void oracle_quantize_groups(const float *v, int64_t rows, int64_t K,
                            uint8_t *packed, float *scales)
{
    const int64_t G = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < rows; ++row) {
        for (int64_t g = 0; g < G; ++g) {
            const float *p = v + row * K + g * GROUP;
            float amax = 0.0f;
            for (int j = 0; j < GROUP; ++j) {
                float a = fabsf(p[j]);
                if (a > amax)
                    amax = a;
            }
            float s = amax / 7.0f;
            scales[row * G + g] = s;
            int q[GROUP];
            int zero = 1;
            float inv = 0.0f;
            if (s != 0.0f) {
                inv = 1.0f / s;
                zero = !isfinite(inv);
            }
            for (int j = 0; j < GROUP; ++j) {
                if (zero) {
                    q[j] = 0;
                    continue;
                }
                float y = p[j] * inv;
                float c = rintf(y);
                if (c > 7.0f)
                    c = 7.0f;
                if (c < -7.0f)
                    c = -7.0f;
                q[j] = (int)c;
            }
            uint8_t *dst = packed + row * (K / 2) + g * (GROUP / 2);
            for (int t = 0; t < GROUP / 16; ++t)
                pack_block(q + 16 * t, dst + 8 * t);
        }
    }
}

/* Decode packed codes [rows, K/2] into one int8 per element [rows, K]:
 * each code's 6-bit field read back bit by bit from its stored bits. */
void oracle_unpack(const uint8_t *packed, int64_t rows, int64_t K, int8_t *codes)
{
    for (int64_t row = 0; row < rows; ++row)
        for (int64_t t = 0; t < K / 16; ++t) {
            const uint8_t *src = packed + row * (K / 2) + 8 * t;
            for (int e = 0; e < 16; ++e) {
                unsigned v = 0;
                for (int b = 0; b < 6; ++b) {
                    if (b == 3 || b == 4)
                        continue;            /* the free bits, zero in the image */
                    const int q = stored_bit(6 * code_field(e) + b);
                    v |= (unsigned)(src[q / 8] >> (q % 8) & 1u) << b;
                }
                const int mag = (int)(v & 7u);
                codes[row * K + 16 * t + e] = (int8_t)((v & 32u) ? -mag : mag);
            }
        }
}

/*
 * Low-rank down-projection of the smoothed activations (stage 3: the
 * low-rank branch runs in 16 bits; the Nunchaku engine design reads the
 * same input for it as for quantization): xl1[m][i] = sum_k xh[m][k] L1[k][i], fp64.
 */
void oracle_down_proj(const float *xh, const uint16_t *L1, int64_t M, int64_t K,
                      int32_t r, double *xl1)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int32_t i = 0; i < r; ++i) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)xh[m * K + k] * (double)bf16_to_float(L1[k * r + i]);
            xl1[m * r + i] = acc;
        }
}

/*
 * Exact per-group integer dot products of the 4-bit codes for the output
 * block rows [m0, m0+tm) x cols [n0, n0+tn):
 *   S[(mi*tn + ni)*G + g] = sum_{k in group g} qa[m0+mi][k] * qw[n0+ni][k].
 */
void oracle_group_sums(const uint8_t *qa, const uint8_t *qw, int64_t M, int64_t N,
                       int64_t K, int64_t m0, int64_t n0, int64_t tm, int64_t tn,
                       int32_t *S)
{
    (void)M;
    (void)N;
    const int64_t G = K / GROUP;
#pragma omp parallel for schedule(static)
    for (int64_t mi = 0; mi < tm; ++mi) {
        int8_t *a = (int8_t *)malloc((size_t)K);
        int8_t *w = (int8_t *)malloc((size_t)K);
        oracle_unpack(qa + (m0 + mi) * (K / 2), 1, K, a);
        for (int64_t ni = 0; ni < tn; ++ni) {
            oracle_unpack(qw + (n0 + ni) * (K / 2), 1, K, w);
            for (int64_t g = 0; g < G; ++g) {
                int32_t s = 0;
                for (int j = 0; j < GROUP; ++j)
                    s += (int32_t)a[g * GROUP + j] * (int32_t)w[g * GROUP + j];
                S[(mi * tn + ni) * G + g] = s;
            }
        }
        free(a);
        free(w);
    }
}

/*
 * The layer output for the listed rows (rows == NULL: rows 0..nrows-1):
 *   acc[m][n] = sum_g sa[m][g] sw[n][g] S[m][n][g]        (4-bit path)
 *             + sum_i xl1[m][i] L2[i][n]                   (low-rank branch)
 *             + bias[n]                                    (bias may be NULL)
 *   acc = GELU(acc) if act == 1
 *   y = bf16 rounding of acc (one rounding, nearest-even)
 * all in fp64.  acc_out / y_out are [nrows, N] (either may be NULL).
 */
void oracle_gemm_rows(const uint8_t *qa, const float *sa, const uint8_t *qw,
                      const float *sw, const double *xl1, const uint16_t *L2,
                      const uint16_t *bias, int32_t act, int64_t M, int64_t N,
                      int64_t K, int32_t r, const int64_t *rows, int64_t nrows,
                      double *acc_out, uint16_t *y_out)
{
    (void)M;
    const int64_t G = K / GROUP;
    int8_t *wcodes = (int8_t *)malloc((size_t)(N * K));
    oracle_unpack(qw, N, K, wcodes);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t ri = 0; ri < nrows; ++ri) {
        int64_t m = rows ? rows[ri] : ri;
        int8_t *a = (int8_t *)malloc((size_t)K);
        oracle_unpack(qa + m * (K / 2), 1, K, a);
        for (int64_t n = 0; n < N; ++n) {
            const int8_t *w = wcodes + n * K;
            double acc = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                int32_t s = 0;
                for (int j = 0; j < GROUP; ++j)
                    s += (int32_t)a[g * GROUP + j] * (int32_t)w[g * GROUP + j];
                acc += (double)sa[m * G + g] * (double)sw[n * G + g] * (double)s;
            }
            for (int32_t i = 0; i < r; ++i)
                acc += xl1[m * r + i] * (double)bf16_to_float(L2[(int64_t)i * N + n]);
            if (bias)
                acc += (double)bf16_to_float(bias[n]);
            if (act == 1)
                acc = oracle_gelu(acc);
            if (acc_out)
                acc_out[ri * N + n] = acc;
            if (y_out)
                y_out[ri * N + n] = oracle_bf16_rne(acc);
        }
        free(a);
    }
    free(wcodes);
}
