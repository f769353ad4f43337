/*
 * qkv_oracle.c -- plain, slow CPU reference for the fused QKV epilogue:
 * per-head RMS normalization of Q and K, rotary position embedding of Q and
 * K, and the attention layout, applied to the exact output of the fused QKV
 * projection.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code, header, table or constant
 * with the HIP implementation.
 *
 * The "Bringing Nunchaku 4-bit inference to Diffusers" blog (its section on
 * the structural rewrites Nunchaku needs, with the to_q / to_k / to_v and
 * fused_qkv_norm_rottary listings) describes the operation: Q, K and V come
 * from one fused projection, are split into heads, Q and K go through
 * norm_q / norm_k and then the rotary embedding, and Nunchaku does all of it
 * in one fused operator.  The pages do not define the norm, its epsilon, the
 * rotary convention or the output layout.  The readings used here:
 *   - the fused projection's columns are [Q | K | V], each H heads of D
 *     consecutive columns (head h of Q is columns h D .. h D + D - 1);
 *   - norm_q / norm_k are RMS norms over the D values of one token and head
 *     with a learned bf16 weight gamma [D]:
 *         v_d = x_d gamma_d / sqrt(mean_d(x_d^2) + eps);
 *   - the rotary embedding turns each adjacent pair (2p, 2p + 1) of a head
 *     by the angle whose cosine and sine the caller gives per position s
 *     and pair p (fp32 tables [S, D/2]):
 *         (a, b) -> (a cos - b sin, a sin + b cos);
 *   - tokens are m = b S + s (batch b, position s); the outputs are bf16
 *     Q, K, V in the attention layout [B, H, S, D];
 *   - everything is taken in fp64 from the projection's exact value (bias
 *     included), with ONE correct rounding to bf16 at the end; V is that
 *     value rounded, only re-laid out.
 *
 * Build: compiled into the same library as svdq_oracle.c.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

uint16_t oracle_bf16_rne(double v); /* svdq_oracle.c */

static double qkv_bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * acc  [nrows, 3 H D] fp64: the exact projection output of the tokens rows[i]
 *      (rows == NULL: token i)
 * gamma_q, gamma_k  bf16 [D];  cos_t, sin_t  fp32 [S, D/2]
 * Outputs (any may be NULL), one entry per (row i, head h, d):
 *   q, k     fp64 [nrows, H, D] before rounding;  qb, kb, vb  bf16 bits [nrows, H, D]
 *   rho_q, rho_k  fp64 [nrows, H]: sqrt(mean(x^2) + eps) of each head
 * (the caller places row i at token rows[i] of the [B, H, S, D] layout).
 */
void oracle_qkv_epilogue(const double *acc, const int64_t *rows, int64_t nrows, int64_t H,
                         int64_t D, int64_t S, const uint16_t *gamma_q, const uint16_t *gamma_k,
                         double eps, const float *cos_t, const float *sin_t, double *q,
                         double *k, uint16_t *qb, uint16_t *kb, uint16_t *vb, double *rho_q,
                         double *rho_k)
{
    const int64_t HD = H * D;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        const int64_t m = rows ? rows[i] : i;
        const int64_t s = m % S;
        const double *a = acc + i * 3 * HD;
        for (int64_t h = 0; h < H; ++h) {
            for (int which = 0; which < 2; ++which) {
                const double *x = a + which * HD + h * D;
                const uint16_t *gamma = which == 0 ? gamma_q : gamma_k;
                double ss = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    ss += x[d] * x[d];
                const double rho = sqrt(ss / (double)D + eps);
                for (int64_t p = 0; p < D / 2; ++p) {
                    const double c = (double)cos_t[s * (D / 2) + p];
                    const double sn = (double)sin_t[s * (D / 2) + p];
                    const double va = x[2 * p] / rho * qkv_bf16_value(gamma[2 * p]);
                    const double vbv = x[2 * p + 1] / rho * qkv_bf16_value(gamma[2 * p + 1]);
                    const double o0 = va * c - vbv * sn;
                    const double o1 = va * sn + vbv * c;
                    const int64_t at = (i * H + h) * D + 2 * p;
                    if (which == 0) {
                        if (q) { q[at] = o0; q[at + 1] = o1; }
                        if (qb) { qb[at] = oracle_bf16_rne(o0); qb[at + 1] = oracle_bf16_rne(o1); }
                    } else {
                        if (k) { k[at] = o0; k[at + 1] = o1; }
                        if (kb) { kb[at] = oracle_bf16_rne(o0); kb[at + 1] = oracle_bf16_rne(o1); }
                    }
                }
                if (which == 0 && rho_q) rho_q[i * H + h] = rho;
                if (which == 1 && rho_k) rho_k[i * H + h] = rho;
            }
            if (vb)
                for (int64_t d = 0; d < D; ++d)
                    vb[(i * H + h) * D + d] = oracle_bf16_rne(a[2 * HD + h * D + d]);
        }
    }
}
