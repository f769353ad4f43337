/*
 * oracle_drive.c -- calls every entry point of the CPU oracle on small seeded
 * inputs and prints a 64-bit FNV-1a hash of each output, one line per call.
 *
 * Test infrastructure: tests/test_oracle_sanitize.py builds it twice with the
 * oracle's C sources, once as the oracle is normally built and once under
 * AddressSanitizer and UndefinedBehaviorSanitizer (every buffer below is
 * allocated at exactly the size the oracle's contract states, so a read or
 * write past it is reported), and requires both runs to succeed and print
 * the same hashes.  Shapes: several groups with a ragged last tile of rows,
 * one-row and one-group cases, r = 0 and r > 0, bias on and off, GELU on and
 * off, sampled row lists, and groups whose scale is zero, subnormal (so that
 * 1/scale overflows) or near the fp32 maximum.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_bf16_rne(double v);
double oracle_gelu(double x);
void oracle_smooth(const uint16_t *X, const float *lam, int64_t M, int64_t K, float *xh);
void oracle_quantize_groups(const float *v, int64_t rows, int64_t K, uint8_t *packed,
                            float *scales);
void oracle_unpack(const uint8_t *packed, int64_t rows, int64_t K, int8_t *codes);
void oracle_down_proj(const float *xh, const uint16_t *L1, int64_t M, int64_t K, int32_t r,
                      double *xl1);
void oracle_group_sums(const uint8_t *qa, const uint8_t *qw, int64_t M, int64_t N, int64_t K,
                       int64_t m0, int64_t n0, int64_t tm, int64_t tn, int32_t *S);
void oracle_gemm_rows(const uint8_t *qa, const float *sa, const uint8_t *qw, const float *sw,
                      const double *xl1, const uint16_t *L2, const uint16_t *bias, int32_t act,
                      int64_t M, int64_t N, int64_t K, int32_t r, const int64_t *rows,
                      int64_t nrows, double *acc_out, uint16_t *y_out);
void oracle_awq_quantize(const float *W, int64_t N, int64_t K, uint8_t *packed, float *scales,
                         uint8_t *zeros);
void oracle_awq_dequant(const uint8_t *packed, const float *scales, const uint8_t *zeros,
                        int64_t N, int64_t K, double *Wq);
void oracle_awq_linear_rows(const uint16_t *X, const uint8_t *packed, const float *scales,
                            const uint8_t *zeros, const uint16_t *bias, int64_t M, int64_t N,
                            int64_t K, const int64_t *rows, int64_t nrows, double *acc,
                            uint16_t *y);
void oracle_qkv_epilogue(const double *acc, const int64_t *rows, int64_t nrows, int64_t H,
                         int64_t D, int64_t S, const uint16_t *gamma_q, const uint16_t *gamma_k,
                         double eps, const float *cos_t, const float *sin_t, double *q,
                         double *k, uint16_t *qb, uint16_t *kb, uint16_t *vb, double *rho_q,
                         double *rho_k);
int oracle_mx_e2m1_code(double y);
double oracle_mx_e2m1_value(int code);
int oracle_mx_scale_byte(double amax);
void oracle_mx_quantize(const float *v, int64_t rows, int64_t K, uint8_t *packed,
                        uint8_t *scales);
void oracle_mx_dequant(const uint8_t *packed, const uint8_t *scales, int64_t rows, int64_t K,
                       double *out);
void oracle_mx_gemm_rows(const uint8_t *qa, const uint8_t *sa, const uint8_t *qw,
                         const uint8_t *sw, const double *xl1, const uint16_t *L2,
                         const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                         int32_t r, const int64_t *rows, int64_t nrows, double *acc_out,
                         uint16_t *y_out);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

/* xorshift64*: uniform 64-bit words */
static uint64_t next_u64(void)
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}

/* uniform in [-1, 1) */
static double uniform(void) { return (double)(next_u64() >> 11) * 0x1.0p-52 - 1.0; }

/* bf16 bits of a value (truncation is enough for test inputs) */
static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static void *alloc(size_t bytes)
{
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static void report(const char *what, const void *p, size_t bytes)
{
    uint64_t h = 0xCBF29CE484222325ull;
    const uint8_t *b = (const uint8_t *)p;
    for (size_t i = 0; i < bytes; ++i) {
        h ^= b[i];
        h *= 0x100000001B3ull;
    }
    printf("%-28s %016llx\n", what, (unsigned long long)h);
}

static uint16_t *bf16_matrix(int64_t n, double scale)
{
    uint16_t *a = (uint16_t *)alloc((size_t)n * 2);
    for (int64_t i = 0; i < n; ++i)
        a[i] = to_bf16((float)(scale * uniform()));
    return a;
}

/* The W4A4 + low-rank path: smoothing, quantization, unpacking, the
 * down-projection, group sums and the layer output. */
static void drive_w4a4(int64_t M, int64_t K, int64_t N, int32_t r, int tag)
{
    char name[64];
    const int64_t G = K / 64;
    uint16_t *X = bf16_matrix(M * K, 4.0);
    /* special groups in row 0: all zero, subnormal (1/scale overflows), huge */
    for (int64_t k = 0; k < 64 && M > 0; ++k) X[k] = 0;
    if (G > 1)
        for (int64_t k = 64; k < 128; ++k) X[k] = (uint16_t)(k & 1 ? 0x0001 : 0x8003);
    if (G > 2)
        for (int64_t k = 128; k < 192; ++k) X[k] = (uint16_t)(k & 1 ? 0x7E80 : 0xFE00);
    float *lam = (float *)alloc((size_t)K * 4);
    for (int64_t k = 0; k < K; ++k) lam[k] = (float)(0.5 + 1.5 * (uniform() + 1.0));
    float *xh = (float *)alloc((size_t)(M * K) * 4);
    oracle_smooth(X, lam, M, K, xh);
    snprintf(name, sizeof name, "smooth/%d", tag);
    report(name, xh, (size_t)(M * K) * 4);

    uint8_t *qa = (uint8_t *)alloc((size_t)(M * K / 2));
    float *sa = (float *)alloc((size_t)(M * G) * 4);
    oracle_quantize_groups(xh, M, K, qa, sa);
    snprintf(name, sizeof name, "quantize_act/%d", tag);
    report(name, qa, (size_t)(M * K / 2));
    report(name, sa, (size_t)(M * G) * 4);

    float *R = (float *)alloc((size_t)(N * K) * 4);
    for (int64_t i = 0; i < N * K; ++i) R[i] = (float)(0.05 * uniform());
    uint8_t *qw = (uint8_t *)alloc((size_t)(N * K / 2));
    float *sw = (float *)alloc((size_t)(N * G) * 4);
    oracle_quantize_groups(R, N, K, qw, sw);
    snprintf(name, sizeof name, "pack_weights/%d", tag);
    report(name, qw, (size_t)(N * K / 2));
    report(name, sw, (size_t)(N * G) * 4);

    int8_t *codes = (int8_t *)alloc((size_t)(M * K));
    oracle_unpack(qa, M, K, codes);
    snprintf(name, sizeof name, "unpack/%d", tag);
    report(name, codes, (size_t)(M * K));

    uint16_t *L1 = r ? bf16_matrix(K * r, 0.1) : NULL;
    uint16_t *L2 = r ? bf16_matrix((int64_t)r * N, 0.1) : NULL;
    double *xl1 = r ? (double *)alloc((size_t)(M * r) * 8) : NULL;
    if (r) {
        oracle_down_proj(xh, L1, M, K, r, xl1);
        snprintf(name, sizeof name, "down_proj/%d", tag);
        report(name, xl1, (size_t)(M * r) * 8);
    }

    /* the whole output, then a block at the ragged corner */
    int32_t *S = (int32_t *)alloc((size_t)(M * N * G) * 4);
    oracle_group_sums(qa, qw, M, N, K, 0, 0, M, N, S);
    snprintf(name, sizeof name, "group_sums/%d", tag);
    report(name, S, (size_t)(M * N * G) * 4);
    const int64_t tm = M > 1 ? 2 : 1, tn = N > 2 ? 3 : 1;
    int32_t *Sb = (int32_t *)alloc((size_t)(tm * tn * G) * 4);
    oracle_group_sums(qa, qw, M, N, K, M - tm, N - tn, tm, tn, Sb);
    report(name, Sb, (size_t)(tm * tn * G) * 4);

    uint16_t *bias = bf16_matrix(N, 0.5);
    double *acc = (double *)alloc((size_t)(M * N) * 8);
    uint16_t *y = (uint16_t *)alloc((size_t)((M < 2 ? 2 : M) * N) * 2);   /* also 2 sampled rows */
    for (int act = 0; act < 2; ++act) {
        oracle_gemm_rows(qa, sa, qw, sw, xl1, L2, act ? bias : NULL, act, M, N, K, r, NULL, M,
                         acc, y);
        snprintf(name, sizeof name, "gemm_rows/%d/act%d", tag, act);
        report(name, acc, (size_t)(M * N) * 8);
        report(name, y, (size_t)(M * N) * 2);
    }
    int64_t rows[2] = {M - 1, 0};
    double *acc2 = (double *)alloc((size_t)(2 * N) * 8);
    oracle_gemm_rows(qa, sa, qw, sw, xl1, L2, bias, 1, M, N, K, r, rows, 2, acc2, NULL);
    snprintf(name, sizeof name, "gemm_rows/%d/rows", tag);
    report(name, acc2, (size_t)(2 * N) * 8);

    /* MXFP4: the same smoothed activations and residual, block-32 E2M1 */
    const int64_t NB = K / 32;
    uint8_t *mqa = (uint8_t *)alloc((size_t)(M * K / 2)), *msa = (uint8_t *)alloc((size_t)(M * NB));
    uint8_t *mqw = (uint8_t *)alloc((size_t)(N * K / 2)), *msw = (uint8_t *)alloc((size_t)(N * NB));
    oracle_mx_quantize(xh, M, K, mqa, msa);
    oracle_mx_quantize(R, N, K, mqw, msw);
    snprintf(name, sizeof name, "mx_quantize/%d", tag);
    report(name, mqa, (size_t)(M * K / 2));
    report(name, msa, (size_t)(M * NB));
    double *deq = (double *)alloc((size_t)(N * K) * 8);
    oracle_mx_dequant(mqw, msw, N, K, deq);
    snprintf(name, sizeof name, "mx_dequant/%d", tag);
    report(name, deq, (size_t)(N * K) * 8);
    oracle_mx_gemm_rows(mqa, msa, mqw, msw, xl1, L2, bias, 1, M, N, K, r, NULL, M, acc, y);
    snprintf(name, sizeof name, "mx_gemm_rows/%d", tag);
    report(name, acc, (size_t)(M * N) * 8);
    report(name, y, (size_t)(M * N) * 2);
    oracle_mx_gemm_rows(mqa, msa, mqw, msw, NULL, NULL, NULL, 0, M, N, K, 0, rows, 2, NULL, y);
    report(name, y, (size_t)(2 * N) * 2);

    free(X); free(lam); free(xh); free(qa); free(sa); free(R); free(qw); free(sw);
    free(codes); free(L1); free(L2); free(xl1); free(S); free(Sb); free(bias); free(acc);
    free(y); free(acc2); free(mqa); free(msa); free(mqw); free(msw); free(deq);
}

/* The W4A16 (AWQ-style) weights and layer. */
static void drive_awq(int64_t M, int64_t K, int64_t N, int tag)
{
    char name[64];
    const int64_t G = K / 64;
    float *W = (float *)alloc((size_t)(N * K) * 4);
    for (int64_t i = 0; i < N * K; ++i) W[i] = (float)(0.05 * uniform());
    for (int64_t k = 0; k < 64; ++k) W[k] = 0.0f;               /* a constant group */
    if (G > 1)
        for (int64_t k = 64; k < 128; ++k) W[k] = 0.25f;         /* all one positive value */
    uint8_t *packed = (uint8_t *)alloc((size_t)(N * K / 2)), *zeros = (uint8_t *)alloc((size_t)(N * G));
    float *scales = (float *)alloc((size_t)(N * G) * 4);
    oracle_awq_quantize(W, N, K, packed, scales, zeros);
    snprintf(name, sizeof name, "awq_quantize/%d", tag);
    report(name, packed, (size_t)(N * K / 2));
    report(name, scales, (size_t)(N * G) * 4);
    report(name, zeros, (size_t)(N * G));
    double *Wq = (double *)alloc((size_t)(N * K) * 8);
    oracle_awq_dequant(packed, scales, zeros, N, K, Wq);
    snprintf(name, sizeof name, "awq_dequant/%d", tag);
    report(name, Wq, (size_t)(N * K) * 8);
    uint16_t *X = bf16_matrix(M * K, 2.0), *bias = bf16_matrix(N, 0.5);
    double *acc = (double *)alloc((size_t)(M * N) * 8);
    uint16_t *y = (uint16_t *)alloc((size_t)(M * N) * 2);
    oracle_awq_linear_rows(X, packed, scales, zeros, bias, M, N, K, NULL, M, acc, y);
    snprintf(name, sizeof name, "awq_linear/%d", tag);
    report(name, acc, (size_t)(M * N) * 8);
    report(name, y, (size_t)(M * N) * 2);
    int64_t rows[1] = {M - 1};
    oracle_awq_linear_rows(X, packed, scales, zeros, NULL, M, N, K, rows, 1, acc, y);
    report(name, acc, (size_t)N * 8);
    free(W); free(packed); free(zeros); free(scales); free(Wq); free(X); free(bias); free(acc);
    free(y);
}

/* The QKV epilogue: per-head RMS norm and rotary turn of Q and K, V copied. */
static void drive_qkv(int64_t R, int64_t H, int64_t D, int64_t S, int tag)
{
    char name[64];
    const int64_t HD = H * D;
    double *acc = (double *)alloc((size_t)(R * 3 * HD) * 8);
    for (int64_t i = 0; i < R * 3 * HD; ++i) acc[i] = 3.0 * uniform();
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;                 /* a zero head: rho = sqrt(eps) */
    uint16_t *gq = bf16_matrix(D, 1.5), *gk = bf16_matrix(D, 1.5);
    float *ct = (float *)alloc((size_t)(S * D / 2) * 4), *st = (float *)alloc((size_t)(S * D / 2) * 4);
    for (int64_t i = 0; i < S * D / 2; ++i) {
        const double a = 3.0 * uniform();
        ct[i] = (float)cos(a);
        st[i] = (float)sin(a);
    }
    double *q = (double *)alloc((size_t)(R * HD) * 8), *k = (double *)alloc((size_t)(R * HD) * 8);
    uint16_t *qb = (uint16_t *)alloc((size_t)(R * HD) * 2), *kb = (uint16_t *)alloc((size_t)(R * HD) * 2);
    uint16_t *vb = (uint16_t *)alloc((size_t)(R * HD) * 2);
    double *rq = (double *)alloc((size_t)(R * H) * 8), *rk = (double *)alloc((size_t)(R * H) * 8);
    oracle_qkv_epilogue(acc, NULL, R, H, D, S, gq, gk, 1e-6, ct, st, q, k, qb, kb, vb, rq, rk);
    snprintf(name, sizeof name, "qkv_epilogue/%d", tag);
    report(name, q, (size_t)(R * HD) * 8);
    report(name, k, (size_t)(R * HD) * 8);
    report(name, qb, (size_t)(R * HD) * 2);
    report(name, kb, (size_t)(R * HD) * 2);
    report(name, vb, (size_t)(R * HD) * 2);
    report(name, rq, (size_t)(R * H) * 8);
    report(name, rk, (size_t)(R * H) * 8);
    /* token rows past the sequence length (positions wrap), only some outputs */
    int64_t rows[2] = {3 * S + 1, 0};
    const int64_t n = R < 2 ? R : 2;
    oracle_qkv_epilogue(acc, rows, n, H, D, S, gq, gk, 0.0, ct, st, NULL, NULL, qb, NULL, NULL,
                        NULL, rk);
    report(name, qb, (size_t)(n * HD) * 2);
    free(acc); free(gq); free(gk); free(ct); free(st); free(q); free(k); free(qb); free(kb);
    free(vb); free(rq); free(rk);
}

static void drive_scalars(void)
{
    static const double v[] = {0.0, -0.0, 1.0, -1.5, 3.0e38, 3.4e38, 1.0e-40, 1.0e-45,
                               INFINITY, -INFINITY, NAN, 0.1, 7.0, -6.0, 2.5, 1.0e300};
    const int n = (int)(sizeof v / sizeof v[0]);
    uint16_t b[16];
    double gl[16];
    int code[16], sb[16];
    double val[16];
    for (int i = 0; i < n; ++i) {
        b[i] = oracle_bf16_rne(v[i]);
        gl[i] = isfinite(v[i]) && fabs(v[i]) < 1e30 ? oracle_gelu(v[i]) : 0.0;
        code[i] = isfinite(v[i]) ? oracle_mx_e2m1_code(v[i]) : 0;
        sb[i] = isfinite(v[i]) ? oracle_mx_scale_byte(fabs(v[i])) : 0;
        val[i] = oracle_mx_e2m1_value(i);
    }
    report("bf16_rne", b, sizeof b);
    report("gelu", gl, sizeof gl);
    report("mx_e2m1_code", code, sizeof code);
    report("mx_scale_byte", sb, sizeof sb);
    report("mx_e2m1_value", val, sizeof val);
}

int main(void)
{
    drive_scalars();
    drive_w4a4(5, 192, 7, 3, 0);     /* three groups, ragged rows and columns, r > 0 */
    drive_w4a4(1, 64, 1, 0, 1);      /* one row, one group, one column, r = 0 */
    drive_w4a4(9, 320, 4, 16, 2);
    drive_awq(3, 192, 5, 0);
    drive_awq(1, 64, 1, 1);
    drive_qkv(3, 2, 8, 2, 0);
    drive_qkv(1, 1, 2, 1, 1);
    return 0;
}
