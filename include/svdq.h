/*
 * svdq.h -- C ABI of the MI355X (gfx950) SVDQuant W4A4 + low-rank linear layer.
 *
 * The layer (SVDQuant: "svdq-int4-flux.1-canny-dev" model card, section
 * "SVDQuant overview", stages 1-3; "Nunchaku 4-bit in Diffusers" blog,
 * sections "Background: SVDQuant and Nunchaku" and "Introducing Nunchaku
 * Lite", kernel family svdq_w4a4) computes, for activations X [M, K]:
 *
 *   Xs = X diag(lambda)^-1                       smoothing (stage 2)
 *   Y  = Q4(Xs) Q4(R)^T  +  (Xs L1) L2  +  bias  4-bit residual path plus the
 *                                                16-bit rank-r branch (stage 3)
 *   Y  = GELU(Y) optionally (erf form)
 *
 * Q4 is symmetric group quantization along K: groups of 64 consecutive
 * inputs, one fp32 scale s = max|v| / 7 per (row, group), code
 * q = rint(fl32(v * fl32(1/s))) (ties to even) in [-7, 7]; s == 0, or a
 * 1/s that is not finite, gives all-zero codes.  The pages leave these
 * details open; this is the reading the library implements and its tests
 * pin.  The product of the two quantized operands is taken as an exact
 * integer sum per group, S[m][n][g] = sum_{k in g} qa[m][k] qw[n][k], then
 * rescaled: Y_4bit[m][n] = sum_g sa[m][g] sw[n][g] S[m][n][g].
 *
 * The engine-design section of the model card fuses the low-rank
 * down-projection with quantization (they read the same input) and the
 * up-projection with the 4-bit product (they write the same output); the
 * entry points below follow that split: svdq_quantize_act_down reads X once
 * and emits codes, scales and X L1; svdq_w4a4_lr_gemm runs the 4-bit GEMM and
 * adds the low-rank up-projection, bias and activation to the same output
 * tile before its single bf16 store.  svdq_linear runs both.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns; all tensors are
 *     row-major and contiguous.  Pointers marked "device" must point to
 *     memory of the current HIP device and be 16-byte aligned.
 *   - Packed INT4 codes (qa, qw): kb = K/2 bytes per row, 4 bits per
 *     code; each block of 16 consecutive codes of a row takes 8 bytes, two
 *     little-endian words W0, W1.  Code e = 8h + i of the block (h = 0, 1;
 *     i = 0..7) is field 2i + h of a 96-bit image, bits 6f .. 6f + 5 for
 *     field f, holding the FP6 E2M3 encoding of c_e / 8: |c_e| in bits 0-2,
 *     bits 3-4 zero, bit 5 set when c_e < 0 (zero is stored without sign).
 *     With the image words I0, I1, I2 (bits 0-31, 32-63, 64-95),
 *     W0 = I0 | (I2 & 0x18618618) and W1 = I1 | (I2 & 0x86186186): the
 *     masks are the always-zero bits 3-4 of the fields of I0 and of I1
 *     (positions p with p mod 6 = 3 or 4), disjoint, and together every bit
 *     I2 can hold.  With this layout the GEMM unfolds the codes into FP6
 *     operands of the matrix unit with four bit operations per 16 codes.
 *     Rows are stored in pairs, [ceil(rows/2),
 *     2 kb] = [ceil(rows/2), K] bytes: each 64-byte chunk of a row (128
 *     codes, one stage of the GEMM) is followed by the same chunk of its
 *     pair partner, so one 128-byte line holds a stage of both rows; when
 *     kb is not a multiple of 64 (an odd group count) the last chunk is 32
 *     bytes and the pair interleaves in 32-byte halves there.  Byte b of row
 *     i sits at (i/2) 2 kb + (b/64) 128 + (i%2) w + b%64, with w = 64, or
 *     kb - 64 (b/64) in a shorter last chunk.  An odd row count's last pair
 *     has an unwritten half.
 *   - Group scales (sa, sw) are stored stage-major in pairs: for R rows and
 *     G = K/64 groups, fp32 [ceil(G/2), R, 2]; the scale of (row i, group g)
 *     is element ((g/2) R + i) 2 + g%2, so that the scales of two consecutive
 *     groups of consecutive rows (one stage of the GEMM's K loop for one tile)
 *     are one contiguous run of 8 bytes per row.  With an odd G the elements
 *     (i, G) of the last stage are padding, written as zero by the producers
 *     of sa and sw.  ceil(G/2) R 2 floats in all.
 *   - The caller owns and allocates every buffer.  The library allocates
 *     nothing and keeps no state except a per-device architecture check.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream)
 *     and the call returns without synchronizing.  Outputs are defined once
 *     the stream reaches that point.
 *   - Every argument is validated before anything is launched, so an error
 *     status means no output was written.  Arguments are checked first,
 *     then the device: argument errors are reported on any host.
 *   - Outputs must not alias inputs.  Calls on different streams may run
 *     concurrently when their buffers are disjoint.
 *   - Results are deterministic: no atomics take part in any sum, so two
 *     runs with the same inputs give bitwise identical outputs.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVDQ_ABI_VERSION 4
#define SVDQ_GROUP 64      /* quantization group along K */
#define SVDQ_MAX_RANK 128  /* largest supported low-rank r */
/* Size limits, so that every offset the kernels form within a tile fits its
 * integer type: K (in-features) at most 2^20, and M (tokens) and N
 * (out-features) at most 2^28 each.  Larger sizes are rejected with
 * SVDQ_ERR_UNSUPPORTED_SHAPE, and so are shapes inside these limits whose
 * launches would need more than 2^32 - 1 work-items (a dispatch's grid size;
 * e.g. the GEMM at M = 2^28 with N = 2^16: far beyond any device memory). */
#define SVDQ_MAX_K (1 << 20)
#define SVDQ_MAX_ROWS (1 << 28)

typedef enum {
    SVDQ_OK = 0,
    SVDQ_ERR_INVALID_ARG = 1,       /* NULL pointer where data is needed, negative size, bad act */
    SVDQ_ERR_UNSUPPORTED_SHAPE = 2, /* K % 64 != 0, K < 64, N % 8 != 0, r not a multiple of 16 or > 128, a size past SVDQ_MAX_K / SVDQ_MAX_ROWS, a launch past 2^32 - 1 work-items */
    SVDQ_ERR_MISALIGNED = 3,        /* a device pointer not 16-byte aligned */
    SVDQ_ERR_WORKSPACE_TOO_SMALL = 4,
    SVDQ_ERR_UNSUPPORTED_DEVICE = 5, /* current device is not gfx950 (or no device) */
    SVDQ_ERR_HIP = 6                 /* HIP runtime / launch error, see svdq_last_error() */
} svdq_status;

typedef enum {
    SVDQ_ACT_NONE = 0,
    SVDQ_ACT_GELU = 1 /* 0.5 x (1 + erf(x / sqrt 2)) */
} svdq_act;

/* ABI version (SVDQ_ABI_VERSION). */
int32_t svdq_abi_version(void);

/* Static, human-readable name of a status code. */
const char *svdq_status_string(int32_t status);

/* Detail of the last error on the calling thread ("" if none). Valid until
 * the next call on this thread. */
const char *svdq_last_error(void);

/*
 * Offline weight preparation of the 4-bit residual (stage 3 of the SVDQuant
 * overview; the offline toolchain's "quantize, pack" steps in the blog's
 * section "Quantize your own model").
 *   R   device fp32 [N, K]  residual weight (nn.Linear orientation, out x in),
 *                           finite (a NaN or an infinity gives unspecified
 *                           codes and scales)
 *   qw  device u8   [ceil(N/2), K] packed 4-bit codes, row pairs (out)
 *   sw  device fp32 [ceil(K/128), N, 2] group scales, stage-major (out)
 * Same quantizer as the activations, without smoothing.  N >= 0 (0: no-op),
 * K % 64 == 0, K >= 64.
 */
int32_t svdq_pack_weights(const float *R, int64_t N, int64_t K, uint8_t *qw, float *sw,
                          void *stream);

/*
 * Weights already quantized elsewhere (e.g. a checkpoint's packed INT4
 * residual) in the common row-major form -> the stored layouts above.
 *   codes   device u8   [N, K/2]  two's-complement nibbles, element 2j in the
 *                                 low nibble of byte j, codes in [-7, 7] (a -8
 *                                 nibble is stored as -7)
 *   scales  device fp32 [N, K/64] group scales, row-major
 *   qw      device u8   [ceil(N/2), K] packed codes, row pairs (out)
 *   sw      device fp32 [ceil(K/128), N, 2] group scales, stage-major (out)
 * A pure re-arrangement: svdq_pack_weights(R) equals this applied to the
 * row-major codes and scales of the same quantization.  N >= 0 (0: no-op),
 * K % 64 == 0, K >= 64.
 */
int32_t svdq_repack_weights(const uint8_t *codes, const float *scales, int64_t N, int64_t K,
                            uint8_t *qw, float *sw, void *stream);

/*
 * Workspace bytes svdq_quantize_act_down needs: when K spans more than one
 * chunk of groups and r > 0, the chunks' partial fp32 sums of the
 * down-projection (chunks x M x r floats, 256-byte aligned); otherwise 0.
 */
size_t svdq_quantize_act_down_workspace_bytes(int64_t M, int64_t K, int32_t r);

/*
 * Smoothing, activation quantization and low-rank down-projection in one
 * pass over X (model card, section "Nunchaku engine design", item (b): the
 * down-projection and the quantizer share their input).
 *   X       device bf16 [M, K]   activations, finite (a NaN or an infinity
 *                                gives unspecified codes and scales)
 *   lambda  device fp32 [K]      smoothing factors, finite and > 0
 *   L1      device bf16 [K, r]   low-rank down factor (NULL iff r == 0)
 *   qa      device u8   [ceil(M/2), K] packed codes of X diag(lambda)^-1 (out)
 *   sa      device fp32 [ceil(K/128), M, 2] group scales, stage-major (out)
 *   xl1     device fp32 [M, r]   (X diag(lambda)^-1) L1, fp32 (out; NULL iff r == 0)
 *   workspace / ws_bytes  device scratch of at least
 *           svdq_quantize_act_down_workspace_bytes(M, K, r) bytes (may be
 *           NULL when that is 0)
 * M >= 0 (0: no-op), K % 64 == 0, r in {0, 16, 32, ..., 128}.
 * qa and sa are bit-exact with the definition above; xl1 is accurate to
 * about 2^-16 relative per term (bf16 hi/lo products, fp32 sums).
 */
int32_t svdq_quantize_act_down(const uint16_t *X, const float *lambda, const uint16_t *L1,
                               int64_t M, int64_t K, int32_t r, uint8_t *qa, float *sa,
                               float *xl1, void *workspace, size_t ws_bytes, void *stream);

/*
 * The W4A4 GEMM with the low-rank up-projection, bias and activation in its
 * epilogue (model card, section "Nunchaku engine design", item (b): the
 * up-projection and the 4-bit compute share their output).
 *   qa, sa     device  codes / scales of the activations (from svdq_quantize_act_down)
 *   qw, sw     device  codes / scales of the residual weight (from svdq_pack_weights)
 *   xl1        device fp32 [M, r]  (NULL iff r == 0)
 *   L2         device bf16 [r, N]  low-rank up factor (NULL iff r == 0)
 *   bias       device bf16 [N] or NULL
 *   act        svdq_act
 *   Y          device bf16 [M, N]  output (out)
 * M >= 0 (0: no-op), N % 8 == 0, N >= 8, K % 64 == 0, r in {0, 16, ..., 128}.
 * Y = act(sum_g sa sw S + xl1 L2 + bias), accumulated in fp32 and rounded
 * once to bf16 (nearest even).
 */
int32_t svdq_w4a4_lr_gemm(const uint8_t *qa, const float *sa, const uint8_t *qw,
                          const float *sw, const float *xl1, const uint16_t *L2,
                          const uint16_t *bias, int32_t act, int64_t M, int64_t N,
                          int64_t K, int32_t r, uint16_t *Y, void *stream);

/* Workspace bytes svdq_linear needs for a given shape (qa, sa, xl1 and the
 * down-projection scratch, each 256-byte aligned). */
size_t svdq_linear_workspace_bytes(int64_t M, int64_t K, int32_t r);

/*
 * The whole layer: svdq_quantize_act_down then svdq_w4a4_lr_gemm on the same
 * stream, with qa/sa/xl1 carved out of `workspace`
 * (>= svdq_linear_workspace_bytes(M, K, r) bytes).  Arguments as above.
 */
int32_t svdq_linear(const uint16_t *X, const float *lambda, const uint16_t *L1,
                    const uint8_t *qw, const float *sw, const uint16_t *L2,
                    const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                    int32_t r, uint16_t *Y, void *workspace, size_t ws_bytes, void *stream);

/*
 * svdq_linear for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the intermediates that svdq_linear carves out of the caller's workspace
 * live instead in a static device array of SVDQ_NOALLOC_SCRATCH_BYTES bytes
 * inside the library, one per device, held from the library's load until the
 * process ends.  The call allocates nothing (no hipMalloc / hipFree, no
 * allocating library routine).  Arguments as svdq_linear, without the
 * workspace.  Shapes whose svdq_linear_workspace_bytes(M, K, r) exceeds
 * SVDQ_NOALLOC_SCRATCH_BYTES are rejected with SVDQ_ERR_WORKSPACE_TOO_SMALL
 * before anything runs.  Every call on one device shares that device's
 * array: calls that overlap in time on one device (other streams, other
 * threads) race and must be serialized by the caller.  No part of the array
 * needs to start at zero.  Results are bitwise identical to svdq_linear's.
 */
#define SVDQ_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int32_t svdq_linear_noalloc(const uint16_t *X, const float *lambda, const uint16_t *L1,
                            const uint8_t *qw, const float *sw, const uint16_t *L2,
                            const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                            int32_t r, uint16_t *Y, void *stream);

/* ------------------------------------------------------------------
 * Fused QKV epilogue.  The blog "Bringing Nunchaku 4-bit inference to
 * Diffusers" (its section on the structural rewrites, the to_q / to_k /
 * to_v and fused_qkv_norm_rottary listings) fuses the Q, K and V
 * projections into one SVDQuant layer whose operator also applies norm_q /
 * norm_k and the rotary embedding.  The pages fix neither the norm nor the
 * rotary convention; here:
 *   - the projection's N = 3 H D columns are [Q | K | V], head h of a
 *     section being its columns h D .. h D + D - 1;
 *   - Q and K: per token m and head, v_d = x_d gamma_d / sqrt(mean(x^2) + eps)
 *     (RMS norm over the head, bias included in x), then every adjacent pair
 *     (2p, 2p + 1) turns: (a, b) -> (a cos - b sin, a sin + b cos) with
 *     cos_t / sin_t [s][p] of the token's position s = m mod S;
 *   - outputs are bf16 in the attention layout [B, H, S, D], M = B S.
 * The norm and the turn act on the fp32 tile before its one bf16 rounding.
 * ------------------------------------------------------------------ */
typedef struct svdq_qkv_epilogue {
    int32_t heads;            /* H >= 1 */
    int32_t head_dim;         /* D: 64 or 128, with H D % 128 == 0 */
    int64_t seq;              /* S >= 1 tokens per sequence, M % S == 0 */
    const uint16_t *gamma_q;  /* device bf16 [D] */
    const uint16_t *gamma_k;  /* device bf16 [D] */
    float eps;                /* >= 0, finite */
    const float *cos_t;       /* device fp32 [S, D/2] */
    const float *sin_t;       /* device fp32 [S, D/2] */
    uint16_t *q;              /* device bf16 [M/S, H, S, D] (out) */
    uint16_t *k;              /* device bf16 [M/S, H, S, D] (out) */
    uint16_t *v;              /* device bf16 [M/S, H, S, D] (out) */
} svdq_qkv_epilogue;

/*
 * The W4A4 GEMM of svdq_w4a4_lr_gemm (N = 3 H D, no activation) with the
 * fused QKV epilogue instead of the [M, N] store.  epi is a host pointer,
 * read during the call only; its device pointers must be 16-byte aligned.
 * Errors as svdq_w4a4_lr_gemm, plus SVDQ_ERR_INVALID_ARG / _UNSUPPORTED_SHAPE
 * for a bad epilogue.  Q and K within 1 bf16 ulp plus the propagated GEMM
 * error (the GEMM tolerance divided by the head's rms); V as Y.
 */
int32_t svdq_w4a4_lr_gemm_qkv(const uint8_t *qa, const float *sa, const uint8_t *qw,
                              const float *sw, const float *xl1, const uint16_t *L2,
                              const uint16_t *bias, int64_t M, int64_t K, int32_t r,
                              const svdq_qkv_epilogue *epi, void *stream);

/*
 * The whole fused QKV layer: svdq_quantize_act_down then
 * svdq_w4a4_lr_gemm_qkv on one stream, intermediates in the caller's
 * workspace of svdq_linear_workspace_bytes(M, K, r) bytes.
 */
int32_t svdq_linear_qkv(const uint16_t *X, const float *lambda, const uint16_t *L1,
                        const uint8_t *qw, const float *sw, const uint16_t *L2,
                        const uint16_t *bias, int64_t M, int64_t K, int32_t r,
                        const svdq_qkv_epilogue *epi, void *workspace, size_t ws_bytes,
                        void *stream);

/* ------------------------------------------------------------------
 * MLP chain.  The blog "Bringing Nunchaku 4-bit inference to Diffusers"
 * (section "Background: SVDQuant and Nunchaku") credits fused GELU/MLP paths
 * for Nunchaku's native speed, and the model card's "Nunchaku engine design"
 * fuses a layer's down-projection with its quantizer because both read the
 * same input.  Here the MLP-up GEMM runs the MLP-down layer's activation step
 * (svdq_quantize_act_down's smoothing, INT4 codes, scales and X L1) on its
 * own output tiles, so the [M, N] intermediate is never written: the codes,
 * scales and xl1 are bit-identical to (xl1: within the bound of)
 * svdq_quantize_act_down applied to what svdq_w4a4_lr_gemm would have stored.
 * ------------------------------------------------------------------ */

/* Workspace (partial down-projections) of svdq_w4a4_lr_gemm_quant_down. */
size_t svdq_w4a4_lr_gemm_quant_down_workspace_bytes(int64_t M, int64_t N, int32_t r_next);

/*
 * The GEMM of svdq_w4a4_lr_gemm (arguments as there, Y omitted) followed by
 * the next layer's activation step on Y:
 *   lambda_next  device fp32 [N]          the next layer's smoothing factors
 *   L1_next      device bf16 [N, r_next]  its down-projection (NULL if r_next == 0)
 *   qa_next      device u8   [ceil(M/2), N] its codes, row pairs (out)
 *   sa_next      device fp32 [N/128, M, 2] its scales, stage-major (out)
 *   xl1_next     device fp32 [M, r_next]  its down-projection (out; NULL if r_next == 0)
 *   workspace    device, svdq_w4a4_lr_gemm_quant_down_workspace_bytes(M, N, r_next)
 * Needs N % 128 == 0 and r_next in {0, 16, 32}; otherwise as svdq_w4a4_lr_gemm.
 */
int32_t svdq_w4a4_lr_gemm_quant_down(const uint8_t *qa, const float *sa, const uint8_t *qw,
                                     const float *sw, const float *xl1, const uint16_t *L2,
                                     const uint16_t *bias, int32_t act, int64_t M, int64_t N,
                                     int64_t K, int32_t r, const float *lambda_next,
                                     const uint16_t *L1_next, int32_t r_next, uint8_t *qa_next,
                                     float *sa_next, float *xl1_next, void *workspace,
                                     size_t ws_bytes, void *stream);

/* Workspace of svdq_mlp. */
size_t svdq_mlp_workspace_bytes(int64_t M, int64_t K, int64_t N_hidden, int32_t r_up,
                                int32_t r_down);

/*
 * A whole MLP of two SVDQuant layers: Y = down(act(up(X))), up: K -> N_hidden
 * (activation act, bias_up), down: N_hidden -> K (no activation, bias_down).
 * Three launches on one stream (plus the reduce launches of the
 * down-projections): K1 of the up layer, the up GEMM with the down layer's
 * activation step in its epilogue, the down GEMM.  Arguments per layer as in
 * svdq_linear; Y device bf16 [M, K] (out).  Needs N_hidden % 128 == 0 and
 * r_down in {0, 16, 32}.
 */
int32_t svdq_mlp(const uint16_t *X, const float *lambda_up, const uint16_t *L1_up,
                 const uint8_t *qw_up, const float *sw_up, const uint16_t *L2_up,
                 const uint16_t *bias_up, const float *lambda_down, const uint16_t *L1_down,
                 const uint8_t *qw_down, const float *sw_down, const uint16_t *L2_down,
                 const uint16_t *bias_down, int32_t act, int64_t M, int64_t K, int64_t N_hidden,
                 int32_t r_up, int32_t r_down, uint16_t *Y, void *workspace, size_t ws_bytes,
                 void *stream);

/* ------------------------------------------------------------------
 * The 4-bit float variant (MXFP4).  The blog "Bringing Nunchaku 4-bit
 * inference to Diffusers" (section "Introducing Nunchaku Lite" and the
 * quantization_config listing) gives svdq_w4a4 a 4-bit float variant beside
 * INT4, for GPUs with native 4-bit float arithmetic, and leaves its scale
 * format open.  The 4-bit float form with matrix-core support on gfx950 is
 * MXFP4 of the OCP Microscaling Formats (MX) specification v1.0, which these
 * entry points use:
 *   - blocks of 32 consecutive values along K share one scale 2^e, stored
 *     as the E8M0 byte e + 127, e = floor(log2 max|v|) - 2 clamped to
 *     [-127, 127]; an all-zero block gets the byte 0 and zero codes;
 *   - each value becomes the E2M1 number (magnitudes 0, 0.5, 1, 1.5, 2, 3,
 *     4, 6; sign in bit 3) nearest to v / 2^e, ties to the even code,
 *     magnitudes above 6 to 6; zero is stored as +0 (inputs must be
 *     finite: a NaN or an infinity gives unspecified codes and scales);
 *   - E2M1 codes two per byte, element 2j in the low nibble of byte j of
 *     its row (the scaled matrix instruction takes them as they are); rows
 *     stored in pairs as the INT4 codes (K % 128 == 0, so every chunk is 64
 *     bytes): byte b of row i sits at (i / 2) K + (b / 64) 128 + (i % 2) 64
 *     + b % 64; scales u8 block-major, [K/32, P] with
 *     P = rows rounded up to a multiple of 16: byte [b][i] scales k block b
 *     of row i; bytes [b][rows .. P) are padding, left unwritten and never
 *     read into a result.  (Row-major bytes would cost the GEMM one memory
 *     request per row and k step, as many as the codes.)
 * Y = act(sum_blocks 2^(ea + ew) sum_k a_k w_k + xl1 L2 + bias), with the
 * smoothing, rank-r branch, bias and activation of the INT4 path; the block
 * sums are formed by the matrix unit in fp32.  K % 128 == 0 throughout.
 * Errors as the INT4 entry points, plus SVDQ_ERR_UNSUPPORTED_SHAPE for K.
 * ------------------------------------------------------------------ */

/* Offline MXFP4 quantization of the residual R (device fp32 [N, K]): codes
 * qw [ceil(N/2), K] (row pairs), scale bytes sw [K/32, roundup(N, 16)]
 * (device, out).  N >= 0 (0: no-op). */
int32_t svdq_mx_pack_weights(const float *R, int64_t N, int64_t K, uint8_t *qw, uint8_t *sw,
                             void *stream);

/* svdq_quantize_act_down with the MXFP4 quantizer: qa [ceil(M/2), K] (row
 * pairs), sa u8 [K/32, roundup(M, 16)] (device, out; bit-exact with the
 * definition above), xl1 as
 * there.  Workspace: svdq_quantize_act_down_workspace_bytes(M, K, r). */
int32_t svdq_mx_quantize_act_down(const uint16_t *X, const float *lambda, const uint16_t *L1,
                                  int64_t M, int64_t K, int32_t r, uint8_t *qa, uint8_t *sa,
                                  float *xl1, void *workspace, size_t ws_bytes, void *stream);

/* svdq_w4a4_lr_gemm on MXFP4 operands (sa u8 [K/32, roundup(M, 16)], sw u8
 * [K/32, roundup(N, 16)]);
 * other arguments and shape rules as there.  Y is accumulated in fp32 and
 * rounded once to bf16. */
int32_t svdq_mx_lr_gemm(const uint8_t *qa, const uint8_t *sa, const uint8_t *qw,
                        const uint8_t *sw, const float *xl1, const uint16_t *L2,
                        const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                        int32_t r, uint16_t *Y, void *stream);

/* Workspace bytes of svdq_mx_linear (qa, sa, xl1, down-projection scratch). */
size_t svdq_mx_linear_workspace_bytes(int64_t M, int64_t K, int32_t r);

/* The whole MXFP4 layer: svdq_mx_quantize_act_down, then svdq_mx_lr_gemm on
 * the same stream, intermediates carved out of `workspace`. */
int32_t svdq_mx_linear(const uint16_t *X, const float *lambda, const uint16_t *L1,
                       const uint8_t *qw, const uint8_t *sw, const uint16_t *L2,
                       const uint16_t *bias, int32_t act, int64_t M, int64_t N, int64_t K,
                       int32_t r, uint16_t *Y, void *workspace, size_t ws_bytes, void *stream);

/*
 * Test hook: the exact per-group integer sums of a block, taken from the
 * GEMM's own tile code (the same global -> LDS staging, code layout, FP6
 * operand form and matrix instruction as svdq_w4a4_lr_gemm; 128 x 128 tiles,
 * or 64 x 64 under SVDQ_TILES_QUARTER), one launch per group of 64.
 *   qa, sa, qw, sw  device codes and scales as svdq_w4a4_lr_gemm takes them
 *                   (the scales are staged as in the GEMM; the sums do not
 *                   depend on them)
 *   S  device int32 [tm, tn, K/64]: S[i][j][g] = sum_{k in g} qa[m0+i][k] qw[n0+j][k]
 * Requires 0 <= m0, m0 + tm <= M, 0 <= n0, n0 + tn <= N.
 */
int32_t svdq_debug_group_sums(const uint8_t *qa, const float *sa, const uint8_t *qw,
                              const float *sw, int64_t M, int64_t N, int64_t K, int64_t m0,
                              int64_t n0, int64_t tm, int64_t tn, int32_t *S, void *stream);

/* ------------------------------------------------------------------
 * 4-bit weights, 16-bit activations (W4A16).  The blog "Bringing Nunchaku
 * 4-bit inference to Diffusers", section "Introducing Nunchaku Lite", names
 * this second layer kind (awq_w4a16) for the adaptive-normalization and
 * modulation projections; its quantization_config gives int4 and group
 * size 64.  The pages fix no more than that; the format here: asymmetric
 * codes q in [0, 15] per group of 64 along K, an fp32 scale s and a u8
 * zero point z per (row, group), weight = (q - z) s, over a range that
 * always contains zero.
 * ------------------------------------------------------------------ */

/*
 * The packed W4A16 weight ("records").  The columns are cut into NB =
 * ceil(N/16) blocks of 16 and K into GQ = ceil(K/256) quads of 4 groups;
 * block b, quad t is one 2368-byte record at byte (b * GQ + t) * 2368.  For
 * column c = n - 16 b, group j = g - 4 t and k = 64 g + 16 s + 8 h + e
 * (s, h, e in [0,4) x [0,2) x [0,8)):
 *   code   in the 32-bit word at byte 1024 (j / 2) + 16 (c + 16 s)
 *          + 8 (j % 2) + 4 h, nibble e / 2 + 4 (e % 2)
 *   scale  fp32 at byte 2048 + 16 c + 4 j
 *   zero   u8 at byte 2304 + 4 c + j
 * Columns past N and groups past K/64 hold zero codes, scales and zeros.
 * This is the order in which one 64-lane matrix-core pass consumes them, so
 * every load of the linear is a contiguous run.
 * Size in bytes of the records for an N x K weight (0 for bad shapes).
 */
int64_t svdq_awq_packed_bytes(int64_t N, int64_t K);

/*
 * Offline quantization of the fp32 weight W [N, K] (row n = output n) into
 * records (device, svdq_awq_packed_bytes(N, K) bytes, out), per group:
 *   s = fl32(fl32(hi - lo) / 15) with lo = min(0, min w), hi = max(0, max w),
 *   z = clamp(rint(fl32(-lo fl32(1/s))), 0, 15),
 *   q = clamp(rint(fl32(w fl32(1/s))) + z, 0, 15), ties to even;
 * a zero scale or a non-finite 1/s gives q = z = 0.  N >= 0 (0: no-op),
 * N % 8 == 0, K % 64 == 0.  Bit-exact with that definition.
 */
int32_t svdq_awq_pack_weights(const float *W, int64_t N, int64_t K, uint8_t *packed,
                              void *stream);

/*
 * Records from an already quantized weight in the common row-major form:
 *   codes   device u8   [N, K/2]  element 2j in the low nibble of byte j
 *   scales  device fp32 [N, K/64]
 *   zeros   device u8   [N, K/64] in [0, 15] (not checked)
 *   packed  device, svdq_awq_packed_bytes(N, K) bytes (out)
 * Same shape rules as svdq_awq_pack_weights; a pure re-arrangement.
 */
int32_t svdq_awq_repack(const uint8_t *codes, const float *scales, const uint8_t *zeros,
                        int64_t N, int64_t K, uint8_t *packed, void *stream);

/*
 * Y = X Wq^T + bias with Wq = (q - z) s from the records.
 *   X       device bf16 [M, K]
 *   packed  device records of svdq_awq_pack_weights / svdq_awq_repack
 *   bias    device bf16 [N] or NULL
 *   Y       device bf16 [M, N] (out)
 * M >= 0 (0: no-op; made for small M, where the weight stream dominates;
 * rows are taken 16 at a time, each 16 re-reading the weight), N % 8 == 0,
 * K % 64 == 0 with 16 activation rows of K fitting the device's
 * per-workgroup LDS (fewer rows per pass otherwise; SVDQ_ERR_UNSUPPORTED_SHAPE
 * when not even one fits).  Products exact, fp32 sums; accurate to 1 bf16
 * ulp + 1e-3 rms of the fp64 result.  Deterministic.
 */
int32_t svdq_awq_w4a16_linear(const uint16_t *X, const uint8_t *packed, const uint16_t *bias,
                              int64_t M, int64_t N, int64_t K, uint16_t *Y, void *stream);

/*
 * Test hook: how svdq_w4a4_lr_gemm (and svdq_linear, svdq_linear_noalloc)
 * tile the output.
 *   SVDQ_TILES_AUTO    the default, with S workgroup slots for 128 x 128
 *                      tiles (two per compute unit): when the output has at
 *                      most one 64 x 64 tile per compute unit (and
 *                      K / 64 >= 3), k-split 64 x 64 tiles (each workgroup's
 *                      two halves run half of the K loop each and add their
 *                      partial sums in LDS); else, when its 128 x 128 tiles
 *                      fill at most 3/4 of S, all 64 x 64 tiles; else
 *                      128 x 128 tiles for whole rounds of S and 64 x 64
 *                      tiles for a partial last round of at most S / 4 tiles
 *                      (a larger one runs as 128 x 128)
 *   SVDQ_TILES_FULL    128 x 128 tiles only
 *   SVDQ_TILES_QUARTER 64 x 64 tiles only
 *   SVDQ_TILES_KSPLIT, SVDQ_TILES_KSPLIT_QUARTER  k-split 128 x 128 / 64 x 64
 *                      tiles only (K / 64 >= 3; otherwise as SVDQ_TILES_AUTO)
 * Process-wide.  FULL and QUARTER (and AUTO where it picks them) give
 * identical results (both tile shapes run the same per-output arithmetic in
 * the same order); the k-split tiles add the two halves' partial sums, a
 * different fp32 order, within the same tolerance.  Returns
 * SVDQ_ERR_INVALID_ARG for any other value.
 */
#define SVDQ_TILES_AUTO 0
#define SVDQ_TILES_FULL 1
#define SVDQ_TILES_QUARTER 2
#define SVDQ_TILES_KSPLIT 3
#define SVDQ_TILES_KSPLIT_QUARTER 4
int32_t svdq_debug_set_tile_policy(int32_t policy);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */
