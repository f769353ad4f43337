// svdq_internal.h -- kernel launchers shared between the HIP translation
// units of libsvdq (internal; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace svdq {

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// MXFP4 scale bytes are block-major, [K/32][P]: P = rows rounded up to a
// multiple of 16 (the bytes past `rows` are padding, never read into a result).
__host__ __device__ inline int64_t mx_scale_rows(int64_t rows) { return (rows + 15) & ~(int64_t)15; }

// Packed 4-bit codes (INT4 and MXFP4 alike) are stored in row pairs: for
// rows 2p and 2p + 1, each 64-byte chunk of a row's kb = K/2 bytes (128
// codes, one GEMM stage) is followed by the same chunk of the other row, so
// one 128-byte line holds a stage of both rows.  When kb is not a multiple
// of 64 (INT4 with an odd group count) the last chunk is 32 bytes wide and
// the pair interleaves in 32-byte halves there.  [ceil(rows/2)][2 kb] bytes;
// an odd count's last pair has an unwritten half.  Byte b of row `row`:
__host__ __device__ inline int64_t code_offset(int64_t row, int64_t kb, int64_t b) {
    const int64_t c = b >> 6;
    const int64_t w = kb - (c << 6) < 64 ? kb - (c << 6) : 64;
    return (row >> 1) * 2 * kb + (c << 7) + (row & 1) * w + (b & 63);
}

// INT4 group scales (sa, sw) are stored stage-major: for R rows and G groups,
// fp32 [ceil(G/2)][R][2], the scale of (row, group g) at
// ((g / 2) R + row) 2 + g % 2, so that one GEMM stage (two groups) of a tile's
// rows is one contiguous run of 8 bytes per row.  With an odd G the slots
// (row, G) of the last stage are padding, written as zero.
__host__ __device__ inline int64_t scale_index(int64_t row, int64_t g, int64_t R) {
    return ((g >> 1) * R + row) * 2 + (g & 1);
}
inline size_t scale_floats(int64_t R, int64_t G) { return (size_t)((G + 1) / 2) * (size_t)R * 2; }

// svdq_quantize_act_down splits K into chunks of kc groups (one workgroup per
// 64 rows and chunk); with more than one chunk and r > 0 the chunks' partial
// x^ L1 sums go to the workspace and a second kernel adds them up.  kc keeps
// the chunk of L1 staged in LDS (kc x 64 x r bf16, r rounded up to 32, 64 or
// 128) at 32 KB or less; below that, shorter chunks give more and shorter
// waves (each wave runs its chunk's groups one after another): 4 groups
// unless K is long (more than 64 groups, where the partial sums would grow),
// 2 for a few hundred tokens.  The last chunk may hold fewer groups.
inline int k1_chunk_groups(int64_t M, int64_t K, int r) {
    if (r > 64) return 2;
    if (r > 32) return 4;
    if (M <= 512) return 2;
    return K / 64 > 64 ? 8 : 4;
}
inline int k1_chunks(int64_t M, int64_t K, int r) {
    const int64_t G = K / 64;
    const int kc = k1_chunk_groups(M, K, r);
    return (int)((G + kc - 1) / kc);
}

// Scratch of svdq_quantize_act_down, carved from the caller's workspace.
struct DownWorkspace {
    float *part;        // [chunks][M][r] partial sums (null when not needed)
};

inline size_t down_workspace_bytes(int64_t M, int64_t K, int r) {
    if (r <= 0 || M <= 0 || K < 64) return 0;
    const int nc = k1_chunks(M, K, r);
    return nc > 1 ? align256((size_t)nc * (size_t)M * (size_t)r * 4) : 0;
}

inline DownWorkspace carve_down_workspace(void *base, int64_t M, int64_t K, int r) {
    DownWorkspace w{nullptr};
    if (down_workspace_bytes(M, K, r) > 0) w.part = static_cast<float *>(base);
    return w;
}

// mx: the MXFP4 variant (block-major E8M0 scale bytes [K/32][mx_scale_rows(rows)] in
// sa / sw)
hipError_t launch_quant_down(const uint16_t *X, const float *lambda, const uint16_t *L1,
                             int64_t M, int64_t K, int r, const DownWorkspace &ws, uint8_t *qa,
                             void *sa, float *xl1, hipStream_t stream, bool mx = false);
hipError_t launch_pack_weights(const float *R, int64_t N, int64_t K, uint8_t *qw, void *sw,
                               hipStream_t stream, bool mx = false);
// row-major two's-complement INT4 codes [N, K/2] and fp32 scales [N, K/64] ->
// the stored row-pair codes and stage-major scales
hipError_t launch_repack_codes(const uint8_t *codes, const float *scales, int64_t N, int64_t K,
                               uint8_t *qw, float *sw, hipStream_t stream);
// W4A16 records (16 columns x 4 groups each)
int64_t awq_packed_bytes(int64_t N, int64_t K);
int awq_rows_per_pass(int64_t K, size_t lds_limit);   // activation rows staged per workgroup
hipError_t launch_awq_pack(const float *W, int64_t N, int64_t K, uint8_t *rec, hipStream_t stream);
hipError_t launch_awq_repack(const uint8_t *codes, const float *scales, const uint8_t *zeros,
                             int64_t N, int64_t K, uint8_t *rec, hipStream_t stream);
hipError_t launch_awq_linear(const uint16_t *X, const uint8_t *rec, const uint16_t *bias,
                             int64_t M, int64_t N, int64_t K, int MT, uint16_t *Y,
                             hipStream_t stream);

// Fused QKV epilogue: the GEMM's columns are [Q | K | V], each H heads of D.
struct QkvArgs {
    int H, D;                      // heads, head_dim (64 or 128; H D % 128 == 0)
    int64_t S;                     // tokens per sequence; M = B S
    const uint16_t *gq, *gk;       // bf16 [D] RMS-norm weights
    float eps;
    const float *cos_t, *sin_t;    // fp32 [S, D/2]
    uint16_t *Q, *K, *V;           // bf16 [B, H, S, D]
};
hipError_t launch_w4a4_gemm_qkv(const uint8_t *qa, const float *sa, const uint8_t *qw,
                                const float *sw, const float *xl1, const uint16_t *L2,
                                const uint16_t *bias, int64_t M, int64_t K, int r,
                                const QkvArgs &qk, hipStream_t stream);

// MLP chain: the next SVDQuant layer's activation step (smoothing, INT4
// codes and scales, partial down-projections) from this GEMM's output tiles.
struct MlpArgs {
    const float *lam;       // fp32 [N]: the next layer's smoothing factors
    const uint16_t *L1;     // bf16 [N, rn]: its down-projection (NULL when rn == 0)
    int rn;                 // 0, 16 or 32
    uint8_t *qa;            // [M, N/2] codes (out)
    float *sa;              // [M, N/64] scales (out)
    float *part;            // [N/128, M, rn] partial down-projections (out, rn > 0)
};
hipError_t launch_w4a4_gemm_mlp(const uint8_t *qa, const float *sa, const uint8_t *qw,
                                const float *sw, const float *xl1, const uint16_t *L2,
                                const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                                int r, const MlpArgs &ma, hipStream_t stream);
hipError_t launch_xl1_reduce(const float *part, int nc, int64_t total, float *xl1,
                             hipStream_t stream);

// k-split tiles (two four-wave halves per workgroup, each on half of K):
// 128 x 128, or 64 x 64 with `quarter`; needs K / 64 >= 3
hipError_t launch_w4a4_gemm_ks(const uint8_t *qa, const float *sa, const uint8_t *qw,
                               const float *sw, const float *xl1, const uint16_t *L2,
                               const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                               int r, uint16_t *Y, bool quarter, hipStream_t stream);

// 0 auto, 1 full tiles only, 2 quarter tiles only, 3 k-split full tiles only,
// 4 k-split quarter tiles only (process-wide test hook)
void set_tile_policy(int policy);
int tile_policy();
int64_t wg_slots();   // 128 x 128 workgroup slots of the current device

hipError_t launch_w4a4_gemm(const uint8_t *qa, const float *sa, const uint8_t *qw,
                            const float *sw, const float *xl1, const uint16_t *L2,
                            const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                            int r, uint16_t *Y, hipStream_t stream);
// MXFP4 variant: block-major E8M0 scale bytes sa [K/32][mx_scale_rows(M)], sw
// [K/32][mx_scale_rows(N)]; K % 128 == 0.
hipError_t launch_w4a4_mx_gemm(const uint8_t *qa, const uint8_t *sa, const uint8_t *qw,
                               const uint8_t *sw, const float *xl1, const uint16_t *L2,
                               const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                               int r, uint16_t *Y, hipStream_t stream);
// Group-sum test hook: the production tile code (128 x 128 tiles, or 64 x 64
// with `quarter`) over the tiles that meet the block, one launch per group.
hipError_t launch_group_sums(const uint8_t *qa, const float *sa, const uint8_t *qw,
                             const float *sw, int64_t M, int64_t N, int64_t K, int64_t m0,
                             int64_t n0, int64_t tm, int64_t tn, int32_t *S, bool quarter,
                             hipStream_t stream);

}  // namespace svdq
