// w4a4_gemm_qkv.hip -- the W4A4 GEMM with the fused QKV epilogue (per-head
// RMS norm and rotary turn of Q and K, [B, H, S, D] outputs; see
// qkv_epilogue in w4a4_tile.h), in a translation unit of its own so that the
// plain kernel's schedule does not depend on it.
#include "w4a4_tile.h"

namespace svdq {

// The GEMM with the fused QKV epilogue: full 128 x 128 tiles only (a head
// of 128 columns is one tile), each XCD taking a contiguous range.
__global__ void __launch_bounds__(NTHR)
w4a4_lr_gemm_qkv_kernel(const uint8_t *__restrict__ qa, const float *__restrict__ sa,
                        const uint8_t *__restrict__ qw, const float *__restrict__ sw,
                        const float *__restrict__ xl1, const uint16_t *__restrict__ L2,
                        const uint16_t *__restrict__ bias, int64_t M, int64_t N, int64_t K,
                        int r, QkvArgs qk, int64_t nfull) {
    __shared__ Smem<2> sm;
    const int64_t nbm = (M + TILE - 1) / TILE, nbn = (N + TILE - 1) / TILE;
    int64_t b = blockIdx.x, tm, tn;
    if ((nfull & 7) == 0) b = (b & 7) * (nfull >> 3) + (b >> 3);
    raster(b, nbm, nbn, tm, tn);
    tile_body<2, EPI_QKV>(qa, sa, qw, sw, xl1, L2, bias, 0, M, N, K, r, nullptr, sm, tm * TILE,
                       tn * TILE, &qk);
}

hipError_t launch_w4a4_gemm_qkv(const uint8_t *qa, const float *sa, const uint8_t *qw,
                                const float *sw, const float *xl1, const uint16_t *L2,
                                const uint16_t *bias, int64_t M, int64_t K, int r,
                                const QkvArgs &qk, hipStream_t stream) {
    const int64_t N = 3 * (int64_t)qk.H * qk.D;
    const int64_t tiles = ((M + TILE - 1) / TILE) * (N / TILE);
    w4a4_lr_gemm_qkv_kernel<<<(unsigned)tiles, NTHR, 0, stream>>>(qa, sa, qw, sw, xl1, L2, bias,
                                                                  M, N, K, r, qk, tiles);
    return hipGetLastError();
}

}  // namespace svdq
