// w4a4_gemm_mlp.hip -- the W4A4 GEMM whose output feeds the next SVDQuant
// layer (the MLP chain): the epilogue produces that layer's codes, scales and
// partial down-projections instead of the [M, N] bf16 output (mlp_epilogue in
// w4a4_tile.h).  A translation unit of its own, so that the plain kernel's
// schedule does not depend on it.
#include "w4a4_tile.h"

namespace svdq {

// Full 128 x 128 tiles only (a group of 64 columns is one wave's share),
// each XCD taking a contiguous range.
__global__ void __launch_bounds__(NTHR)
w4a4_lr_gemm_mlp_kernel(const uint8_t *__restrict__ qa, const float *__restrict__ sa,
                        const uint8_t *__restrict__ qw, const float *__restrict__ sw,
                        const float *__restrict__ xl1, const uint16_t *__restrict__ L2,
                        const uint16_t *__restrict__ bias, int act, int64_t M, int64_t N,
                        int64_t K, int r, MlpArgs ma, int64_t nfull) {
    __shared__ Smem<2> sm;
    const int64_t nbm = (M + TILE - 1) / TILE, nbn = (N + TILE - 1) / TILE;
    int64_t b = blockIdx.x, tm, tn;
    if ((nfull & 7) == 0) b = (b & 7) * (nfull >> 3) + (b >> 3);
    raster(b, nbm, nbn, tm, tn);
    tile_body<2, EPI_MLP>(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, nullptr, sm,
                          tm * TILE, tn * TILE, &ma);
}

hipError_t launch_w4a4_gemm_mlp(const uint8_t *qa, const float *sa, const uint8_t *qw,
                                const float *sw, const float *xl1, const uint16_t *L2,
                                const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                                int r, const MlpArgs &ma, hipStream_t stream) {
    const int64_t tiles = ((M + TILE - 1) / TILE) * (N / TILE);
    w4a4_lr_gemm_mlp_kernel<<<(unsigned)tiles, NTHR, 0, stream>>>(qa, sa, qw, sw, xl1, L2, bias,
                                                                  act, M, N, K, r, ma, tiles);
    return hipGetLastError();
}

}  // namespace svdq
