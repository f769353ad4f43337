// w4a4_mx_gemm.hip -- the 4-bit float (MXFP4) variant of the SVDQuant W4A4
// GEMM on gfx950.  The "Bringing Nunchaku 4-bit inference to Diffusers" blog
// (sections "Introducing Nunchaku Lite" and the quantization_config listing)
// gives the svdq_w4a4 family a 4-bit float variant beside INT4; the 4-bit
// float format with matrix-core support on this chip is MXFP4 of the OCP
// Microscaling (MX) specification v1.0: E2M1 codes, one E8M0 power-of-two
// scale per 32 values along K.  The low-rank branch, bias, activation and
// store are the INT4 kernel's.  The tile code is in w4a4_tile.h (its MXF
// path); this file holds the kernel and its launcher, in a translation unit
// of its own.
#include "w4a4_tile.h"

namespace svdq {

// Same tile order as the INT4 kernel: workgroups [0, nq) are quarter tiles of
// a partial last round, then full tiles with an XCD-contiguous mapping.
__global__ void __launch_bounds__(NTHR)
w4a4_mx_lr_gemm_kernel(const uint8_t *__restrict__ qa, const uint8_t *__restrict__ sa,
                       const uint8_t *__restrict__ qw, const uint8_t *__restrict__ sw,
                       const float *__restrict__ xl1, const uint16_t *__restrict__ L2,
                       const uint16_t *__restrict__ bias, int act, int64_t M, int64_t N,
                       int64_t K, int r, uint16_t *__restrict__ Y, int64_t nq, int64_t nfull) {
    __shared__ union {
        Smem<2> full;
        Smem<1> quarter;
    } sm;
    const int64_t nbm = (M + TILE - 1) / TILE, nbn = (N + TILE - 1) / TILE;
    int64_t b = blockIdx.x, tm, tn;
    if (b < nq) {
        raster(nfull + b / 4, nbm, nbn, tm, tn);
        const int64_t m0 = tm * TILE + 64 * (b & 1);
        const int64_t n0 = tn * TILE + 64 * ((b >> 1) & 1);
        if (m0 >= M || n0 >= N) return;   // quadrant outside a ragged edge
        tile_body<1, EPI_STORE, true>(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y,
                                      sm.quarter, m0, n0);
    } else {
        b -= nq;
        if ((nfull & 7) == 0) b = (b & 7) * (nfull >> 3) + (b >> 3);
        raster(b, nbm, nbn, tm, tn);
        tile_body<2, EPI_STORE, true>(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, sm.full,
                                      tm * TILE, tn * TILE);
    }
}

hipError_t launch_w4a4_mx_gemm(const uint8_t *qa, const uint8_t *sa, const uint8_t *qw,
                               const uint8_t *sw, const float *xl1, const uint16_t *L2,
                               const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                               int r, uint16_t *Y, hipStream_t stream) {
    const int64_t tiles = ((M + TILE - 1) / TILE) * ((N + TILE - 1) / TILE);
    const int policy = tile_policy();
    int64_t rest = 0;
    if (policy == 2) {
        rest = tiles;
    } else if (policy == 0) {
        const int64_t slots = wg_slots();
        rest = tiles % slots;
        if (rest * 4 > slots * 3) rest = 0;
    }
    const int64_t full = tiles - rest;
    w4a4_mx_lr_gemm_kernel<<<(unsigned)(4 * rest + full), NTHR, 0, stream>>>(
        qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, 4 * rest, full);
    return hipGetLastError();
}

}  // namespace svdq
