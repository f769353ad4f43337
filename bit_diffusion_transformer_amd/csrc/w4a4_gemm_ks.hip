// w4a4_gemm_ks.hip -- the W4A4 GEMM (plain [M, N] epilogue) with k-split
// tiles: 512-thread workgroups whose two halves run the K loop of one tile
// over the two halves of K and add their partial sums in LDS (tile_body<..,
// KS = 2> in w4a4_tile.h).  For grids of at most one tile per compute unit
// (a few hundred tokens), where one four-wave workgroup per compute unit
// leaves each SIMD a single wave: here each SIMD runs two, on half the K
// loop each, and nothing goes through memory but the operands and Y.  A
// translation unit of its own, so that the other kernels' schedules do not
// depend on it.
#include "w4a4_tile.h"

namespace svdq {

// One workgroup per BT x BT tile (BT = 64 WB) of the output, in the GROUP_M
// raster order of the BT grid; when the tile count is a multiple of 8 each
// XCD takes a contiguous range of tiles (workgroups go round robin over the
// eight XCDs).
template <int WB>
__global__ void __launch_bounds__(2 * NTHR)
w4a4_lr_gemm_ks_kernel(const uint8_t *__restrict__ qa, const float *__restrict__ sa,
                       const uint8_t *__restrict__ qw, const float *__restrict__ sw,
                       const float *__restrict__ xl1, const uint16_t *__restrict__ L2,
                       const uint16_t *__restrict__ bias, int act, int64_t M, int64_t N,
                       int64_t K, int r, uint16_t *__restrict__ Y, int64_t ntile) {
    __shared__ Smem<WB> sm[2];
    constexpr int BT = 64 * WB;
    const int64_t nbm = (M + BT - 1) / BT, nbn = (N + BT - 1) / BT;
    int64_t b = blockIdx.x, tm, tn;
    if ((ntile & 7) == 0) b = (b & 7) * (ntile >> 3) + (b >> 3);
    raster(b, nbm, nbn, tm, tn);
    tile_body<WB, EPI_STORE, false, 2>(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, sm[0],
                                       tm * BT, tn * BT);
}

hipError_t launch_w4a4_gemm_ks(const uint8_t *qa, const float *sa, const uint8_t *qw,
                               const float *sw, const float *xl1, const uint16_t *L2,
                               const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                               int r, uint16_t *Y, bool quarter, hipStream_t stream) {
    const int64_t BT = quarter ? 64 : 128;
    const int64_t ntile = ((M + BT - 1) / BT) * ((N + BT - 1) / BT);
    if (quarter)
        w4a4_lr_gemm_ks_kernel<1><<<(unsigned)ntile, 2 * NTHR, 0, stream>>>(
            qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, ntile);
    else
        w4a4_lr_gemm_ks_kernel<2><<<(unsigned)ntile, 2 * NTHR, 0, stream>>>(
            qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, ntile);
    return hipGetLastError();
}

}  // namespace svdq
