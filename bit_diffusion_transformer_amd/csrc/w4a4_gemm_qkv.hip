// w4a4_gemm_qkv.hip -- the W4A4 GEMM with the fused QKV epilogue (per-head
// RMS norm and rotary turn of Q and K, [B, H, S, D] outputs; see
// qkv_epilogue in w4a4_tile.h), in a translation unit of its own so that the
// plain kernel's schedule does not depend on it.
#include "w4a4_tile.h"

namespace svdq {

// Tiles are enumerated section by section: first the Q and K tiles, then the
// V tiles, each section in raster order.  Workgroups [0, nq) are quarter
// tiles (64 x 64) of the last tiles of that order -- V tiles, which need no
// norm -- for a partial last round of the device's workgroup slots; they come
// first so that they run alongside the first round.  Workgroups
// [nq, nq + nfull) are full tiles 0 .. nfull - 1, each XCD taking a
// contiguous range.
__device__ __forceinline__ void qkv_tile(int64_t id, int64_t nbm, int64_t nqk, int64_t nv,
                                         int64_t &tm, int64_t &tn) {
    const int64_t first = nbm * nqk;
    if (id < first) {
        raster(id, nbm, nqk, tm, tn);
    } else {
        raster(id - first, nbm, nv, tm, tn);
        tn += nqk;
    }
}

__global__ void __launch_bounds__(NTHR)
w4a4_lr_gemm_qkv_kernel(const uint8_t *__restrict__ qa, const float *__restrict__ sa,
                        const uint8_t *__restrict__ qw, const float *__restrict__ sw,
                        const float *__restrict__ xl1, const uint16_t *__restrict__ L2,
                        const uint16_t *__restrict__ bias, int64_t M, int64_t N, int64_t K,
                        int r, QkvArgs qk, int64_t nq, int64_t tq0, int64_t nfull) {
    __shared__ union {
        Smem<2> full;
        Smem<1> quarter;
    } sm;
    const int64_t nbm = (M + TILE - 1) / TILE;
    const int64_t nv = (int64_t)qk.H * qk.D / TILE, nqk = 2 * nv;
    int64_t b = blockIdx.x, tm, tn;
    if (b < nq) {
        qkv_tile(tq0 + b / 4, nbm, nqk, nv, tm, tn);
        const int64_t m0 = tm * TILE + 64 * (b & 1);
        const int64_t n0 = tn * TILE + 64 * ((b >> 1) & 1);
        if (m0 >= M) return;   // quadrant below a ragged edge
        tile_body<1, EPI_QKV>(qa, sa, qw, sw, xl1, L2, bias, 0, M, N, K, r, nullptr, sm.quarter,
                              m0, n0, &qk);
    } else {
        b -= nq;
        if ((nfull & 7) == 0) b = (b & 7) * (nfull >> 3) + (b >> 3);
        qkv_tile(b, nbm, nqk, nv, tm, tn);
        tile_body<2, EPI_QKV>(qa, sa, qw, sw, xl1, L2, bias, 0, M, N, K, r, nullptr, sm.full,
                              tm * TILE, tn * TILE, &qk);
    }
}

// Full tiles for whole rounds of the workgroup slots; a partial last round
// of at most three quarters of them, if it holds only V tiles, runs as
// quarter tiles.  The tile-policy test hook applies as for the plain GEMM
// (quarter: every V tile as quarter tiles).
hipError_t launch_w4a4_gemm_qkv(const uint8_t *qa, const float *sa, const uint8_t *qw,
                                const float *sw, const float *xl1, const uint16_t *L2,
                                const uint16_t *bias, int64_t M, int64_t K, int r,
                                const QkvArgs &qk, hipStream_t stream) {
    const int64_t N = 3 * (int64_t)qk.H * qk.D;
    const int64_t nbm = (M + TILE - 1) / TILE;
    const int64_t tiles = nbm * (N / TILE);
    const int64_t vtiles = nbm * ((int64_t)qk.H * qk.D / TILE);
    const int policy = tile_policy();
    int64_t rest = 0;
    if (policy == 2) {
        rest = vtiles;
    } else if (policy == 0) {
        const int64_t slots = wg_slots();
        rest = tiles % slots;
        if (rest * 4 > slots * 3 || rest > vtiles) rest = 0;
    }
    const int64_t full = tiles - rest;
    w4a4_lr_gemm_qkv_kernel<<<(unsigned)(4 * rest + full), NTHR, 0, stream>>>(
        qa, sa, qw, sw, xl1, L2, bias, M, N, K, r, qk, 4 * rest, full, full);
    return hipGetLastError();
}

}  // namespace svdq
