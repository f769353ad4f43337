// w4a4_gemm.hip -- the W4A4 GEMM of the SVDQuant layer on gfx950 with the
// rank-r up-projection, bias and GELU applied to the same output tile before
// its single bf16 store (the "Nunchaku engine design" section of the
// svdq-int4-flux.1-canny-dev model card fuses the up-projection with the
// 4-bit compute because both produce the same output).  The tile code is in
// w4a4_tile.h; this file holds the plain kernel and its launcher.
#include "w4a4_tile.h"

#include <atomic>

namespace svdq {

// One launch covers the whole output.  Workgroups [0, nq) are quarter tiles
// (64 x 64): quadrant b % 4 of tile tq0 + b / 4 of the 128 x 128 tile grid,
// used for the tiles of a partial last round.  They come first so that they
// run alongside the first round of full tiles instead of alone after the
// last one.  Workgroups [nq, nq + nfull) are full tiles 0 .. nfull - 1, each
// XCD taking a contiguous range of them (consecutive workgroups go to
// different XCDs, round robin over 8) so that tiles sharing operands share
// that XCD's L2.
__global__ void __launch_bounds__(NTHR)
w4a4_lr_gemm_kernel(const uint8_t *__restrict__ qa, const float *__restrict__ sa,
                    const uint8_t *__restrict__ qw, const float *__restrict__ sw,
                    const float *__restrict__ xl1, const uint16_t *__restrict__ L2,
                    const uint16_t *__restrict__ bias, int act, int64_t M, int64_t N,
                    int64_t K, int r, uint16_t *__restrict__ Y, int64_t nq, int64_t tq0,
                    int64_t nfull) {
    __shared__ union {
        Smem<2> full;
        Smem<1> quarter;
    } sm;
    const int64_t nbm = (M + TILE - 1) / TILE, nbn = (N + TILE - 1) / TILE;
    int64_t b = blockIdx.x, tm, tn;
    if (b < nq) {
        raster(tq0 + b / 4, nbm, nbn, tm, tn);
        const int64_t m0 = tm * TILE + 64 * (b & 1);
        const int64_t n0 = tn * TILE + 64 * ((b >> 1) & 1);
        if (m0 >= M || n0 >= N) return;   // quadrant outside a ragged edge
        tile_body<1>(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, sm.quarter, m0, n0);
    } else {
        b -= nq;
        if ((nfull & 7) == 0) b = (b & 7) * (nfull >> 3) + (b >> 3);
        raster(b, nbm, nbn, tm, tn);
        tile_body<2>(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, sm.full, tm * TILE,
                     tn * TILE);
    }
}

// The whole output as 64 x 64 tiles, one workgroup each, rastered on their
// own grid with each XCD taking a contiguous range (as the full tiles
// above).  A kernel of its own so that its register budget allows three or
// four workgroups per compute unit (the shared kernel is sized for 128 x 128
// tiles: two).
__global__ void __launch_bounds__(NTHR, 3)
w4a4_lr_gemm_quarter_kernel(const uint8_t *__restrict__ qa, const float *__restrict__ sa,
                            const uint8_t *__restrict__ qw, const float *__restrict__ sw,
                            const float *__restrict__ xl1, const uint16_t *__restrict__ L2,
                            const uint16_t *__restrict__ bias, int act, int64_t M, int64_t N,
                            int64_t K, int r, uint16_t *__restrict__ Y) {
    __shared__ Smem<1> sm;
    const int64_t nqm = (M + 63) / 64, nqn = (N + 63) / 64, nq = nqm * nqn;
    int64_t b = blockIdx.x, tm, tn;
    if ((nq & 7) == 0) b = (b & 7) * (nq >> 3) + (b >> 3);
    raster(b, nqm, nqn, tm, tn);
    tile_body<1>(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, sm, 64 * tm, 64 * tn);
}

static std::atomic<int> g_tile_policy{0};

void set_tile_policy(int policy) { g_tile_policy.store(policy, std::memory_order_relaxed); }
int tile_policy() { return g_tile_policy.load(std::memory_order_relaxed); }

// Workgroup slots of the device (two 128 x 128 workgroups per compute
// unit), cached per device.
int64_t wg_slots() {
    static int64_t slots[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
    if (slots[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = 256;
        slots[dev] = 2 * (int64_t)cus;
    }
    return slots[dev];
}

// Full 128 x 128 tiles for whole rounds of the device's workgroup slots; if
// a partial last round is left of at most three quarters of the slots, its
// tiles run as 64 x 64 quarter tiles (four times the workgroups, a quarter
// of the work each) in the same launch.
hipError_t launch_w4a4_gemm(const uint8_t *qa, const float *sa, const uint8_t *qw,
                            const float *sw, const float *xl1, const uint16_t *L2,
                            const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                            int r, uint16_t *Y, hipStream_t stream) {
    const int64_t tiles = ((M + TILE - 1) / TILE) * ((N + TILE - 1) / TILE);
    const int policy = tile_policy();
    // The automatic choice (measured on the layer shapes at 64 .. 4096 tokens):
    //   - at most one 64 x 64 tile per compute unit: k-split 64 x 64 tiles
    //     (two waves per SIMD on half the K loop each), given three groups or
    //     more (each half gets one);
    //   - 128 x 128 tiles for at most 3/4 of the workgroup slots: all 64 x 64
    //     tiles (four times the workgroups, up to four per compute unit);
    //   - otherwise 128 x 128 tiles, with a partial last round of at most a
    //     quarter of the slots run as 64 x 64 tiles alongside the first round.
    const int64_t slots = wg_slots();
    const int64_t cus = slots / 2;
    const int64_t qtiles = ((M + 63) / 64) * ((N + 63) / 64);
    const bool ks_ok = K / kGroup >= 3;
    const int pol = (policy == 3 || policy == 4) && !ks_ok ? 0 : policy;
    if (pol == 3 || pol == 4 || (pol == 0 && ks_ok && qtiles <= cus))
        return launch_w4a4_gemm_ks(qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, pol != 3,
                                   stream);
    int64_t rest = 0;
    if (pol == 2) {
        rest = tiles;
    } else if (pol == 0) {
        if (4 * tiles <= 3 * slots) {
            rest = tiles;
        } else {
            rest = tiles % slots;
            if (rest * 4 > slots) rest = 0;
        }
    }
    if (rest == tiles) {
        w4a4_lr_gemm_quarter_kernel<<<(unsigned)qtiles, NTHR, 0, stream>>>(
            qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y);
        return hipGetLastError();
    }
    const int64_t full = tiles - rest;
    const int64_t nq = 4 * rest;
    w4a4_lr_gemm_kernel<<<(unsigned)(nq + full), NTHR, 0, stream>>>(
        qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, nq, full, full);
    return hipGetLastError();
}

}  // namespace svdq
