// w4a4_gemm.hip -- the W4A4 GEMM of the SVDQuant layer on gfx950 with the
// rank-r up-projection, bias and GELU applied to the same output tile before
// its single bf16 store (the "Nunchaku engine design" section of the
// svdq-int4-flux.1-canny-dev model card fuses the up-projection with the
// 4-bit compute because both produce the same output).  The tile code is in
// w4a4_tile.h; this file holds the plain kernel, its launcher and the
// group-sum test hook.
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

// Test hook: per-group integer sums with the GEMM's k split, FP8 operand
// form and matrix instruction; one wave per 32 x 32 block of (n, m),
// operands read from memory.  The sums are exact integers in fp32.
__global__ void __launch_bounds__(64)
group_sums_kernel(const uint8_t *__restrict__ qa, const uint8_t *__restrict__ qw, int64_t M,
                  int64_t N, int64_t K, int64_t m0, int64_t n0, int64_t tm, int64_t tn,
                  int32_t *__restrict__ S) {
    const int lane = threadIdx.x;
    const int r32 = lane & 31, ks2 = lane >> 5;
    const int64_t nb = blockIdx.x, mb = blockIdx.y;
    const int64_t G = K / kGroup;
    int64_t n = n0 + nb * 32 + r32, m = m0 + mb * 32 + r32;
    if (n >= N) n = N - 1;
    if (m >= M) m = M - 1;
    for (int64_t g = 0; g < G; ++g) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(qw + code_offset(n, K / 2, g * 32 + 16 * ks2));
        const u32x4 b = *reinterpret_cast<const u32x4 *>(qa + code_offset(m, K / 2, g * 32 + 16 * ks2));
        const f32x16 D = mfma_codes_32x32x64(codes_to_fp8(a), codes_to_fp8(b));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t nl = nb * 32 + 8 * (i / 4) + 4 * ks2 + (i % 4);
            const int64_t ml = mb * 32 + r32;
            if (nl < tn && ml < tm) S[(ml * tn + nl) * G + g] = (int32_t)D[i];
        }
    }
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
    int64_t rest = 0;
    if (policy == 2) {
        rest = tiles;
    } else if (policy == 0) {
        const int64_t slots = wg_slots();
        rest = tiles % slots;
        if (rest * 4 > slots * 3) rest = 0;
    }
    const int64_t full = tiles - rest;
    const int64_t nq = 4 * rest;
    w4a4_lr_gemm_kernel<<<(unsigned)(nq + full), NTHR, 0, stream>>>(
        qa, sa, qw, sw, xl1, L2, bias, act, M, N, K, r, Y, nq, full, full);
    return hipGetLastError();
}

hipError_t launch_group_sums(const uint8_t *qa, const uint8_t *qw, int64_t M, int64_t N,
                             int64_t K, int64_t m0, int64_t n0, int64_t tm, int64_t tn,
                             int32_t *S, hipStream_t stream) {
    dim3 grid((unsigned)((tn + 31) / 32), (unsigned)((tm + 31) / 32));
    group_sums_kernel<<<grid, 64, 0, stream>>>(qa, qw, M, N, K, m0, n0, tm, tn, S);
    return hipGetLastError();
}

}  // namespace svdq
