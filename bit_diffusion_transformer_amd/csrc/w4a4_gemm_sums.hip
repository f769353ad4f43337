// w4a4_gemm_sums.hip -- test hook: the exact per-group integer sums of the
// W4A4 GEMM, taken from the production tile code (w4a4_tile.h: the same
// global -> LDS ring, swizzle, row-pair copies, odd-group tail stage, FP6
// operand form and matrix instruction as the GEMM), one group per launch.
// A translation unit of its own, so that the GEMM's schedule does not depend
// on it.
#include "w4a4_tile.h"

namespace svdq {

// One workgroup per BT x BT tile (BT = 64 WB) of the tile grid that meets the
// requested block [m0, m0 + tm) x [n0, n0 + tn): tiles tmf + b % ntm along m
// and tnf + b / ntm along n.
template <int WB>
__global__ void __launch_bounds__(NTHR)
w4a4_group_sums_kernel(const uint8_t *__restrict__ qa, const float *__restrict__ sa,
                       const uint8_t *__restrict__ qw, const float *__restrict__ sw, int64_t M,
                       int64_t N, int64_t K, int64_t tmf, int64_t tnf, int64_t ntm,
                       SumsArgs sg) {
    __shared__ Smem<WB> sm;
    constexpr int BT = 64 * WB;
    const int64_t b = blockIdx.x;
    const int64_t m0 = (tmf + b % ntm) * BT, n0 = (tnf + b / ntm) * BT;
    tile_body<WB, EPI_SUMS>(qa, sa, qw, sw, nullptr, nullptr, nullptr, 0, M, N, K, 0, nullptr,
                            sm, m0, n0, &sg);
}

hipError_t launch_group_sums(const uint8_t *qa, const float *sa, const uint8_t *qw,
                             const float *sw, int64_t M, int64_t N, int64_t K, int64_t m0,
                             int64_t n0, int64_t tm, int64_t tn, int32_t *S, bool quarter,
                             hipStream_t stream) {
    const int64_t BT = quarter ? 64 : 128;
    const int64_t tmf = m0 / BT, tml = (m0 + tm - 1) / BT;
    const int64_t tnf = n0 / BT, tnl = (n0 + tn - 1) / BT;
    const int64_t ntm = tml - tmf + 1, ntn = tnl - tnf + 1;
    const unsigned blocks = (unsigned)(ntm * ntn);
    const int G = (int)(K / kGroup);
    for (int g = 0; g < G; ++g) {
        const SumsArgs sg{S, m0, n0, tm, tn, G, g};
        if (quarter)
            w4a4_group_sums_kernel<1><<<blocks, NTHR, 0, stream>>>(qa, sa, qw, sw, M, N, K, tmf,
                                                                   tnf, ntm, sg);
        else
            w4a4_group_sums_kernel<2><<<blocks, NTHR, 0, stream>>>(qa, sa, qw, sw, M, N, K, tmf,
                                                                   tnf, ntm, sg);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace svdq
