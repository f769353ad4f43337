// svdq_internal.h -- kernel launchers shared between the HIP translation
// units of libsvdq (internal; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace svdq {

// Scratch of svdq_quantize_act_down, carved from the caller's workspace.
struct DownWorkspace {
    float *inv_lam;     // [K]
    uint16_t *l1_hi;    // [r][K]  bf16 hi part of L1[k][i] / lambda[k], transposed
    uint16_t *l1_lo;    // [r][K]  bf16 lo part
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// inv_lam is always needed; the L1 parts only when r > 0.
inline size_t down_workspace_bytes(int64_t K, int r) {
    return align256((size_t)K * 4) + 2 * align256((size_t)K * (size_t)r * 2);
}

inline DownWorkspace carve_down_workspace(void *base, int64_t K, int r) {
    DownWorkspace w{nullptr, nullptr, nullptr};
    char *p = static_cast<char *>(base);
    w.inv_lam = reinterpret_cast<float *>(p);
    p += align256((size_t)K * 4);
    if (r == 0) return w;
    w.l1_hi = reinterpret_cast<uint16_t *>(p);
    p += align256((size_t)K * (size_t)r * 2);
    w.l1_lo = reinterpret_cast<uint16_t *>(p);
    return w;
}

hipError_t launch_prep_down(const float *lambda, const uint16_t *L1, int64_t K, int r,
                            const DownWorkspace &ws, hipStream_t stream);
hipError_t launch_quant_down(const uint16_t *X, int64_t M, int64_t K, int r,
                             const DownWorkspace &ws, uint8_t *qa, float *sa, float *xl1,
                             hipStream_t stream);
hipError_t launch_pack_weights(const float *R, int64_t N, int64_t K, uint8_t *qw, float *sw,
                               hipStream_t stream);
// 0 auto, 1 full tiles only, 2 quarter tiles only (process-wide test hook)
void set_tile_policy(int policy);

hipError_t launch_w4a4_gemm(const uint8_t *qa, const float *sa, const uint8_t *qw,
                            const float *sw, const float *xl1, const uint16_t *L2,
                            const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                            int r, uint16_t *Y, hipStream_t stream);
hipError_t launch_group_sums(const uint8_t *qa, const uint8_t *qw, int64_t M, int64_t N,
                             int64_t K, int64_t m0, int64_t n0, int64_t tm, int64_t tn,
                             int32_t *S, hipStream_t stream);

}  // namespace svdq
