// awq_w4a16.hip -- the second layer kind of the pages: 4-bit weights with
// 16-bit activations (the "Bringing Nunchaku 4-bit inference to Diffusers"
// blog, section "Introducing Nunchaku Lite": awq_w4a16, used for the
// adaptive-normalization and modulation projections; quantization_config:
// int4, group size 64), on gfx950.
//
// Weights: asymmetric group-64 codes q in [0, 15] with an fp32 scale s and a
// zero point z per (row, group); the weight stands for (q - z) s.  These
// projections see a handful of conditioning vectors (small M) against a wide
// weight (e.g. 3072 -> 6 x 3072), so the layer streams the packed weight
// from HBM once; the arithmetic rides on the matrix unit:
//   - B operand = codes as bf16 (128 + q is exactly 0x4300 | q), A operand =
//     the bf16 activations (rows past M are zero);
//   - per group, v_mfma_f32_16x16x32_bf16 accumulates sum x (128 + q) and
//     then sum x (-(128 + z)) into the same tile, which leaves
//     sum x (q - z) (exact products, fp32 sums);
//   - the VALU adds s times that to the output, four values per lane.
#include "svdq_device.h"
#include "svdq_internal.h"

namespace svdq {

// ------------------------------------------------------------------ pack
// One thread per (row, group): lo = min(0, min w), hi = max(0, max w),
// s = fl32(fl32(hi - lo) / 15), inv = fl32(1 / s),
// z = clamp(rint(fl32(-lo inv)), 0, 15), q = clamp(rint(fl32(w inv)) + z, 0, 15)
// (IEEE division, ties to even, no contraction); a zero scale or a
// non-finite 1/s gives q = z = 0.
__global__ void __launch_bounds__(256)
awq_pack_kernel(const float *__restrict__ W, int64_t N, int64_t K, uint8_t *__restrict__ qw,
                float *__restrict__ scales, uint8_t *__restrict__ zeros) {
    const int64_t G = K / kGroup;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= N * G) return;
    const int64_t n = t / G;
    const int64_t g = t - n * G;
    const f32x4 *w4 = reinterpret_cast<const f32x4 *>(W + n * K + g * kGroup);
    float v[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup / 4; ++i) {
        const f32x4 x = w4[i];
        v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
    }
    float lo = 0.0f, hi = 0.0f;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
        lo = v[j] < lo ? v[j] : lo;
        hi = v[j] > hi ? v[j] : hi;
    }
    const float s = (hi - lo) / 15.0f;
    float inv = 0.0f;
    bool degenerate = true;
    if (s != 0.0f) {
        inv = 1.0f / s;
        degenerate = !__builtin_isfinite(inv);
    }
    float z = 0.0f;
    if (!degenerate) z = fminf(fmaxf(__builtin_rintf(-lo * inv), 0.0f), 15.0f);
    uint32_t words[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float q = 0.0f;
            if (!degenerate) q = fminf(fmaxf(__builtin_rintf(v[8 * b + e] * inv) + z, 0.0f), 15.0f);
            word |= (uint32_t)q << (4 * e);
        }
        words[b] = word;
    }
    u32x4 *dst = reinterpret_cast<u32x4 *>(qw + n * (K / 2) + g * (kGroup / 2));
    dst[0] = u32x4{words[0], words[1], words[2], words[3]};
    dst[1] = u32x4{words[4], words[5], words[6], words[7]};
    scales[t] = s;
    zeros[t] = (uint8_t)z;
}

// ------------------------------------------------------------------ linear
// One workgroup = 16 output columns x 16 rows of X (rows past M are zero);
// its four waves take a quarter of the groups each and their partial tiles
// are added in wave order in LDS, so the result does not depend on
// scheduling.  Per group, lane l supplies column / row l % 16 and the 16
// consecutive k at 16 (l / 16) of the group: k-slot l / 16 of MFMA call c
// holds k = 64 g + 16 (l / 16) + 8 c .. + 7 on both operands.  The loads of
// up to AWQ_DEPTH groups are in flight ahead of their use.
constexpr int AWQ_DEPTH = 8;

namespace {

// 8 codes (one dword, element 2i in the low nibble of byte i) -> 8 bf16 of
// 128 + q, pairs in dwords.
__device__ __forceinline__ u32x4 codes_to_bf16(uint32_t p) {
    const uint32_t lo = p & 0x0F0F0F0Fu;          // byte i = element 2i
    const uint32_t hi = (p >> 4) & 0x0F0F0F0Fu;   // byte i = element 2i + 1
    u32x4 r;
    // bytes: lo.b_i, 0, hi.b_i, 0 (v_perm selector 0x0C gives 0x00), then
    // the bf16 exponent bits of 128 in both halves
    r.x = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x43004300u;
    r.y = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x43004300u;
    r.z = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x43004300u;
    r.w = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x43004300u;
    return r;
}

struct AwqGroup {
    u32x2 q;          // 16 codes of the lane's column
    u32x4 x0, x1;     // 16 activations of the lane's row (zero past M)
    float s;
    uint32_t z;
};

__device__ __forceinline__ void awq_load(AwqGroup &d, const uint8_t *qrow, const float *srow,
                                         const uint8_t *zrow, const uint16_t *xrow, bool x_ok,
                                         int64_t g, int ks) {
    d.q = *reinterpret_cast<const u32x2 *>(qrow + g * 32 + 8 * ks);
    d.s = srow[g];
    d.z = zrow[g];
    if (x_ok) {
        const uint16_t *xp = xrow + g * kGroup + 16 * ks;
        d.x0 = *reinterpret_cast<const u32x4 *>(xp);
        d.x1 = *reinterpret_cast<const u32x4 *>(xp + 8);
    } else {
        d.x0 = u32x4{0u, 0u, 0u, 0u};
        d.x1 = d.x0;
    }
}

__device__ __forceinline__ void awq_group(f32x4 &acc, const AwqGroup &d) {
    const u32x4 b0 = codes_to_bf16(d.q.x);
    const u32x4 b1 = codes_to_bf16(d.q.y);
    // -(128 + z) in bf16 (an integer below 256: exact), in every element
    const uint32_t zb = __float_as_uint(-(128.0f + (float)d.z)) >> 16;
    const uint32_t zz = zb | (zb << 16);
    const u32x4 bz = u32x4{zz, zz, zz, zz};
    f32x4 t = mfma_bf16_16x16x32(d.x0, b0, f32x4{0.f, 0.f, 0.f, 0.f});
    t = mfma_bf16_16x16x32(d.x1, b1, t);
    t = mfma_bf16_16x16x32(d.x0, bz, t);
    t = mfma_bf16_16x16x32(d.x1, bz, t);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(d.s, t[j], acc[j]);
}

}  // namespace

__global__ void __launch_bounds__(256)
awq_linear_kernel(const uint16_t *__restrict__ X, const uint8_t *__restrict__ qw,
                  const float *__restrict__ scales, const uint8_t *__restrict__ zeros,
                  const uint16_t *__restrict__ bias, int64_t M, int64_t N, int64_t K,
                  uint16_t *__restrict__ Y) {
    __shared__ float red[4][16][17];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rl = lane & 15;
    const int ks = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t m0 = (int64_t)blockIdx.y * 16;
    const int64_t G = K / kGroup;
    const int64_t g_begin = G * wave / 4;
    const int64_t g_end = G * (wave + 1) / 4;
    const int64_t n = n0 + rl < N ? n0 + rl : N - 1;     // column of the B operand
    const int64_t m = m0 + rl;                           // row of the A operand
    const bool x_ok = m < M;
    const uint8_t *qrow = qw + n * (K / 2);
    const float *srow = scales + n * G;
    const uint8_t *zrow = zeros + n * G;
    const uint16_t *xrow = X + (x_ok ? m : 0) * K;

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int64_t gb = g_begin; gb < g_end; gb += AWQ_DEPTH) {
        AwqGroup d[AWQ_DEPTH];
#pragma unroll
        for (int i = 0; i < AWQ_DEPTH; ++i) {
            const int64_t g = gb + i < g_end ? gb + i : g_end - 1;
            awq_load(d[i], qrow, srow, zrow, xrow, x_ok, g, ks);
        }
#pragma unroll
        for (int i = 0; i < AWQ_DEPTH; ++i)
            if (gb + i < g_end) awq_group(acc, d[i]);
    }

    // lane holds rows 4 ks + j, column rl of this wave's partial tile
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wave][4 * ks + j][rl] = acc[j];
    __syncthreads();
    const int tr = threadIdx.x >> 4, tc = threadIdx.x & 15;
    const int64_t om = m0 + tr, on = n0 + tc;
    if (om < M && on < N) {
        float v = red[0][tr][tc];
        v += red[1][tr][tc];
        v += red[2][tr][tc];
        v += red[3][tr][tc];
        if (bias) v += bf16_to_f32(bias[on]);
        Y[om * N + on] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_awq_pack(const float *W, int64_t N, int64_t K, uint8_t *qw, float *scales,
                           uint8_t *zeros, hipStream_t stream) {
    const int64_t threads = N * (K / kGroup);
    awq_pack_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(W, N, K, qw, scales,
                                                                         zeros);
    return hipGetLastError();
}

hipError_t launch_awq_linear(const uint16_t *X, const uint8_t *qw, const float *scales,
                             const uint8_t *zeros, const uint16_t *bias, int64_t M, int64_t N,
                             int64_t K, uint16_t *Y, hipStream_t stream) {
    dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + 15) / 16));
    awq_linear_kernel<<<grid, 256, 0, stream>>>(X, qw, scales, zeros, bias, M, N, K, Y);
    return hipGetLastError();
}

}  // namespace svdq
