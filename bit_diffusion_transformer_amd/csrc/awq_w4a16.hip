// awq_w4a16.hip -- the second layer kind of the pages: 4-bit weights with
// 16-bit activations (the "Bringing Nunchaku 4-bit inference to Diffusers"
// blog, section "Introducing Nunchaku Lite": awq_w4a16, used for the
// adaptive-normalization and modulation projections; quantization_config:
// int4, group size 64), on gfx950.
//
// Weights: asymmetric group-64 codes q in [0, 15] with an fp32 scale s and a
// zero point z per (column, group); the weight stands for (q - z) s.  These
// projections see a handful of conditioning vectors (small M) against a wide
// weight (e.g. 3072 -> 6 x 3072), so the layer is one pass over the packed
// weight in HBM.  The weight is stored as records of 16 columns x 4 groups
// laid out in the order a 64-lane matrix-core pass consumes them (see the
// header), so each wave's loads are contiguous 1 KB / 256 B / 64 B runs.
//
// Per group the arithmetic rides on v_mfma_f32_16x16x32_bf16:
//   - B operand = codes as bf16: 128 + q is exactly 0x4300 | q, built with one
//     v_and_or_b32 per code pair;
//   - A operand = the bf16 activations of up to 16 rows, staged once per
//     workgroup in LDS (rows past M repeat the last row: their outputs are
//     dropped);
//   - two passes accumulate sum x (128 + q), two more add sum x (-(128 + z))
//     (bf16 bits 0xC300 | z, one v_perm), leaving sum x (q - z) exactly
//     (exact products, fp32 sums);
//   - the VALU adds s times that to the output, four values per lane.
#include "svdq_device.h"
#include "svdq_internal.h"

namespace svdq {

constexpr int kAwqRecord = 2368;   // 2048 codes + 256 scales + 64 zeros

// ------------------------------------------------------------------ records

// Store the 64 codes, scale and zero of (column n, group g) into its record.
__device__ __forceinline__ void awq_store_group(uint8_t *rec, int64_t GQ, int64_t n, int64_t g,
                                                const uint32_t (&q)[64], float s, uint32_t z) {
    const int64_t b = n >> 4, t = g >> 2;
    const int c = (int)(n & 15), j = (int)(g & 3);
    uint8_t *r = rec + (b * GQ + t) * kAwqRecord;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                word |= q[16 * sl + 8 * h + e] << (4 * (e / 2 + 4 * (e % 2)));
            *reinterpret_cast<uint32_t *>(r + 1024 * (j >> 1) + 16 * (c + 16 * sl) + 8 * (j & 1) +
                                          4 * h) = word;
        }
    }
    *reinterpret_cast<float *>(r + 2048 + 16 * c + 4 * j) = s;
    r[2304 + 4 * c + j] = (uint8_t)z;
}

// One thread per (column, group) of the padded grid NB*16 x GQ*4; columns
// past N and groups past K/64 store zeros.
//   s = fl32(fl32(hi - lo) / 15) with lo = min(0, min w), hi = max(0, max w),
//   inv = fl32(1 / s), z = clamp(rint(fl32(-lo inv)), 0, 15),
//   q = clamp(rint(fl32(w inv)) + z, 0, 15)
// (IEEE division, ties to even, no contraction); a zero scale or a
// non-finite 1/s gives q = z = 0.
__global__ void __launch_bounds__(256)
awq_pack_kernel(const float *__restrict__ W, int64_t N, int64_t K, uint8_t *__restrict__ rec) {
    const int64_t G = K / kGroup, GQ = (G + 3) / 4, G4 = 4 * GQ;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t NB = (N + 15) / 16;
    if (t >= NB * 16 * G4) return;
    const int64_t n = t / G4, g = t - n * G4;
    uint32_t q[64];
    float s = 0.0f;
    uint32_t z = 0;
    if (n < N && g < G) {
        const f32x4 *w4 = reinterpret_cast<const f32x4 *>(W + n * K + g * kGroup);
        float v[kGroup];
#pragma unroll
        for (int i = 0; i < kGroup / 4; ++i) {
            const f32x4 x = w4[i];
            v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
        }
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int e = 0; e < kGroup; ++e) {
            lo = v[e] < lo ? v[e] : lo;
            hi = v[e] > hi ? v[e] : hi;
        }
        s = (hi - lo) / 15.0f;
        float inv = 0.0f;
        bool degenerate = true;
        if (s != 0.0f) {
            inv = 1.0f / s;
            degenerate = !__builtin_isfinite(inv);
        }
        float zf = 0.0f;
        if (!degenerate) zf = fminf(fmaxf(__builtin_rintf(-lo * inv), 0.0f), 15.0f);
        z = (uint32_t)zf;
#pragma unroll
        for (int e = 0; e < kGroup; ++e)
            q[e] = degenerate ? 0u
                              : (uint32_t)fminf(fmaxf(__builtin_rintf(v[e] * inv) + zf, 0.0f), 15.0f);
    } else {
#pragma unroll
        for (int e = 0; e < kGroup; ++e) q[e] = 0u;
    }
    awq_store_group(rec, GQ, n, g, q, s, z);
}

// The same records from row-major codes (element 2j in the low nibble of
// byte j), scales and zeros.
__global__ void __launch_bounds__(256)
awq_repack_kernel(const uint8_t *__restrict__ codes, const float *__restrict__ scales,
                  const uint8_t *__restrict__ zeros, int64_t N, int64_t K,
                  uint8_t *__restrict__ rec) {
    const int64_t G = K / kGroup, GQ = (G + 3) / 4, G4 = 4 * GQ;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t NB = (N + 15) / 16;
    if (t >= NB * 16 * G4) return;
    const int64_t n = t / G4, g = t - n * G4;
    uint32_t q[64];
    float s = 0.0f;
    uint32_t z = 0;
    if (n < N && g < G) {
        const u32x4 *p4 = reinterpret_cast<const u32x4 *>(codes + n * (K / 2) + g * (kGroup / 2));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const u32x4 w = p4[i];
#pragma unroll
            for (int d = 0; d < 4; ++d)
#pragma unroll
                for (int b = 0; b < 8; ++b) q[32 * i + 8 * d + b] = (w[d] >> (4 * b)) & 15u;
        }
        s = scales[n * G + g];
        z = zeros[n * G + g];
    } else {
#pragma unroll
        for (int e = 0; e < kGroup; ++e) q[e] = 0u;
    }
    awq_store_group(rec, GQ, n, g, q, s, z);
}

// ------------------------------------------------------------------ linear
// One workgroup = one 16-column block x up to MT (<= 16) rows of X.  Its
// four waves take a quarter of the quads each, keep kAwqDepth records in
// flight, and add their partial tiles in LDS in wave order (deterministic).
// The rows' activations are staged once per workgroup in LDS, zero-padded to
// whole quads; their first loads are issued before the weight loads so the
// two latencies overlap.

constexpr int kAwqDepth = 2;   // records in flight per wave
constexpr int kAwqXUnits = 4;  // 16-byte activation units per thread held across the weight issue

namespace {

struct AwqQuad {
    u32x4 c0, c1;   // codes of groups 0-1 and 2-3 (this lane's column and k-slot)
    f32x4 s;        // scales of the 4 groups (this lane's column)
    uint32_t z;     // zero points of the 4 groups, one per byte
};

__device__ __forceinline__ void awq_load_quad(AwqQuad &d, const uint8_t *r, int lane, int col) {
    d.c0 = *reinterpret_cast<const u32x4 *>(r + 16 * lane);
    d.c1 = *reinterpret_cast<const u32x4 *>(r + 1024 + 16 * lane);
    d.s = *reinterpret_cast<const f32x4 *>(r + 2048 + 16 * col);
    d.z = *reinterpret_cast<const uint32_t *>(r + 2304 + 4 * col);
}

// 8 codes (one word of a record) -> 8 bf16 of 128 + q in k order.  The
// masks live in registers so that each pair is one v_and_or_b32.
__device__ __forceinline__ u32x4 awq_codes_to_bf16(uint32_t p, uint32_t mask, uint32_t bias128) {
    u32x4 r;
    r.x = (p & mask) | bias128;
    r.y = ((p >> 4) & mask) | bias128;
    r.z = ((p >> 8) & mask) | bias128;
    r.w = ((p >> 12) & mask) | bias128;
    return r;
}

}  // namespace

__global__ void __launch_bounds__(256)
awq_linear_kernel(const uint16_t *__restrict__ X, const uint8_t *__restrict__ rec,
                  const uint16_t *__restrict__ bias, int M, int N, int K, int MT,
                  uint16_t *__restrict__ Y) {
    extern __shared__ __attribute__((aligned(16))) uint8_t awq_smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, ks = lane >> 4;
    const int G = K >> 6, GQ = (G + 3) >> 2, G4 = 4 * GQ;
    const int cb = blockIdx.x;
    const int m0 = blockIdx.y * MT;
    const int R = M - m0 < MT ? M - m0 : MT;
    const int xstride = 128 * G4 + 16;   // bytes per staged row (16-byte pad against bank conflicts)

    // 1. first round of activation units into registers (addresses clamped)
    const int upr = K >> 3, units = R * upr;
    const float inv_upr = 1.0f / (float)upr;   // row = floor((u + 0.5) / upr), exact for u < 2^20
    const uint16_t *Xt = X + (size_t)m0 * K;
    u32x4 xv[kAwqXUnits];
#pragma unroll
    for (int i = 0; i < kAwqXUnits; ++i) {
        const int u0 = tid + 256 * i, u = u0 < units ? u0 : units - 1;
        const int r = (int)(((float)u + 0.5f) * inv_upr);
        xv[i] = *reinterpret_cast<const u32x4 *>(Xt + (size_t)r * K + 8 * (u - r * upr));
    }
    // 2. the first records of this wave's quads
    const int qb = GQ * wave / 4, qe = GQ * (wave + 1) / 4;
    const uint8_t *rbase = rec + (size_t)cb * GQ * kAwqRecord;
    AwqQuad ring[kAwqDepth];
#pragma unroll
    for (int d = 0; d < kAwqDepth; ++d)
        if (qb + d < qe) awq_load_quad(ring[d], rbase + (size_t)(qb + d) * kAwqRecord, lane, col);
    // 3. stage the activations (zero past K up to whole quads)
#pragma unroll
    for (int i = 0; i < kAwqXUnits; ++i) {
        const int u = tid + 256 * i;
        if (u < units) {
            const int r = (int)(((float)u + 0.5f) * inv_upr);
            *reinterpret_cast<u32x4 *>(awq_smem + r * xstride + 16 * (u - r * upr)) = xv[i];
        }
    }
    for (int u = kAwqXUnits * 256 + tid; u < units; u += 256) {
        const int r = (int)(((float)u + 0.5f) * inv_upr), c = u - r * upr;
        *reinterpret_cast<u32x4 *>(awq_smem + r * xstride + 16 * c) =
            *reinterpret_cast<const u32x4 *>(Xt + (size_t)r * K + 8 * c);
    }
    const int pad = (G4 - G) * 8;   // 16-byte units of zero padding per row
    for (int e = tid; e < R * pad; e += 256) {
        const int r = e / pad, c = e - r * pad;
        *reinterpret_cast<u32x4 *>(awq_smem + r * xstride + 128 * G + 16 * c) =
            u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();

    uint32_t mask, bias128;
    asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(mask));
    asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(bias128));
    const int xr = col < R ? col : R - 1;
    const uint8_t *xs = awq_smem + xr * xstride + 32 * ks;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int q0 = qb; q0 < qe; q0 += kAwqDepth) {
#pragma unroll
        for (int d = 0; d < kAwqDepth; ++d) {
            const int q = q0 + d;
            if (q < qe) {
                const AwqQuad cur = ring[d];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int g = 4 * q + j;
                    const u32x4 x0 = *reinterpret_cast<const u32x4 *>(xs + g * 128);
                    const u32x4 x1 = *reinterpret_cast<const u32x4 *>(xs + g * 128 + 16);
                    const u32x4 cp = j < 2 ? cur.c0 : cur.c1;
                    const uint32_t w0 = cp[2 * (j & 1)], w1 = cp[2 * (j & 1) + 1];
                    // -(128 + z) as a bf16 pair: byte j of the zero word under 0xC3
                    const uint32_t zz =
                        __builtin_amdgcn_perm(cur.z, 0xC3C3C3C3u, (4u + j) | ((4u + j) << 16));
                    const u32x4 bz = u32x4{zz, zz, zz, zz};
                    f32x4 t = mfma_bf16_16x16x32(x0, awq_codes_to_bf16(w0, mask, bias128),
                                                 f32x4{0.f, 0.f, 0.f, 0.f});
                    t = mfma_bf16_16x16x32(x1, awq_codes_to_bf16(w1, mask, bias128), t);
                    t = mfma_bf16_16x16x32(x0, bz, t);
                    t = mfma_bf16_16x16x32(x1, bz, t);
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(cur.s[j], t[r], acc[r]);
                }
                if (q + kAwqDepth < qe)
                    awq_load_quad(ring[d], rbase + (size_t)(q + kAwqDepth) * kAwqRecord, lane, col);
            }
        }
    }

    // lane holds rows 4 ks + r, column col of this wave's partial tile
    __syncthreads();
    float *red = reinterpret_cast<float *>(awq_smem);   // [4][16][17]
#pragma unroll
    for (int r = 0; r < 4; ++r) red[(wave * 16 + 4 * ks + r) * 17 + col] = acc[r];
    __syncthreads();
    const int tr = tid >> 4, tc = tid & 15;
    const int om = m0 + tr, on = cb * 16 + tc;
    if (tr < R && on < N) {
        float v = red[tr * 17 + tc];
        v += red[(16 + tr) * 17 + tc];
        v += red[(32 + tr) * 17 + tc];
        v += red[(48 + tr) * 17 + tc];
        if (bias) v += bf16_to_f32(bias[on]);
        Y[(size_t)om * N + on] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    }
}

// ------------------------------------------------------------------ launchers

int64_t awq_packed_bytes(int64_t N, int64_t K) {
    const int64_t NB = (N + 15) / 16, GQ = (K / kGroup + 3) / 4;
    return NB * GQ * kAwqRecord;
}

int awq_rows_per_pass(int64_t K, size_t lds_limit) {
    const int64_t GQ = (K / kGroup + 3) / 4;
    const size_t xstride = (size_t)(128 * 4 * GQ + 16);
    const size_t rows = lds_limit / xstride;
    return (int)(rows < 16 ? rows : 16);
}

hipError_t launch_awq_pack(const float *W, int64_t N, int64_t K, uint8_t *rec, hipStream_t stream) {
    const int64_t threads = (N + 15) / 16 * 16 * 4 * ((K / kGroup + 3) / 4);
    awq_pack_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(W, N, K, rec);
    return hipGetLastError();
}

hipError_t launch_awq_repack(const uint8_t *codes, const float *scales, const uint8_t *zeros,
                             int64_t N, int64_t K, uint8_t *rec, hipStream_t stream) {
    const int64_t threads = (N + 15) / 16 * 16 * 4 * ((K / kGroup + 3) / 4);
    awq_repack_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(codes, scales, zeros,
                                                                           N, K, rec);
    return hipGetLastError();
}

hipError_t launch_awq_linear(const uint16_t *X, const uint8_t *rec, const uint16_t *bias,
                             int64_t M, int64_t N, int64_t K, int MT, uint16_t *Y,
                             hipStream_t stream) {
    const int64_t GQ = (K / kGroup + 3) / 4;
    const int rows = (int)(M < MT ? M : MT);
    size_t lds = (size_t)rows * (128 * 4 * GQ + 16);
    if (lds < 4 * 16 * 17 * sizeof(float)) lds = 4 * 16 * 17 * sizeof(float);
    dim3 grid((unsigned)((N + 15) / 16), (unsigned)((M + MT - 1) / MT));
    awq_linear_kernel<<<grid, 256, lds, stream>>>(X, rec, bias, (int)M, (int)N, (int)K, MT, Y);
    return hipGetLastError();
}

}  // namespace svdq
