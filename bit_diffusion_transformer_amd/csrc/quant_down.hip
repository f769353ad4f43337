// quant_down.hip -- activation side of the SVDQuant W4A4 layer on gfx950:
// smoothing, group-64 INT4 quantization and the rank-r down-projection in a
// single pass over X (the "Nunchaku engine design" section of the
// svdq-int4-flux.1-canny-dev model card fuses the down-projection with the
// quantizer because both read the same input), plus the offline weight
// quantizer, which uses the same group quantizer without smoothing.
#include "svdq_device.h"
#include "svdq_internal.h"

namespace svdq {

// ------------------------------------------------------------------ prep
// inv_lam[k] = fl32(1 / lambda[k]);  L1s = fl32(L1[k][i] * inv_lam[k]) split
// into bf16 hi = rn(L1s), lo = rn(L1s - hi), stored transposed [r][K] so the
// down-projection reads 8 consecutive k per lane.  X diag(lambda)^-1 L1 is
// then computed as X (L1s_hi + L1s_lo) with X exact in bf16: every product
// is exact in fp32 and the split keeps ~16 significant bits of L1s.
__global__ void __launch_bounds__(256)
prep_down_kernel(const float *__restrict__ lambda, const uint16_t *__restrict__ L1,
                 int64_t K, int r, float *__restrict__ inv_lam,
                 uint16_t *__restrict__ l1_hi, uint16_t *__restrict__ l1_lo) {
    const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (k >= K) return;
    const float il = 1.0f / lambda[k];
    if (blockIdx.y == 0) inv_lam[k] = il;
    for (int i = blockIdx.y; i < r; i += gridDim.y) {
        const float s = bf16_to_f32(L1[k * r + i]) * il;
        const uint32_t hi_lo = pack_bf16x2(s, 0.0f);
        const float hi = bf16_lo(hi_lo);
        const uint32_t lo_pair = pack_bf16x2(s - hi, 0.0f);
        l1_hi[(int64_t)i * K + k] = (uint16_t)(hi_lo & 0xFFFFu);
        l1_lo[(int64_t)i * K + k] = (uint16_t)(lo_pair & 0xFFFFu);
    }
}

// ------------------------------------------------------------------ K1
// One workgroup = 16 rows of X and KW waves that split the K groups between
// them.  Lane l owns row l % 16 and, inside every group of 64, the 16
// consecutive elements starting at 16 * (l / 16): the four lanes of a group
// reduce the absmax with two lane exchanges.  The same registers feed the
// bf16 MFMA of the down-projection as its A operand (16x16x32: lane l holds
// 8 consecutive k of row l % 16 in k-slot l / 16), with the transposed hi/lo
// factor as the B operand; the partial products of the KW waves are summed
// in LDS in wave order, so the result does not depend on scheduling.
template <int KW, int NTMAX>
__global__ void __launch_bounds__(64 * KW)
quant_down_kernel(const uint16_t *__restrict__ X, const float *__restrict__ inv_lam,
                  const uint16_t *__restrict__ l1_hi, const uint16_t *__restrict__ l1_lo,
                  int64_t M, int64_t K, int r, uint8_t *__restrict__ qa,
                  float *__restrict__ sa, float *__restrict__ xl1) {
    extern __shared__ float red[];   // [KW][16][r]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int rl = lane & 15;
    const int ks = lane >> 4;
    const int64_t row = (int64_t)blockIdx.x * 16 + rl;
    const bool row_ok = row < M;
    const int64_t rowc = row_ok ? row : M - 1;
    const int64_t G = K / kGroup;
    const int64_t g_begin = G * wave / KW;
    const int64_t g_end = G * (wave + 1) / KW;
    const int nt = r >> 4;

    f32x4 acc[NTMAX];
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Software pipeline: the next group's X and 1/lambda are in flight while
    // the current group is quantized; the current group's down-projection
    // operands are issued before the quantizer math that hides their latency.
    const uint16_t *xrow = X + rowc * K;
    u32x4 nxa = u32x4{0u, 0u, 0u, 0u}, nxb = nxa;
    f32x4 ni0 = f32x4{0.f, 0.f, 0.f, 0.f}, ni1 = ni0, ni2 = ni0, ni3 = ni0;
    if (g_begin < g_end) {
        const int64_t k0 = g_begin * kGroup + 16 * ks;
        nxa = *reinterpret_cast<const u32x4 *>(xrow + k0);
        nxb = *reinterpret_cast<const u32x4 *>(xrow + k0 + 8);
        const f32x4 *il4 = reinterpret_cast<const f32x4 *>(inv_lam + k0);
        ni0 = il4[0]; ni1 = il4[1]; ni2 = il4[2]; ni3 = il4[3];
    }
    for (int64_t g = g_begin; g < g_end; ++g) {
        const int64_t k0 = g * kGroup + 16 * ks;
        const u32x4 xa = nxa, xb = nxb;
        const f32x4 i0 = ni0, i1 = ni1, i2 = ni2, i3 = ni3;
        if (g + 1 < g_end) {
            nxa = *reinterpret_cast<const u32x4 *>(xrow + k0 + kGroup);
            nxb = *reinterpret_cast<const u32x4 *>(xrow + k0 + kGroup + 8);
            const f32x4 *il4 = reinterpret_cast<const f32x4 *>(inv_lam + k0 + kGroup);
            ni0 = il4[0]; ni1 = il4[1]; ni2 = il4[2]; ni3 = il4[3];
        }
        u32x4 bh[NTMAX][2], bl[NTMAX][2];
#pragma unroll
        for (int t = 0; t < NTMAX; ++t) {
            if (t < nt) {
                const int64_t col = (int64_t)(16 * t + rl);
                bh[t][0] = *reinterpret_cast<const u32x4 *>(l1_hi + col * K + k0);
                bh[t][1] = *reinterpret_cast<const u32x4 *>(l1_hi + col * K + k0 + 8);
                bl[t][0] = *reinterpret_cast<const u32x4 *>(l1_lo + col * K + k0);
                bl[t][1] = *reinterpret_cast<const u32x4 *>(l1_lo + col * K + k0 + 8);
            }
        }
        float v[16];
        v[0] = bf16_lo(xa.x) * i0.x;  v[1] = bf16_hi(xa.x) * i0.y;
        v[2] = bf16_lo(xa.y) * i0.z;  v[3] = bf16_hi(xa.y) * i0.w;
        v[4] = bf16_lo(xa.z) * i1.x;  v[5] = bf16_hi(xa.z) * i1.y;
        v[6] = bf16_lo(xa.w) * i1.z;  v[7] = bf16_hi(xa.w) * i1.w;
        v[8] = bf16_lo(xb.x) * i2.x;  v[9] = bf16_hi(xb.x) * i2.y;
        v[10] = bf16_lo(xb.y) * i2.z; v[11] = bf16_hi(xb.y) * i2.w;
        v[12] = bf16_lo(xb.z) * i3.x; v[13] = bf16_hi(xb.z) * i3.y;
        v[14] = bf16_lo(xb.w) * i3.z; v[15] = bf16_hi(xb.w) * i3.w;
        u32x2 packed;
        const float s = quantize_group16(v, packed);
        if (row_ok) {
            *reinterpret_cast<u32x2 *>(qa + row * (K / 2) + g * (kGroup / 2) + 8 * ks) = packed;
            if (ks == 0) sa[row * G + g] = s;
        }
#pragma unroll
        for (int t = 0; t < NTMAX; ++t) {
            if (t < nt) {
                acc[t] = mfma_bf16_16x16x32(xa, bh[t][0], acc[t]);
                acc[t] = mfma_bf16_16x16x32(xa, bl[t][0], acc[t]);
                acc[t] = mfma_bf16_16x16x32(xb, bh[t][1], acc[t]);
                acc[t] = mfma_bf16_16x16x32(xb, bl[t][1], acc[t]);
            }
        }
    }
    if (nt == 0) return;

    // Partial XL1 of this wave: lane holds rows 4*ks + j, column 16 t + rl.
#pragma unroll
    for (int t = 0; t < NTMAX; ++t) {
        if (t < nt) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red[(wave * 16 + 4 * ks + j) * r + 16 * t + rl] = acc[t][j];
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * r; idx += 64 * KW) {
        const int rr = idx / r;
        const int c = idx - rr * r;
        float sum = 0.0f;
        for (int w = 0; w < KW; ++w) sum += red[(w * 16 + rr) * r + c];
        const int64_t orow = (int64_t)blockIdx.x * 16 + rr;
        if (orow < M) xl1[orow * r + c] = sum;
    }
}

// ------------------------------------------------------------------ pack
// Offline quantization of the fp32 residual R [N, K]: one wave per 16 rows,
// the same lane layout and group quantizer as K1 (no smoothing).
__global__ void __launch_bounds__(256)
pack_weights_kernel(const float *__restrict__ R, int64_t N, int64_t K,
                    uint8_t *__restrict__ qw, float *__restrict__ sw) {
    const int lane = threadIdx.x & 63;
    const int64_t wave_id = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int rl = lane & 15;
    const int ks = lane >> 4;
    const int64_t row = wave_id * 16 + rl;
    if (wave_id * 16 >= N) return;
    const bool row_ok = row < N;
    const int64_t rowc = row_ok ? row : N - 1;
    const int64_t G = K / kGroup;
    for (int64_t g = 0; g < G; ++g) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(R + rowc * K + g * kGroup + 16 * ks);
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 t = p[q];
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
        u32x2 packed;
        const float s = quantize_group16(v, packed);
        if (row_ok) {
            *reinterpret_cast<u32x2 *>(qw + row * (K / 2) + g * (kGroup / 2) + 8 * ks) = packed;
            if (ks == 0) sw[row * G + g] = s;
        }
    }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_prep_down(const float *lambda, const uint16_t *L1, int64_t K, int r,
                            const DownWorkspace &ws, hipStream_t stream) {
    dim3 grid((unsigned)((K + 255) / 256), (unsigned)(r > 0 ? (r < 8 ? r : 8) : 1));
    prep_down_kernel<<<grid, 256, 0, stream>>>(lambda, L1, K, r, ws.inv_lam, ws.l1_hi, ws.l1_lo);
    return hipGetLastError();
}

int choose_kw(int64_t M, int64_t K, int r) {
    const int64_t blocks = (M + 15) / 16;
    const int64_t G = K / kGroup;
    int kw = 1;
    while (kw < 16 && blocks * kw < 2048 && 2 * kw <= G && 2 * kw * r <= 1024) kw *= 2;
    return kw;
}

hipError_t launch_quant_down(const uint16_t *X, int64_t M, int64_t K, int r,
                             const DownWorkspace &ws, uint8_t *qa, float *sa, float *xl1,
                             hipStream_t stream) {
    const int kw = choose_kw(M, K, r);
    const unsigned blocks = (unsigned)((M + 15) / 16);
    const size_t lds = (size_t)kw * 16 * (size_t)r * sizeof(float);
#define SVDQ_K1(KWV, NTM)                                                                  \
    quant_down_kernel<KWV, NTM><<<blocks, 64 * KWV, lds, stream>>>(                        \
        X, ws.inv_lam, ws.l1_hi, ws.l1_lo, M, K, r, qa, sa, xl1)
#define SVDQ_K1_KW(NTM)                                                                    \
    switch (kw) {                                                                          \
        case 1: SVDQ_K1(1, NTM); break;                                                    \
        case 2: SVDQ_K1(2, NTM); break;                                                    \
        case 4: SVDQ_K1(4, NTM); break;                                                    \
        case 8: SVDQ_K1(8, NTM); break;                                                    \
        case 16: SVDQ_K1(16, NTM); break;                                                  \
        default: return hipErrorInvalidValue;                                              \
    }
    const int nt = r / 16;
    if (nt <= 2) {
        SVDQ_K1_KW(2)
    } else if (nt <= 4) {
        SVDQ_K1_KW(4)
    } else {
        SVDQ_K1_KW(8)
    }
#undef SVDQ_K1_KW
#undef SVDQ_K1
    return hipGetLastError();
}

hipError_t launch_pack_weights(const float *R, int64_t N, int64_t K, uint8_t *qw, float *sw,
                               hipStream_t stream) {
    const int64_t waves = (N + 15) / 16;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    pack_weights_kernel<<<blocks, 256, 0, stream>>>(R, N, K, qw, sw);
    return hipGetLastError();
}

}  // namespace svdq
