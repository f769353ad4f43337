// quant_down.hip -- activation side of the SVDQuant W4A4 layer on gfx950:
// smoothing, group-64 INT4 quantization and the rank-r down-projection in a
// single pass over X (the "Nunchaku engine design" section of the
// svdq-int4-flux.1-canny-dev model card fuses the down-projection with the
// quantizer because both read the same input), plus the offline weight
// quantizer, which uses the same group quantizer without smoothing.
#include "svdq_device.h"
#include "svdq_internal.h"

namespace svdq {

// ------------------------------------------------------------------ K1
// One workgroup = 64 rows of X (four waves of 16) and a chunk of KC groups
// of K.  Everything the chunk needs is requested up front, in this order:
// lambda and the chunk of L1 (small, read first so that their use does not
// wait for the rest), then the X of all KC groups of the wave's rows, which
// stays in flight while the workgroup computes fl32(1 / lambda) and stages
// the chunk of L1 transposed in LDS ([column][k], 8 consecutive k = one
// 16-byte read), shared by the four waves.  The loads have fixed counts
// (addresses past the chunk or the rank are clamped and the data ignored),
// so each group waits only for its own X.  (X is deliberately not declared
// restrict: loads from a read-only restrict argument may be re-issued after
// the barrier instead of being kept in registers.)
//
// Per group, lane l owns row l % 16 and the 16 consecutive elements at
// 16 (l / 16): the four lanes of a group reduce the absmax with two lane
// exchanges.  The down-projection uses the smoothed values x^ themselves,
// split into bf16 hi + lo (x^ - hi), as the A operand of a bf16 MFMA
// (16x16x32: lane l holds 8 consecutive k of row l % 16 in k-slot l / 16)
// against the raw bf16 L1: every product is exact in fp32 and the split keeps
// about 16 significant bits of x^.  A chunk's result is either xl1 itself
// (one chunk) or a partial sum that xl1_reduce_kernel adds up in a fixed order,
// so the result does not depend on scheduling.
constexpr int K1_ROWS = 64;

// KC groups per chunk (k1_chunk_groups); the staged L1 chunk is 64 KC x 16 NT bf16.
// MX: the 4-bit float (MXFP4) variant -- the same smoothing and
// down-projection, the MX quantizer per 32-value block, E8M0 scale bytes block-major in sa
// ([K/32][mx_scale_rows(M)]).
template <int NT, int KC, bool MX = false>
__global__ void __launch_bounds__(256)
quant_down_kernel(const uint16_t *X, const float *__restrict__ lambda,
                  const uint16_t *__restrict__ L1, int64_t M, int64_t K, int r, int nc,
                  uint8_t *__restrict__ qa, void *__restrict__ sa, float *__restrict__ out,
                  int64_t out_chunk_stride) {
    constexpr int S = KC * kGroup + 8;                 // LDS row of the L1 chunk, bf16
    constexpr int NLAM = (KC * kGroup + 255) / 256;    // lambda loads per thread
    constexpr int NL1 = NT > 0 ? KC * NT / 2 : 0;      // 16-byte L1 pieces per thread
    __shared__ float inv[KC * kGroup];
    __shared__ __align__(16) uint16_t l1t[NT > 0 ? 16 * NT * S : 8];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int rl = lane & 15;
    const int ks = lane >> 4;
    const int64_t c = blockIdx.x % nc;                 // chunk
    const int64_t rb = blockIdx.x / nc;                // row block
    const int64_t G = K / kGroup;
    const int64_t g0 = c * KC;
    const int gc = (int)((G - g0) < KC ? (G - g0) : KC);
    const int64_t row = rb * K1_ROWS + wave * 16 + rl;
    const bool row_ok = row < M;
    const int64_t rowc = row_ok ? row : M - 1;
    const int nt = r >> 4;
    const int64_t kbase = g0 * kGroup;
    const int kvalid = gc * kGroup;
    // Stored addresses: a per-lane part here, a wave-uniform part per group.
    // Codes (row pairs, code_offset): byte 32 g + 8 ks of the row is at
    // (row / 2) K + (row % 2) w + 64 g - 32 (g % 2) + 8 ks, w = 64 except in
    // the 32-byte last chunk of an odd group count (w = 32).  Scales
    // (stage-major, scale_index): 2 row + 2 M (g / 2) + g % 2.
    const int64_t kb = K / 2;
    uint8_t *const qrow = qa + (row >> 1) * 2 * kb + 8 * ks;
    const int64_t qodd = (row & 1) * 64;
    float *const srow = static_cast<float *>(sa) + 2 * row;

    // 1. lambda and the L1 chunk, then X, all in flight together
    float lam[NLAM];
#pragma unroll
    for (int j = 0; j < NLAM; ++j) {
        const int k = tid + 256 * j;
        lam[j] = lambda[kbase + (k < kvalid ? k : kvalid - 1)];
    }
    u32x4 l1v[NL1 > 0 ? NL1 : 1];
    int l1k[NL1 > 0 ? NL1 : 1], l1n[NL1 > 0 ? NL1 : 1];
#pragma unroll
    for (int j = 0; j < NL1; ++j) {
        const int q = tid + 256 * j;                   // piece: k = q / (2 NT), columns 8 (q % 2NT)
        constexpr int PR = NT > 0 ? 2 * NT : 1;        // pieces per k row
        const int kk = q / PR;
        const int n0 = 8 * (q - kk * PR);
        l1k[j] = kk;
        l1n[j] = n0;
        const int kc_ = kk < kvalid ? kk : kvalid - 1;
        const int nc_ = n0 < r ? n0 : 0;
        l1v[j] = *reinterpret_cast<const u32x4 *>(L1 + (kbase + kc_) * r + nc_);
    }
    __builtin_amdgcn_sched_barrier(0);                 // keep the small loads first
    u32x4 xa[KC], xb[KC];
    const uint16_t *xrow = X + rowc * K + kbase + 16 * ks;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int ic = i < gc ? i : gc - 1;
        xa[i] = *reinterpret_cast<const u32x4 *>(xrow + ic * kGroup);
        xb[i] = *reinterpret_cast<const u32x4 *>(xrow + ic * kGroup + 8);
    }
    __builtin_amdgcn_sched_barrier(0);

    // 2. 1/lambda and the transposed L1 chunk into LDS (X still in flight)
#pragma unroll
    for (int j = 0; j < NLAM; ++j) {
        const int k = tid + 256 * j;
        if (256 * (j + 1) <= KC * kGroup || k < KC * kGroup) inv[k] = 1.0f / lam[j];
    }
    // (columns past r hold copies that are never read; writing them keeps the
    // loads above unconditional)
#pragma unroll
    for (int j = 0; j < NL1; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            l1t[(l1n[j] + 2 * e) * S + l1k[j]] = (uint16_t)(l1v[j][e] & 0xFFFFu);
            l1t[(l1n[j] + 2 * e + 1) * S + l1k[j]] = (uint16_t)(l1v[j][e] >> 16);
        }
    }
    // LDS writes done, then a barrier without a memory fence (the X loads
    // stay outstanding across it)
    __builtin_amdgcn_s_waitcnt(0xC07F);                // lgkmcnt(0); vmcnt, expcnt untouched
    asm volatile("s_barrier" ::: "memory");

    f32x4 acc[NT > 0 ? NT : 1];
#pragma unroll
    for (int t = 0; t < (NT > 0 ? NT : 1); ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < KC; ++i) {
        if (i < gc) {
            const int64_t g = g0 + i;
            const f32x4 *ip = reinterpret_cast<const f32x4 *>(inv + i * kGroup + 16 * ks);
            const f32x4 i0 = ip[0], i1 = ip[1], i2 = ip[2], i3 = ip[3];
            const u32x4 x0 = xa[i], x1 = xb[i];
            float v[16];
            v[0] = bf16_lo(x0.x) * i0.x;  v[1] = bf16_hi(x0.x) * i0.y;
            v[2] = bf16_lo(x0.y) * i0.z;  v[3] = bf16_hi(x0.y) * i0.w;
            v[4] = bf16_lo(x0.z) * i1.x;  v[5] = bf16_hi(x0.z) * i1.y;
            v[6] = bf16_lo(x0.w) * i1.z;  v[7] = bf16_hi(x0.w) * i1.w;
            v[8] = bf16_lo(x1.x) * i2.x;  v[9] = bf16_hi(x1.x) * i2.y;
            v[10] = bf16_lo(x1.y) * i2.z; v[11] = bf16_hi(x1.y) * i2.w;
            v[12] = bf16_lo(x1.z) * i3.x; v[13] = bf16_hi(x1.z) * i3.y;
            v[14] = bf16_lo(x1.w) * i3.z; v[15] = bf16_hi(x1.w) * i3.w;
            u32x2 packed;
            if constexpr (MX) {
                const uint32_t sb = mx_quantize16(v, packed);
                if (row_ok) {
                    *reinterpret_cast<u32x2 *>(qa + code_offset(row, K / 2, g * (kGroup / 2) + 8 * ks)) =
                        packed;
                    if ((ks & 1) == 0)
                        static_cast<uint8_t *>(sa)[(2 * g + (ks >> 1)) * mx_scale_rows(M) + row] =
                            (uint8_t)sb;
                }
            } else {
                const float s = quantize_group16(v, packed);
                if (row_ok) {
                    const bool half = (G & 1) && g == G - 1;           // 32-byte last chunk
                    const int64_t go = 64 * g - 32 * (g & 1);
                    *reinterpret_cast<u32x2 *>(qrow + go + (half ? qodd / 2 : qodd)) = packed;
                    if (ks == 0) {
                        const int64_t so = 2 * M * (g >> 1) + (g & 1);
                        srow[so] = s;
                        if (half) srow[so + 1] = 0.0f;                  // pad (g even here)
                    }
                }
            }
            if (NT > 0) {
                u32x4 h[2], l[2];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t hp = pack_bf16x2(v[2 * e], v[2 * e + 1]);
                    h[e >> 2][e & 3] = hp;
                    l[e >> 2][e & 3] = pack_bf16x2(v[2 * e] - bf16_lo(hp), v[2 * e + 1] - bf16_hi(hp));
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if (t < nt) {
                        const uint16_t *bp = l1t + (16 * t + rl) * S + i * kGroup + 16 * ks;
                        const u32x4 b0 = *reinterpret_cast<const u32x4 *>(bp);
                        const u32x4 b1 = *reinterpret_cast<const u32x4 *>(bp + 8);
                        acc[t] = mfma_bf16_16x16x32(h[0], b0, acc[t]);
                        acc[t] = mfma_bf16_16x16x32(l[0], b0, acc[t]);
                        acc[t] = mfma_bf16_16x16x32(h[1], b1, acc[t]);
                        acc[t] = mfma_bf16_16x16x32(l[1], b1, acc[t]);
                    }
                }
            }
        }
    }
    if (NT == 0) return;

    // This chunk's x^ L1: lane holds rows 4 ks + j, column 16 t + rl.
    float *o = out + c * out_chunk_stride;
#pragma unroll
    for (int t = 0; t < (NT > 0 ? NT : 1); ++t) {
        if (t < nt) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t orow = rb * K1_ROWS + wave * 16 + 4 * ks + j;
                if (orow < M) o[orow * r + 16 * t + rl] = acc[t][j];
            }
        }
    }
}

// xl1 = the sum of the nc partial sums [nc][total].  A workgroup takes 64
// consecutive f32x4 of the output and splits the partials into four slices
// of ceil(nc / 4); wave j adds the partials of slice j in order (eight loads
// in flight at a time), then the slice sums are added as ((s0 + s1) + s2) +
// s3.  The order is fixed, so the result does not depend on scheduling.
constexpr int kReduceCols = 64;   // f32x4 outputs per workgroup
__global__ void __launch_bounds__(256)
xl1_reduce_kernel(const float *__restrict__ part, int nc, int64_t total, float *__restrict__ xl1) {
    __shared__ f32x4 red[3][kReduceCols];
    const int lane = threadIdx.x & 63, j = threadIdx.x >> 6;
    const int64_t i = ((int64_t)blockIdx.x * kReduceCols + lane) * 4;
    const bool ok = i < total;
    const int per = (nc + 3) / 4;
    const int c0 = j * per < nc ? j * per : nc;
    const int c1 = c0 + per < nc ? c0 + per : nc;
    f32x4 s{0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
        int c = c0;
        for (; c + 8 <= c1; c += 8) {
            f32x4 p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                p[e] = *reinterpret_cast<const f32x4 *>(part + (int64_t)(c + e) * total + i);
#pragma unroll
            for (int e = 0; e < 8; ++e) s = f32x4{s.x + p[e].x, s.y + p[e].y, s.z + p[e].z, s.w + p[e].w};
        }
        for (; c < c1; ++c) {
            const f32x4 p = *reinterpret_cast<const f32x4 *>(part + (int64_t)c * total + i);
            s = f32x4{s.x + p.x, s.y + p.y, s.z + p.z, s.w + p.w};
        }
    }
    if (j > 0) red[j - 1][lane] = s;
    __syncthreads();
    if (j == 0 && ok) {
#pragma unroll
        for (int q = 0; q < 3; ++q) {
            const f32x4 p = red[q][lane];
            s = f32x4{s.x + p.x, s.y + p.y, s.z + p.z, s.w + p.w};
        }
        *reinterpret_cast<f32x4 *>(xl1 + i) = s;
    }
}

// ------------------------------------------------------------------ pack
// Offline quantization of the fp32 residual R [N, K]: one wave per 16 rows,
// the same lane layout and group quantizer as K1 (no smoothing).
template <bool MX = false>
__global__ void __launch_bounds__(256)
pack_weights_kernel(const float *__restrict__ R, int64_t N, int64_t K,
                    uint8_t *__restrict__ qw, void *__restrict__ sw) {
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
        if constexpr (MX) {
            const uint32_t sb = mx_quantize16(v, packed);
            if (row_ok) {
                *reinterpret_cast<u32x2 *>(qw + code_offset(row, K / 2, g * (kGroup / 2) + 8 * ks)) = packed;
                if ((ks & 1) == 0)
                    static_cast<uint8_t *>(sw)[(2 * g + (ks >> 1)) * mx_scale_rows(N) + row] =
                        (uint8_t)sb;
            }
        } else {
            const float s = quantize_group16(v, packed);
            if (row_ok) {
                *reinterpret_cast<u32x2 *>(qw + code_offset(row, K / 2, g * (kGroup / 2) + 8 * ks)) = packed;
                if (ks == 0) {
                    float *sp = static_cast<float *>(sw);
                    sp[scale_index(row, g, N)] = s;
                    if ((G & 1) && g == G - 1) sp[scale_index(row, G, N)] = 0.0f;   // pad
                }
            }
        }
    }
}

// ------------------------------------------------------------------ repack
// Already quantized weights in the common row-major form (codes: two's
// complement nibbles, element 2j in the low nibble of byte j, [N, K/2];
// scales fp32 [N, K/64]) -> the stored layouts: one thread per block of 16
// codes (8 bytes), the same conversion as the quantizers' (store_code_words),
// written to the row-pair position; the thread of a group's first block also
// moves the group's scale (and, for an odd group count, zeroes the pad).  A
// nibble 8 (-8, outside the symmetric range) is stored as -7.
__global__ void __launch_bounds__(256)
repack_codes_kernel(const uint8_t *__restrict__ codes, const float *__restrict__ scales,
                    int64_t N, int64_t K, uint8_t *__restrict__ qw, float *__restrict__ sw) {
    const int64_t kb = K / 2, per_row = K / 16, G = K / kGroup;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N * per_row) return;
    const int64_t row = i / per_row, t = i - row * per_row;
    const u32x2 w = *reinterpret_cast<const u32x2 *>(codes + row * kb + 8 * t);
    auto no_m8 = [](uint32_t x) {
        // nibbles equal to 8: sign bit set, magnitude bits zero -> 9 (-7)
        const uint32_t zero_mag = ~((x & 0x77777777u) + 0x77777777u) & 0x88888888u;
        return x | ((x & zero_mag & 0x88888888u) >> 3);
    };
    *reinterpret_cast<u32x2 *>(qw + code_offset(row, kb, 8 * t)) =
        store_code_words(no_m8(w.x), no_m8(w.y));
    if ((t & 3) == 0) {
        const int64_t g = t >> 2;
        sw[scale_index(row, g, N)] = scales[row * G + g];
        if ((G & 1) && g == G - 1) sw[scale_index(row, G, N)] = 0.0f;
    }
}

// ------------------------------------------------------------------ launchers

hipError_t launch_quant_down(const uint16_t *X, const float *lambda, const uint16_t *L1,
                             int64_t M, int64_t K, int r, const DownWorkspace &ws, uint8_t *qa,
                             void *sa, float *xl1, hipStream_t stream, bool mx) {
    const int nc = k1_chunks(M, K, r);
    const int kc = k1_chunk_groups(M, K, r);
    const int64_t rbs = (M + K1_ROWS - 1) / K1_ROWS;
    const unsigned blocks = (unsigned)(rbs * nc);
    const bool partial = r > 0 && nc > 1;
    float *out = partial ? ws.part : xl1;
    const int64_t stride = partial ? M * (int64_t)r : 0;
#define SVDQ_K1(NTV, KCV)                                                                  \
    do {                                                                                   \
        if (mx)                                                                            \
            quant_down_kernel<NTV, KCV, true><<<blocks, 256, 0, stream>>>(                  \
                X, lambda, L1, M, K, r, nc, qa, sa, out, stride);                          \
        else                                                                               \
            quant_down_kernel<NTV, KCV><<<blocks, 256, 0, stream>>>(                        \
                X, lambda, L1, M, K, r, nc, qa, sa, out, stride);                          \
    } while (0)
#define SVDQ_K1_KC(NTV)                                                                    \
    do {                                                                                   \
        if (kc == 8) SVDQ_K1(NTV, 8);                                                      \
        else if (kc == 4) SVDQ_K1(NTV, 4);                                                 \
        else SVDQ_K1(NTV, 2);                                                              \
    } while (0)
    if (r == 0) SVDQ_K1_KC(0);
    else if (r <= 32) SVDQ_K1_KC(2);
    else if (r <= 64) SVDQ_K1(4, 4);
    else SVDQ_K1(8, 2);
#undef SVDQ_K1_KC
#undef SVDQ_K1
    if (partial) {
        const int64_t total = M * (int64_t)r;
        const unsigned rblocks = (unsigned)((total / 4 + kReduceCols - 1) / kReduceCols);
        xl1_reduce_kernel<<<rblocks, 256, 0, stream>>>(ws.part, nc, total, xl1);
    }
    return hipGetLastError();
}

hipError_t launch_xl1_reduce(const float *part, int nc, int64_t total, float *xl1,
                             hipStream_t stream) {
    const unsigned rblocks = (unsigned)((total / 4 + kReduceCols - 1) / kReduceCols);
    xl1_reduce_kernel<<<rblocks, 256, 0, stream>>>(part, nc, total, xl1);
    return hipGetLastError();
}

hipError_t launch_repack_codes(const uint8_t *codes, const float *scales, int64_t N, int64_t K,
                               uint8_t *qw, float *sw, hipStream_t stream) {
    const int64_t threads = N * (K / 16);
    repack_codes_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, stream>>>(codes, scales, N, K,
                                                                             qw, sw);
    return hipGetLastError();
}

hipError_t launch_pack_weights(const float *R, int64_t N, int64_t K, uint8_t *qw, void *sw,
                               hipStream_t stream, bool mx) {
    const int64_t waves = (N + 15) / 16;
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (mx) pack_weights_kernel<true><<<blocks, 256, 0, stream>>>(R, N, K, qw, sw);
    else pack_weights_kernel<<<blocks, 256, 0, stream>>>(R, N, K, qw, sw);
    return hipGetLastError();
}

}  // namespace svdq
