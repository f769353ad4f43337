// w4a4_gemm.hip -- the W4A4 GEMM of the SVDQuant layer on gfx950 with the
// rank-r up-projection, bias and GELU applied to the same output tile before
// its single bf16 store (the "Nunchaku engine design" section of the
// svdq-int4-flux.1-canny-dev model card fuses the up-projection with the
// 4-bit compute because both produce the same output).
//
// Output tiles are computed transposed, D[n][m] = Y[m][n]: the weight codes
// are the MFMA A operand and the activation codes the B operand, so that an
// output lane holds four consecutive n of one token row and stores them as
// one 8-byte write.
#include "svdq_device.h"
#include "svdq_internal.h"

namespace svdq {

namespace {

constexpr int BN = 128;           // tile rows in n (weights)
constexpr int BM = 128;           // tile cols in m (tokens)
constexpr int GC = 4;             // K groups per LDS stage
constexpr int ROWB = GC * 32;     // packed bytes of one row per stage
constexpr int ASTR = ROWB + 8;    // LDS row stride (bytes); +8 spreads the banks
constexpr int NTHR = 256;         // 4 waves, 2 (n) x 2 (m), 64 x 64 each
constexpr int GROUP_M = 8;        // m-tiles per raster group (L2 reuse of weights)

struct __align__(16) Smem {
    uint8_t a[2][BN * ASTR];
    uint8_t b[2][BM * ASTR];
    float sw[2][GC][BN];
    float sa[2][GC][BM];
};
static_assert(sizeof(Smem) <= 80 * 1024, "LDS budget");

struct StageRegs {
    u32x4 a[4];
    u32x4 b[4];
    float s[GC];
};

__device__ __forceinline__ void load_stage(StageRegs &st, const uint8_t *__restrict__ qw,
                                           const uint8_t *__restrict__ qa,
                                           const float *__restrict__ sw,
                                           const float *__restrict__ sa, int64_t M, int64_t N,
                                           int64_t K, int64_t G, int64_t n0, int64_t m0,
                                           int64_t c) {
    const int tid = threadIdx.x;
    const int64_t kb = K / 2;
    const int64_t gleft = G - c * GC;                 // groups left in this stage
    const int valid_bytes = (int)(gleft >= GC ? ROWB : gleft * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + NTHR * i;
        const int row = q >> 3;
        const int seg = (q & 7) * 16;
        const int64_t n = n0 + row < N ? n0 + row : N - 1;
        const int64_t m = m0 + row < M ? m0 + row : M - 1;
        if (seg < valid_bytes) {
            st.a[i] = *reinterpret_cast<const u32x4 *>(qw + n * kb + c * ROWB + seg);
            st.b[i] = *reinterpret_cast<const u32x4 *>(qa + m * kb + c * ROWB + seg);
        } else {
            st.a[i] = u32x4{0u, 0u, 0u, 0u};
            st.b[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    const bool is_w = tid < BN;
    const int row = is_w ? tid : tid - BN;
    const int64_t idx = is_w ? (n0 + row < N ? n0 + row : N - 1) : (m0 + row < M ? m0 + row : M - 1);
    const float *src = is_w ? sw : sa;
#pragma unroll
    for (int gi = 0; gi < GC; ++gi)
        st.s[gi] = (gi < gleft) ? src[idx * G + c * GC + gi] : 0.0f;
}

__device__ __forceinline__ void store_stage(const StageRegs &st, Smem &sm, int buf) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = tid + NTHR * i;
        const int row = q >> 3;
        const int seg = (q & 7) * 16;
        *reinterpret_cast<u32x4 *>(&sm.a[buf][row * ASTR + seg]) = st.a[i];
        *reinterpret_cast<u32x4 *>(&sm.b[buf][row * ASTR + seg]) = st.b[i];
    }
    // The weight scale carries the 2^-8 that undoes the x16 of both widened
    // operands (exact: a power-of-two scaling).
    if (tid < BN) {
#pragma unroll
        for (int gi = 0; gi < GC; ++gi) sm.sw[buf][gi][tid] = st.s[gi] * 0.00390625f;
    } else {
#pragma unroll
        for (int gi = 0; gi < GC; ++gi) sm.sa[buf][gi][tid - BN] = st.s[gi];
    }
}

__device__ __forceinline__ void tile_coords(int64_t M, int64_t N, int64_t &tm, int64_t &tn) {
    const int64_t nbm = (M + BM - 1) / BM;
    const int64_t nbn = (N + BN - 1) / BN;
    const int64_t total = nbm * nbn;
    int64_t b = blockIdx.x;
    // Consecutive workgroups go to different XCDs (round robin over 8); give
    // each XCD a contiguous range of tiles so the tiles sharing operands share
    // that XCD's L2.
    if ((total & 7) == 0) b = (b & 7) * (total >> 3) + (b >> 3);
    const int64_t per_group = (int64_t)GROUP_M * nbn;
    const int64_t grp = b / per_group;
    const int64_t first_m = grp * GROUP_M;
    const int64_t gsize = (nbm - first_m) < GROUP_M ? (nbm - first_m) : GROUP_M;
    const int64_t in_grp = b - grp * per_group;
    tm = first_m + in_grp % gsize;
    tn = in_grp / gsize;
}

}  // namespace

__global__ void __launch_bounds__(NTHR)
w4a4_lr_gemm_kernel(const uint8_t *__restrict__ qa, const float *__restrict__ sa,
                    const uint8_t *__restrict__ qw, const float *__restrict__ sw,
                    const float *__restrict__ xl1, const uint16_t *__restrict__ L2,
                    const uint16_t *__restrict__ bias, int act, int64_t M, int64_t N,
                    int64_t K, int r, uint16_t *__restrict__ Y) {
    __shared__ Smem sm;
    int64_t tm, tn;
    tile_coords(M, N, tm, tn);
    const int64_t m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave >> 1, wm = wave & 1;
    const int rl = lane & 15, ks = lane >> 4;
    const int64_t G = K / kGroup;
    const int64_t nstages = (G + GC - 1) / GC;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    StageRegs st;
    load_stage(st, qw, qa, sw, sa, M, N, K, G, n0, m0, 0);
    store_stage(st, sm, 0);
    __syncthreads();

    for (int64_t c = 0; c < nstages; ++c) {
        const int buf = (int)(c & 1);
        if (c + 1 < nstages) load_stage(st, qw, qa, sw, sa, M, N, K, G, n0, m0, c + 1);
        const int64_t gleft = G - c * GC;
        const int ng = gleft >= GC ? GC : (int)gleft;
        for (int gi = 0; gi < ng; ++gi) {
            i32x4 A[4], B[4];
            f32x4 swv[4];
            float sav[4];
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) {
                const int row = wn * 64 + 16 * bi + rl;
                A[bi] = widen_nibbles(
                    *reinterpret_cast<const u32x2 *>(&sm.a[buf][row * ASTR + gi * 32 + 8 * ks]));
                swv[bi] = *reinterpret_cast<const f32x4 *>(&sm.sw[buf][gi][wn * 64 + 16 * bi + 4 * ks]);
            }
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int row = wm * 64 + 16 * bj + rl;
                B[bj] = widen_nibbles(
                    *reinterpret_cast<const u32x2 *>(&sm.b[buf][row * ASTR + gi * 32 + 8 * ks]));
                sav[bj] = sm.sa[buf][gi][wm * 64 + 16 * bj + rl];
            }
            i32x4 S[4][4];
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj)
                    S[bi][bj] = mfma_i8_16x16x64(A[bi], B[bj], i32x4{0, 0, 0, 0});
#pragma unroll
            for (int bi = 0; bi < 4; ++bi)
#pragma unroll
                for (int bj = 0; bj < 4; ++bj)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[bi][bj][j] = __builtin_fmaf((float)S[bi][bj][j], swv[bi][j] * sav[bj],
                                                        acc[bi][bj][j]);
        }
        if (c + 1 < nstages) store_stage(st, sm, buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: rank-r up-projection on the same tile (bf16 MFMA, the
    // fp32 xl1 split into a bf16 hi/lo pair), then bias, activation, store.
    if (r > 0) {
        const int lstr = r + 8;   // bf16 elements per LDS row of L2^T
        uint16_t *l2t = reinterpret_cast<uint16_t *>(&sm.a[0][0]);
        for (int q = tid; q < r * (BN / 8); q += NTHR) {
            const int i = q / (BN / 8);
            const int seg = (q - i * (BN / 8)) * 8;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (n0 + seg < N) v = *reinterpret_cast<const u32x4 *>(L2 + (int64_t)i * N + n0 + seg);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                l2t[(seg + 2 * e) * lstr + i] = (uint16_t)(v[e] & 0xFFFFu);
                l2t[(seg + 2 * e + 1) * lstr + i] = (uint16_t)(v[e] >> 16);
            }
        }
        __syncthreads();
        for (int c32 = 0; c32 < r; c32 += 32) {
            const int i0 = c32 + 8 * ks;
            const bool live = i0 < r;
            u32x4 AL[4];
#pragma unroll
            for (int bi = 0; bi < 4; ++bi) {
                const int row = wn * 64 + 16 * bi + rl;
                AL[bi] = live ? *reinterpret_cast<const u32x4 *>(&l2t[row * lstr + i0])
                              : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int bj = 0; bj < 4; ++bj) {
                const int64_t m = m0 + wm * 64 + 16 * bj + rl;
                const int64_t mc = m < M ? m : M - 1;
                u32x4 hi = u32x4{0u, 0u, 0u, 0u}, lo = u32x4{0u, 0u, 0u, 0u};
                if (live) {
                    const f32x4 *p = reinterpret_cast<const f32x4 *>(xl1 + mc * r + i0);
                    const f32x4 x0 = p[0], x1 = p[1];
                    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t h = pack_bf16x2(xs[2 * e], xs[2 * e + 1]);
                        hi[e] = h;
                        lo[e] = pack_bf16x2(xs[2 * e] - bf16_lo(h), xs[2 * e + 1] - bf16_hi(h));
                    }
                }
#pragma unroll
                for (int bi = 0; bi < 4; ++bi) {
                    acc[bi][bj] = mfma_bf16_16x16x32(AL[bi], hi, acc[bi][bj]);
                    acc[bi][bj] = mfma_bf16_16x16x32(AL[bi], lo, acc[bi][bj]);
                }
            }
        }
    }

#pragma unroll
    for (int bi = 0; bi < 4; ++bi) {
        const int64_t n = n0 + wn * 64 + 16 * bi + 4 * ks;
        if (n >= N) continue;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias) {
            const u32x2 b2 = *reinterpret_cast<const u32x2 *>(bias + n);
            bv[0] = bf16_lo(b2.x); bv[1] = bf16_hi(b2.x);
            bv[2] = bf16_lo(b2.y); bv[3] = bf16_hi(b2.y);
        }
#pragma unroll
        for (int bj = 0; bj < 4; ++bj) {
            const int64_t m = m0 + wm * 64 + 16 * bj + rl;
            if (m >= M) continue;
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x = acc[bi][bj][j] + bv[j];
                if (act == 1) x = 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
                o[j] = x;
            }
            u32x2 out;
            out.x = pack_bf16x2(o[0], o[1]);
            out.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<u32x2 *>(Y + m * N + n) = out;
        }
    }
}

// Test hook: per-group integer sums with the GEMM's operand widening and
// int8 MFMA; one wave per 16 x 16 block of (n, m), operands read from memory.
__global__ void __launch_bounds__(64)
group_sums_kernel(const uint8_t *__restrict__ qa, const uint8_t *__restrict__ qw, int64_t M,
                  int64_t N, int64_t K, int64_t m0, int64_t n0, int64_t tm, int64_t tn,
                  int32_t *__restrict__ S) {
    const int lane = threadIdx.x;
    const int rl = lane & 15, ks = lane >> 4;
    const int64_t nb = blockIdx.x, mb = blockIdx.y;
    const int64_t G = K / kGroup;
    int64_t n = n0 + nb * 16 + rl, m = m0 + mb * 16 + rl;
    if (n >= N) n = N - 1;
    if (m >= M) m = M - 1;
    for (int64_t g = 0; g < G; ++g) {
        const i32x4 A = widen_nibbles(*reinterpret_cast<const u32x2 *>(qw + n * (K / 2) + g * 32 + 8 * ks));
        const i32x4 B = widen_nibbles(*reinterpret_cast<const u32x2 *>(qa + m * (K / 2) + g * 32 + 8 * ks));
        const i32x4 D = mfma_i8_16x16x64(A, B, i32x4{0, 0, 0, 0});
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t nl = nb * 16 + 4 * ks + j;
            const int64_t ml = mb * 16 + rl;
            if (nl < tn && ml < tm) S[(ml * tn + nl) * G + g] = D[j] >> 8;
        }
    }
}

hipError_t launch_w4a4_gemm(const uint8_t *qa, const float *sa, const uint8_t *qw,
                            const float *sw, const float *xl1, const uint16_t *L2,
                            const uint16_t *bias, int act, int64_t M, int64_t N, int64_t K,
                            int r, uint16_t *Y, hipStream_t stream) {
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    w4a4_lr_gemm_kernel<<<(unsigned)tiles, NTHR, 0, stream>>>(qa, sa, qw, sw, xl1, L2, bias, act,
                                                              M, N, K, r, Y);
    return hipGetLastError();
}

hipError_t launch_group_sums(const uint8_t *qa, const uint8_t *qw, int64_t M, int64_t N,
                             int64_t K, int64_t m0, int64_t n0, int64_t tm, int64_t tn,
                             int32_t *S, hipStream_t stream) {
    dim3 grid((unsigned)((tn + 15) / 16), (unsigned)((tm + 15) / 16));
    group_sums_kernel<<<grid, 64, 0, stream>>>(qa, qw, M, N, K, m0, n0, tm, tn, S);
    return hipGetLastError();
}

}  // namespace svdq
