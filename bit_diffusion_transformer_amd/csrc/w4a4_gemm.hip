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
//
// Per group of 64 along K and per 16 x 16 output block, the wave issues
//   - one v_mfma_i32_16x16x64_i8 on the widened codes: S, exact int32;
//   - one v_mfma_f32_16x16x16_bf16 that forms the scale products
//     P[n][m] = sw[n] sa[m] as an outer product of bf16 hi/lo pairs
//     ((sw_hi + sw_lo)(sa_hi + sa_lo), exact bf16 products, fp32 sums,
//     ~2^-16 relative to the fp32 product) in the same output layout;
// and the VALU does only acc = fma(float(S), P, acc).  The rescale is the
// VALU-bound part of the layer on this chip (one group of 64 MACs per
// output against 3 VALU ops when the scale product is also formed on the
// VALU), so moving the product onto the matrix unit, which has slack, leaves
// two VALU ops per output and group.
#include "svdq_device.h"
#include "svdq_internal.h"

#define SVDQ_MAX_RANK_DEV 128

namespace svdq {

namespace {

constexpr int BN = 128;            // tile rows in n (weights)
constexpr int BM = 128;            // tile cols in m (tokens)
constexpr int GC = 2;              // K groups per LDS stage
constexpr int ROWP = GC * 32;      // packed bytes of one row per stage
constexpr int ASTR = ROWP + 8;     // LDS row stride: 72 B = 18 banks, so the 16
                                   // rows read by one 16-lane phase hit distinct banks
constexpr int NBUF = 3;            // LDS stages in flight
constexpr int NTHR = 256;          // 4 waves, 2 (n) x 2 (m), 64 x 64 each
constexpr int GROUP_M = 8;         // m-tiles per raster group (L2 reuse of weights)

// LDS.  Codes stay packed (4 bit) in LDS and are widened to int8 in
// registers by each wave.  Three stage buffers rotate: one being computed,
// one already published (the next group's fragments are read from it while
// the current group computes), one being filled from registers.
// Scale operands: per (group, row) one 8-byte bf16 quadruple, weights as
// (hi, hi, lo, lo), activations as (hi, lo, hi, lo); lanes of k-slots 1..3
// read the activation side from `zero`, so only k-slot 0 contributes.
struct __align__(16) Smem {
    union {
        struct {
            uint8_t a[NBUF][BN * ASTR];
            uint8_t b[NBUF][BM * ASTR];
        } t;
        uint16_t l2t[BN * (SVDQ_MAX_RANK_DEV + 8)];
    } u;
    u32x2 swop[NBUF][GC][BN];
    u32x2 saop[NBUF][GC][BM];
    u32x2 zero[64];
};
static_assert(sizeof(Smem) <= 80 * 1024, "two workgroups per CU");

// Per-thread, loop-invariant offsets of the global -> LDS copy.
struct CopyPlan {
    int voff[2];        // byte offsets of this thread's two 16-byte pieces (rows clamped)
    int voff_tail[2];   // same for a stage holding one group: the second group re-reads the first
    int soff;           // element offset of this thread's scale row (times G)
    int lds_off[2];     // LDS byte offsets (row * ASTR + seg) of the two pieces
};

struct StageRegs {
    u32x4 a[2];
    u32x4 b[2];
    float s[GC];
};

// Global -> registers for stage c; every address is in bounds (see CopyPlan).
__device__ __forceinline__ void load_stage(StageRegs &st, const CopyPlan &cp,
                                           const uint8_t *__restrict__ qw0,
                                           const uint8_t *__restrict__ qa0,
                                           const float *__restrict__ s0, int G, int c,
                                           bool partial) {
    const uint8_t *qws = qw0 + c * ROWP;
    const uint8_t *qas = qa0 + c * ROWP;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int off = partial ? cp.voff_tail[i] : cp.voff[i];
        st.a[i] = *reinterpret_cast<const u32x4 *>(qws + off);
        st.b[i] = *reinterpret_cast<const u32x4 *>(qas + off);
    }
    const float *ss = s0 + c * GC;
    st.s[0] = ss[cp.soff];
    st.s[1] = partial ? st.s[0] : ss[cp.soff + 1];
    (void)G;
}

// Registers -> LDS buffer `buf` for a stage with `gvalid` (1 or 2) groups;
// the scales of a missing group are zero, so that group adds exactly zero.
__device__ __forceinline__ void store_stage(const StageRegs &st, const CopyPlan &cp, Smem &sm,
                                            int buf, int gvalid) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        u32x2 *pa = reinterpret_cast<u32x2 *>(&sm.u.t.a[buf][cp.lds_off[i]]);
        u32x2 *pb = reinterpret_cast<u32x2 *>(&sm.u.t.b[buf][cp.lds_off[i]]);
        pa[0] = u32x2{st.a[i].x, st.a[i].y};
        pa[1] = u32x2{st.a[i].z, st.a[i].w};
        pb[0] = u32x2{st.b[i].x, st.b[i].y};
        pb[1] = u32x2{st.b[i].z, st.b[i].w};
    }
    // The weight scale carries the 2^-8 that undoes the x16 of both widened
    // operands (a power-of-two scaling, exact).
    if (tid < BN) {
#pragma unroll
        for (int gi = 0; gi < GC; ++gi) {
            const float v = gi < gvalid ? st.s[gi] * 0.00390625f : 0.0f;
            const uint32_t h = pack_bf16x2(v, v);
            const uint32_t l = pack_bf16x2(v - bf16_lo(h), v - bf16_lo(h));
            sm.swop[buf][gi][tid] = u32x2{h, l};
        }
    } else {
#pragma unroll
        for (int gi = 0; gi < GC; ++gi) {
            const float v = gi < gvalid ? st.s[gi] : 0.0f;
            const uint32_t h = pack_bf16x2(v, 0.0f);
            const uint32_t hl = pack_bf16x2(v, v - bf16_lo(h));
            sm.saop[buf][gi][tid - BN] = u32x2{hl, hl};
        }
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

// Fragments of one group for the wave's 64 x 64 tile: widened codes of the
// four 16-row blocks of A (weights) and B (tokens), and the scale operands.
struct Frags {
    i32x4 A[4], B[4];
    u32x2 AS[4], BS[4];
};

// Per-lane, loop-invariant LDS offsets of the fragment reads.
struct ReadPlan {
    int a_off, b_off;     // byte offsets into sm.u.t.a[0] / .b[0]
    int as_off;           // element offset into sm.swop[0][0]
    int bs_off, bs_step;  // element offset into sm.saop (or the zero row), and 1 / 0
};

__device__ __forceinline__ void load_frags(Frags &f, const Smem &sm, const ReadPlan &rp,
                                           int buf, int gi) {
    const uint8_t *abase = &sm.u.t.a[buf][rp.a_off + gi * 32];
    const uint8_t *bbase = &sm.u.t.b[buf][rp.b_off + gi * 32];
    const u32x2 *asc = &sm.swop[buf][gi][rp.as_off];
    // k-slot 0 lanes read the activation scale operands, the others a zero row
    const u32x2 *bsc = &sm.saop[0][0][0] + rp.bs_off + rp.bs_step * ((buf * GC + gi) * BM);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.A[i] = widen_nibbles(*reinterpret_cast<const u32x2 *>(abase + i * 16 * ASTR));
        f.B[i] = widen_nibbles(*reinterpret_cast<const u32x2 *>(bbase + i * 16 * ASTR));
        f.AS[i] = asc[16 * i];
        f.BS[i] = bsc[16 * i];
    }
}

// One group for the wave's 16 blocks: the MFMAs of block t + 2 are issued
// before the VALU converts and accumulates block t, so the matrix unit and
// the VALU overlap within the wave.
__device__ __forceinline__ void group_compute(f32x4 (&acc)[4][4], const Frags &f) {
    i32x4 S[3];
    f32x4 P[3];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        S[t] = mfma_i8_16x16x64(f.A[t >> 2], f.B[t & 3], i32x4{0, 0, 0, 0});
        P[t] = mfma_bf16_16x16x16(f.AS[t >> 2], f.BS[t & 3], f32x4{0.f, 0.f, 0.f, 0.f});
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
        const int bi = t >> 2, bj = t & 3;
        if (t + 2 < 16) {
            const int u = t + 2;
            S[u % 3] = mfma_i8_16x16x64(f.A[u >> 2], f.B[u & 3], i32x4{0, 0, 0, 0});
            P[u % 3] = mfma_bf16_16x16x16(f.AS[u >> 2], f.BS[u & 3], f32x4{0.f, 0.f, 0.f, 0.f});
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[bi][bj][j] = __builtin_fmaf((float)S[t % 3][j], P[t % 3][j], acc[bi][bj][j]);
        // Keep the issue order (at most three blocks of results live): the
        // empty asm pins the updated accumulator to this point so later
        // passes cannot sink the VALU work below the following MFMAs.
        asm volatile("" : "+v"(acc[bi][bj]));
        __builtin_amdgcn_sched_barrier(0);
    }
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
    const int G = (int)(K / kGroup);
    const int kb = (int)(K / 2);
    const int ns = (G + GC - 1) / GC;          // stages; only the last may hold one group
    const int glast = G - (ns - 1) * GC;       // groups in the last stage (1 or 2)
    const int nlast = (int)((N - n0 < BN ? N - n0 : BN) - 1);
    const int mlast = (int)((M - m0 < BM ? M - m0 : BM) - 1);

    if (tid < 64) sm.zero[tid] = u32x2{0u, 0u};

    // Loop-invariant offsets.
    CopyPlan cp;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = tid + NTHR * i;
        const int row = q >> 2;
        const int part = q & 3;
        const int seg = part * 16;
        // the weight and token tiles share the same per-thread layout; rows
        // past the end are clamped (weights to nlast, tokens to mlast) by
        // using the larger tile bound below for both and clamping each
        cp.lds_off[i] = row * ASTR + seg;
        cp.voff[i] = seg;               // row part added below per operand
        cp.voff_tail[i] = part >= 2 ? seg - 32 : seg;
    }
    // Operand base pointers at the tile's first row; each thread's row offset
    // is folded into per-operand offsets (rows clamped separately).
    const int q0 = tid, q1 = tid + NTHR;
    const int rowa0 = min(q0 >> 2, nlast), rowa1 = min(q1 >> 2, nlast);
    const int rowb0 = min(q0 >> 2, mlast), rowb1 = min(q1 >> 2, mlast);
    CopyPlan cpa = cp, cpb = cp;
    cpa.voff[0] += rowa0 * kb; cpa.voff[1] += rowa1 * kb;
    cpa.voff_tail[0] += rowa0 * kb; cpa.voff_tail[1] += rowa1 * kb;
    cpb.voff[0] += rowb0 * kb; cpb.voff[1] += rowb1 * kb;
    cpb.voff_tail[0] += rowb0 * kb; cpb.voff_tail[1] += rowb1 * kb;
    const bool is_w = tid < BN;
    cp.soff = (is_w ? min(tid, nlast) : min(tid - BN, mlast)) * G;
    const float *s0 = is_w ? sw + n0 * (int64_t)G : sa + m0 * (int64_t)G;
    const uint8_t *qw0 = qw + n0 * (int64_t)kb;
    const uint8_t *qa0 = qa + m0 * (int64_t)kb;

    ReadPlan rp;
    rp.a_off = (wn * 64 + rl) * ASTR + 8 * ks;
    rp.b_off = (wm * 64 + rl) * ASTR + 8 * ks;
    rp.as_off = wn * 64 + rl;
    if (ks == 0) {
        rp.bs_off = wm * 64 + rl;
        rp.bs_step = 1;
    } else {
        rp.bs_off = (int)(&sm.zero[rl] - &sm.saop[0][0][0]);
        rp.bs_step = 0;
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Loads for stage c go through registers `st`: A rows use cpa, B rows cpb.
    StageRegs st;
    auto load = [&](int c) {
        const bool partial = (c == ns - 1) && glast < GC;
        StageRegs t;
        const uint8_t *qws = qw0 + c * ROWP;
        const uint8_t *qas = qa0 + c * ROWP;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            t.a[i] = *reinterpret_cast<const u32x4 *>(qws + (partial ? cpa.voff_tail[i] : cpa.voff[i]));
            t.b[i] = *reinterpret_cast<const u32x4 *>(qas + (partial ? cpb.voff_tail[i] : cpb.voff[i]));
        }
        const float *ss = s0 + c * GC;
        t.s[0] = ss[cp.soff];
        t.s[1] = partial ? t.s[0] : ss[cp.soff + 1];
        st = t;
    };
    auto store = [&](int c) {
        const int gvalid = c == ns - 1 ? glast : GC;
        store_stage(st, cp, sm, c % NBUF, gvalid);
    };

    // Prologue: stages 0 and 1 in LDS, stage 2 in flight, group 0 in registers.
    load(0);
    store(0);
    if (ns > 1) {
        load(1);
        store(1);
    }
    if (ns > 2) load(2);
    __syncthreads();
    Frags f0, f1;
    load_frags(f0, sm, rp, 0, 0);

    for (int s = 0; s < ns; ++s) {
        const int b = s % NBUF;
        // group 2s (f0) computes while group 2s + 1 is read from LDS
        load_frags(f1, sm, rp, b, 1);
        __builtin_amdgcn_sched_barrier(0);
        group_compute(acc, f0);
        __builtin_amdgcn_sched_barrier(0);
        // stage s + 2 -> LDS (its global loads were issued a stage ago), then
        // publish it; buffer (s + 2) % 3 was last read before the previous barrier
        if (s + 2 < ns) store(s + 2);
        __syncthreads();
        if (s + 3 < ns) load(s + 3);
        // group 2s + 1 (f1) computes while group 2s + 2 is read from LDS
        if (s + 1 < ns) load_frags(f0, sm, rp, (s + 1) % NBUF, 0);
        __builtin_amdgcn_sched_barrier(0);
        group_compute(acc, f1);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();

    // ---- epilogue: rank-r up-projection on the same tile (bf16 MFMA, the
    // fp32 xl1 split into a bf16 hi/lo pair), then bias, activation, store.
    if (r > 0) {
        const int lstr = r + 8;   // bf16 elements per LDS row of L2^T
        uint16_t *l2t = sm.u.l2t;
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
