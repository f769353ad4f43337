// w4a4_tile.h -- the tile code of the SVDQuant W4A4 GEMM on gfx950 (internal;
// not part of the ABI): operand staging, the K loops (INT4 and MXFP4), the
// rank-r epilogue and the three output epilogues (plain [M, N] store; fused
// QKV; the MLP chain's next-layer activation step).  Included by the plain,
// fused-QKV, MLP-chain and MXFP4 GEMMs, each in its own translation unit, so
// that each kernel is scheduled on its own.
#pragma once

// The W4A4 GEMM of the SVDQuant layer on gfx950 with the
// rank-r up-projection, bias and GELU applied to the same output tile before
// its single bf16 store (the "Nunchaku engine design" section of the
// svdq-int4-flux.1-canny-dev model card fuses the up-projection with the
// 4-bit compute because both produce the same output).
//
// Output tiles are computed transposed, D[n][m] = Y[m][n]: the weight codes
// are the MFMA A operand and the activation codes the B operand, so that an
// output lane holds four consecutive n of one token row; the tile is staged
// in LDS in [m][n] order and leaves as 16-byte row segments.
//
// Per group of 64 along K and per 32 x 32 output block the wave issues
//   - one v_mfma_scale_f32_32x32x64_f8f6f4 on the codes as FP6 (the stored
//     code layout unfolds into E2M3 subnormals with four VALU ops per 16
//     codes, svdq_device.h; FP6 runs at twice the FP8 rate): S, the group's
//     exact integer sums, in fp32;
//   - half of a v_mfma_f32_32x32x1_2b_f32, which forms the scale products
//     P[n][m] = fl32(sw[n] sa[m]) of two 32 x 32 blocks at once (fp32
//     outer products, straight from the fp32 scales in LDS) in the same
//     output layout;
// and the VALU does only acc = fma(S, P, acc): the fp32 product of the two
// scales, then one fp32 fma per output and group.  The VALU is what bounds
// this kernel on this chip (one group of 64 MACs per output costs 1/64 of a
// 32x32x64 MFMA but a wave-wide VALU op), so the matrix unit takes every
// step it can: with the int8 instruction S came out as an integer and
// needed a convert per output and group, and forming P on the VALU, or its
// bf16 operands, would cost as much again.
//
// Data movement: packed 4-bit codes (rows in pairs, so that a stage of two
// rows is one 128-byte line) and raw fp32 scales go from global memory
// straight into a four-stage LDS ring with global_load_lds (no registers, no
// LDS write instructions), up to three stages ahead of the one being read; each wave reads its fragments with 16-byte LDS reads
// (XOR-swizzled rows, no bank conflicts) and turns the codes into FP6 in
// registers.
#include "svdq_device.h"
#include "svdq_internal.h"

#define SVDQ_MAX_RANK_DEV 128

namespace svdq {

namespace {

// Tiles are BT x BT outputs with BT = 64 WB, four waves in a 2 x 2 grid,
// each wave WB x WB blocks of 32 x 32.  WB = 2 (128 x 128 tiles) is the main
// shape; WB = 1 (64 x 64 quarter tiles) serves the tiles of a partial last
// round, so that they spread over four times as many workgroups.
constexpr int GC = 2;              // K groups per stage
constexpr int ROWP = GC * 32;      // packed bytes of one row per stage (4 x 16)
constexpr int PAIRP = 2 * ROWP;    // global bytes of one row pair per stage (row-pair codes)
constexpr int NBUF = 4;            // stages in the LDS ring
constexpr int NTHR = 256;          // 4 waves
constexpr int TILE = 128;          // the tile grid (a quarter tile is a quadrant of one)
constexpr int GROUP_M = 8;         // m-tiles per raster group (L2 reuse of weights)

template <int WB>
struct Cfg {
    static constexpr int BT = 64 * WB;
    static constexpr int NB = WB * WB;                 // blocks per wave
    // One stage in LDS: codes of the BT weight rows, then of the BT token
    // rows (64 bytes per row; 16-byte segment s of tile row R sits at slot
    // s ^ swz(R)), then the raw fp32 scales [row][group] of both.
    static constexpr int A_OFF = 0;
    static constexpr int B_OFF = A_OFF + BT * ROWP;
    static constexpr int SA_OFF = B_OFF + BT * ROWP;
    static constexpr int SB_OFF = SA_OFF + BT * GC * 4;
    static constexpr int STAGE = SB_OFF + BT * GC * 4;
    // global_load_lds instructions per wave per stage: WB code transfers per
    // operand, and one scale transfer per operand (WB = 2) or one in total
    static constexpr int LOADS = 2 * WB + (WB == 2 ? 2 : 1);
};

// Row swizzle of the 16-byte segments.  A 16-byte LDS read by 8 consecutive
// lanes (rows R..R+7 of one segment) or by 16 consecutive lanes touches 8
// (16) distinct 16-byte bank groups of 128 (256) bytes with this mapping.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

template <int WB>
struct __align__(16) Smem {
    union {
        uint8_t ring[NBUF][Cfg<WB>::STAGE];
        uint16_t l2t[Cfg<WB>::BT * (SVDQ_MAX_RANK_DEV + 8)];
    } u;
};
static_assert(sizeof(Smem<2>) <= 80 * 1024, "two workgroups per CU");

typedef __attribute__((address_space(3))) void lds_void;

// Linear tile index -> (tm, tn) on the 128 x 128 grid: GROUP_M m-tiles per
// raster group, so that consecutive tiles share weight rows in L2.
__device__ __forceinline__ void raster(int64_t id, int64_t nbm, int64_t nbn, int64_t &tm,
                                       int64_t &tn) {
    const int64_t per_group = (int64_t)GROUP_M * nbn;
    const int64_t grp = id / per_group;
    const int64_t first_m = grp * GROUP_M;
    const int64_t gsize = (nbm - first_m) < GROUP_M ? (nbm - first_m) : GROUP_M;
    const int64_t in_grp = id - grp * per_group;
    tm = first_m + in_grp % gsize;
    tn = in_grp / gsize;
}

// Loop-invariant plan of one wave's global -> LDS copies of a stage.  Code
// transfers: 1 KB each, lane l carries row 16 WB w + 16 i + l / 4 of its
// operand into LDS slot l % 4.  Scale transfers: 256 bytes, lane l carries
// row 32 j + l / 2, group l % 2 (WB = 2: block j = w of both operands;
// WB = 1: waves 0, 1 the weight rows, waves 2, 3 the token rows).  Rows past
// the matrix re-read its last row (never stored); a stage that holds only
// one group (odd group count) re-reads that group for the second.  Codes are
// in row pairs (code_offset); offsets are unsigned bytes from the tile's
// first pair, so each copy is a uniform (scalar) base plus a per-lane 32-bit
// offset.
template <int WB>
struct CopyPlan {
    uint32_t a_off[WB], b_off[WB];   // code transfers
    uint32_t a_tail[WB], b_tail[WB]; // same for a one-group stage
    uint32_t s_off[2], s_tail[2];    // scale transfers (weights, tokens)
    int wave;                        // wave index (uniform)
};

struct Operands {
    const uint8_t *qw0, *qa0;      // first row of the tile
    const uint8_t *sw0, *sa0;      // (scales, as bytes)
    int64_t sws, sas;              // INT4: bytes per stage of the stage-major scales (8 rows)
};

template <int WB>
__device__ __forceinline__ void issue_copies(uint8_t *st, const Operands &op, int c, int wave,
                                             const uint32_t (&ao)[WB], const uint32_t (&bo)[WB],
                                             const uint32_t (&so)[2]) {
    using C = Cfg<WB>;
    const uint8_t *qws = op.qw0 + c * PAIRP;
    const uint8_t *qas = op.qa0 + c * PAIRP;
#pragma unroll
    for (int i = 0; i < WB; ++i) {
        const int row = 16 * WB * wave + 16 * i;
        __builtin_amdgcn_global_load_lds(qws + ao[i], (lds_void *)(st + C::A_OFF + row * ROWP), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(qas + bo[i], (lds_void *)(st + C::B_OFF + row * ROWP), 16, 0, 0);
    }
    if (WB == 2) {
        __builtin_amdgcn_global_load_lds(op.sw0 + c * op.sws + so[0],
                                         (lds_void *)(st + C::SA_OFF + 32 * wave * GC * 4), 4, 0, 0);
        __builtin_amdgcn_global_load_lds(op.sa0 + c * op.sas + so[1],
                                         (lds_void *)(st + C::SB_OFF + 32 * wave * GC * 4), 4, 0, 0);
    } else if (wave < 2) {
        __builtin_amdgcn_global_load_lds(op.sw0 + c * op.sws + so[0],
                                         (lds_void *)(st + C::SA_OFF + 32 * wave * GC * 4), 4, 0, 0);
    } else {
        __builtin_amdgcn_global_load_lds(op.sa0 + c * op.sas + so[1],
                                         (lds_void *)(st + C::SB_OFF + 32 * (wave - 2) * GC * 4), 4, 0, 0);
    }
}

template <int WB>
__device__ __forceinline__ void issue_stage(uint8_t *st, const CopyPlan<WB> &cp,
                                            const Operands &op, int c, bool one_group) {
    if (one_group)
        issue_copies<WB>(st, op, c, cp.wave, cp.a_tail, cp.b_tail, cp.s_tail);
    else
        issue_copies<WB>(st, op, c, cp.wave, cp.a_off, cp.b_off, cp.s_off);
}

// Wait until at most `n` stages of this wave's copies are in flight (in the
// main loop the only outstanding vector-memory instructions are these) and
// this wave's LDS reads have returned (the barrier that follows releases the
// buffer they read for refilling).
template <int L>
__device__ __forceinline__ void wait_stages(int n) {
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
    constexpr int kNoExp = (0x7 << 4);
    constexpr int v1 = L, v2 = 2 * L, v3 = 3 * L;
    switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(kNoExp); break;
    case 1: __builtin_amdgcn_s_waitcnt((v1 & 0xF) | ((v1 >> 4) << 14) | kNoExp); break;
    case 2: __builtin_amdgcn_s_waitcnt((v2 & 0xF) | ((v2 >> 4) << 14) | kNoExp); break;
    default: __builtin_amdgcn_s_waitcnt((v3 & 0xF) | ((v3 >> 4) << 14) | kNoExp); break;
    }
}

// The wait inside the K loop before stage s + 1 is published: at most
// min(ns - 2 - s, 2) younger stages may stay in flight.  The steady state
// (two) is one uniform branch to a constant count; only the last stages take
// the general form (s_waitcnt takes an immediate, so a run-time count costs a
// branch tree).
template <int L>
__device__ __forceinline__ void wait_next_stage(int s, int ns) {
    if (__builtin_expect(s + 3 < ns, 1)) {
        constexpr int v2 = 2 * L;
        __builtin_amdgcn_s_waitcnt((v2 & 0xF) | ((v2 >> 4) << 14) | (0x7 << 4));
    } else {
        wait_stages<L>(s + 1 < ns ? ns - 2 - s : 0);
    }
}

// Workgroup barrier without a memory fence: the copies of the other stages
// stay in flight across it.  The clobber keeps the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// Loop-invariant LDS offsets of one lane's fragment reads.  Scales (the
// operands of the two-block outer product): WB = 2, per group: the weight
// scale of row l of the wave's 64 rows (a_scale), the token scale of column
// l (b_scale) and of column l ^ 32 (b_scale1) of its 64 columns; WB = 1, per
// stage: the scales of row / column l % 32 for group l / 32 of the stage.
struct ReadPlan {
    int a_code[GC], b_code[GC];    // block 0; block j is 32 j rows further
    int a_scale, b_scale, b_scale1;
};

template <int WB>
struct Raw {
    u32x4 a[WB], b[WB];
    float sw, sa0, sa1;
};
template <int WB>
struct Frags {
    i32x8 A[WB], B[WB];            // FP6 codes of the group, per block (6 of 8 words used)
    float PA, PB0, PB1;            // outer-product operands (weight, token scales)
};

// Group gi of a stage: the code fragments, and (WB = 2: every group; WB = 1:
// group 0, for both groups of the stage) the scale operands.
template <int WB>
__device__ __forceinline__ void read_raw(Raw<WB> &rw, const uint8_t *st, const ReadPlan &rp,
                                         int gi) {
#pragma unroll
    for (int blk = 0; blk < WB; ++blk) {
        rw.a[blk] = *reinterpret_cast<const u32x4 *>(st + rp.a_code[gi] + blk * 32 * ROWP);
        rw.b[blk] = *reinterpret_cast<const u32x4 *>(st + rp.b_code[gi] + blk * 32 * ROWP);
    }
    if (WB == 2) {
        rw.sw = *reinterpret_cast<const float *>(st + rp.a_scale + 4 * gi);
        rw.sa0 = *reinterpret_cast<const float *>(st + rp.b_scale + 4 * gi);
        rw.sa1 = *reinterpret_cast<const float *>(st + rp.b_scale1 + 4 * gi);
    } else if (gi == 0) {
        rw.sw = *reinterpret_cast<const float *>(st + rp.a_scale);
        rw.sa0 = *reinterpret_cast<const float *>(st + rp.b_scale);
    }
}

// FP6 codes and the outer-product operands.  A lane holds 32 codes of its
// row (the group's k half ks2), the same 32 k in both operands.  A token
// scale operand that is zero makes every product of its group zero, so the
// group adds exactly nothing: `keep` false zeroes a group past K (the empty
// half of an odd count's last stage, or a stage a k-split half runs only to
// pair its barriers).  WB = 1 builds the operands of both groups of a stage
// with its group 0 (lanes 32-63 carry group 1, kept if `keep1`).
template <int WB>
__device__ __forceinline__ void make_frags(Frags<WB> &f, const Raw<WB> &rw, bool keep,
                                           bool keep1 = true, bool scales = true) {
#pragma unroll
    for (int blk = 0; blk < WB; ++blk) {
        f.A[blk] = codes_to_fp6(rw.a[blk]);
        f.B[blk] = codes_to_fp6(rw.b[blk]);
    }
    if (WB == 2) {
        f.PA = rw.sw;
        f.PB0 = keep ? rw.sa0 : 0.0f;
        f.PB1 = keep ? rw.sa1 : 0.0f;
    } else if (scales) {
        const bool k = (threadIdx.x & 32) ? keep && keep1 : keep;
        f.PA = rw.sw;
        f.PB0 = k ? rw.sa0 : 0.0f;
    }
}

// The MFMA -> VALU pipeline of a wave.  The blocks of the two groups of a
// stage form one stream j = 0 .. 2 NB - 1 (group j / NB, result slot j & 1),
// in the order of the outer products: WB = 2 visits blocks (0,0), (1,1),
// (0,1), (1,0), so that elements 2q and 2q + 1 are the two blocks of one
// two-block product (rows l / 32 with columns l / 32, then with columns
// 1 - l / 32); WB = 1 has one block, and its product covers the two groups.
// The product of elements 2q, 2q + 1 goes out once element 2q - 1 has read
// the previous one; the code MFMA of element j goes out while the VALU
// accumulates element j - 1, so the matrix unit and the VALU work side by
// side, also across the group boundary.
struct Pipe {
    f32x16 S[2];
    f32x32 P;
};

template <int WB>
__device__ __forceinline__ constexpr int block_of(int j) {
    return WB == 1 ? 0 : (j % 4 == 0 ? 0 : j % 4 == 1 ? 3 : j % 4 == 2 ? 1 : 2);
}

template <int WB>
__device__ __forceinline__ void issue_block(Pipe &p, const Frags<WB> &f, int j) {
    const int t = block_of<WB>(j), bi = t / WB, bj = t % WB;
    p.S[j & 1] = mfma_codes_32x32x64(f.A[bi], f.B[bj]);
}

template <int WB>
__device__ __forceinline__ void issue_scales(Pipe &p, const Frags<WB> &f, int j) {
    p.P = mfma_f32_outer2(f.PA, (WB == 2 && (j % 4) == 2) ? f.PB1 : f.PB0);
}

// What the VALU does with the group sums of stream element jj (block jj % NB,
// group jj / NB of the stage, result slot jj & 1).  NoSink: the rescale,
// acc += S P (the product path).  TakeGroup: acc = S for the one group whose
// stage-relative index is `gsel` (the exact sums of one group captured from
// the production K loop, for the group-sum test hook); other groups leave
// acc as it is.
struct NoSink {
    static constexpr bool on = false;
    int gsel;
};
struct TakeGroup {
    static constexpr bool on = true;
    int gsel;   // the wanted group minus twice the current stage
};

template <int NB, class SK>
__device__ __forceinline__ void valu_block(f32x16 (&acc)[NB], const Pipe &p, int jj, const SK &sk) {
    constexpr int WB = NB == 4 ? 2 : 1;
    const int t = block_of<WB>(jj), k = jj & 1;
    f32x16 P;
#pragma unroll
    for (int i = 0; i < 16; ++i) P[i] = p.P[16 * k + i];
    if constexpr (SK::on) {
        // acc += S w with w = 1 for the wanted group and 0 for the others (acc
        // starts at zero, so it ends as that group's sums).  w is taken
        // through fma(P, 0, w), so that, as in the rescale, the VALU reads
        // the scale product as well as the sums and waits for both results
        // of the matrix unit.
        const float w = jj / NB == sk.gsel ? 1.0f : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc[t][i] = __builtin_fmaf(p.S[k][i], __builtin_fmaf(P[i], 0.0f, w), acc[t][i]);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = __builtin_fmaf(p.S[k][i], P[i], acc[t][i]);
    }
}

// Issue stream element j while the VALU finishes element j - 1: the code
// MFMA, the VALU work, and (even j with WB = 2) the next outer product after
// it, which overwrites the one element j - 1 has just read.  The empty asm
// pins the updated accumulator so later passes cannot sink the VALU work
// below the following MFMAs.
template <int WB, class SK>
__device__ __forceinline__ void pair(f32x16 (&acc)[WB * WB], Pipe &p, const Frags<WB> &f, int j,
                                     const SK &sk) {
    constexpr int NB = WB * WB;
    issue_block<WB>(p, f, j);
    valu_block<NB>(acc, p, j - 1, sk);
    asm volatile("" : "+v"(acc[block_of<WB>(j - 1)]));
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
    if (WB == 2 && (j & 1) == 0) {
        __builtin_amdgcn_sched_barrier(0);
        issue_scales<WB>(p, f, j);
    }
    __builtin_amdgcn_sched_barrier(0);
}

template <int WB, class SK>
__device__ __forceinline__ void group_first(f32x16 (&acc)[WB * WB], Pipe &p, const Frags<WB> &f,
                                            const SK &sk) {
    issue_block<WB>(p, f, 0);
    issue_scales<WB>(p, f, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 1; j < WB * WB; ++j) pair<WB>(acc, p, f, j, sk);
}
template <int WB, class SK>
__device__ __forceinline__ void group_second(f32x16 (&acc)[WB * WB], Pipe &p, const Frags<WB> &f,
                                             const SK &sk) {
#pragma unroll
    for (int j = WB * WB; j < 2 * WB * WB; ++j) pair<WB>(acc, p, f, j, sk);
}
template <int WB, class SK>
__device__ __forceinline__ void group_drain(f32x16 (&acc)[WB * WB], Pipe &p, const SK &sk) {
    constexpr int NB = WB * WB;
    valu_block<NB>(acc, p, 2 * NB - 1, sk);
    asm volatile("" : "+v"(acc[block_of<WB>(2 * NB - 1)]));
    __builtin_amdgcn_sched_barrier(0);
}

// The K loop.  The four ring buffers are separate restrict pointers so that
// the compiler can tell a read of one stage from the copies still landing in
// the others (otherwise every LDS read would wait for all copies).  ODD: the
// last real stage holds one group (an odd group count; a compile-time
// choice, so that an even count carries no per-stage selects for it).  SK:
// what the VALU does with the group sums (NoSink: the rescale; TakeGroup:
// capture the sums of group sink.gsel).  NULLS: the loop runs ns stages of
// which only the first nr are real (the halves of a k-split workgroup run
// the same number of stages, so that their barriers pair up); a stage past
// nr re-reads the last real one and adds nothing (its token scales are
// zero, so every fma adds S * 0).
// With NULLS the tail is a run-time choice (nodd), so that both halves of a
// k-split workgroup share one instance of the loop.
template <int WB, bool ODD, class SK = NoSink, bool NULLS = false>
__device__ __forceinline__ void k_loop(uint8_t *__restrict__ b0, uint8_t *__restrict__ b1,
                                       uint8_t *__restrict__ b2, uint8_t *__restrict__ b3,
                                       const CopyPlan<WB> &cp, const ReadPlan &rp,
                                       const Operands &op, int ns,
                                       f32x16 (&acc)[WB * WB], SK sink = SK{}, int nr = 0,
                                       bool nodd = false) {
    const bool odd = NULLS ? nodd : ODD;
    constexpr int L = Cfg<WB>::LOADS;
    // the stage whose data loop stage c copies, and whether that is the
    // one-group tail
    auto src = [&](int c) {
        if constexpr (NULLS) return c < nr ? c : nr - 1;
        else return c;
    };
    auto tail = [&](int c) {
        if constexpr (NULLS) return odd && src(c) == nr - 1;
        else return odd && c == ns - 1;
    };
    // prologue: stages 0..3 in flight, stage 0 visible, group 0 in registers
    issue_stage<WB>(b0, cp, op, src(0), tail(0));
    if (ns > 1) issue_stage<WB>(b1, cp, op, src(1), tail(1));
    if (ns > 2) issue_stage<WB>(b2, cp, op, src(2), tail(2));
    if (ns > 3) issue_stage<WB>(b3, cp, op, src(3), tail(3));
    wait_stages<L>(ns < 4 ? ns - 1 : 3);
    barrier();
    // the last real stage, whose second group is empty for an odd count
    const int last = NULLS ? nr - 1 : ns - 1;
    Raw<WB> raw;
    Frags<WB> f;
    read_raw<WB>(raw, b0, rp, 0);
    make_frags<WB>(f, raw, !NULLS || nr > 0, !(odd && last == 0));

    // Stage s: group 2s computes while group 2s + 1 is read; then stage
    // s + 1 is published and stage s's buffer (read by every wave before
    // the barrier) is refilled with stage s + 4; group 2s + 1 computes
    // while the first group of stage s + 1 is read.
    auto step = [&](int s, uint8_t *cur, uint8_t *nxt) {
        Pipe p;
        SK sk = sink;
        if constexpr (SK::on) sk.gsel = sink.gsel - 2 * s;
        read_raw<WB>(raw, cur, rp, 1);
        __builtin_amdgcn_sched_barrier(0);
        group_first<WB>(acc, p, f, sk);
        make_frags<WB>(f, raw, (!NULLS || s < nr) && !(odd && s == last), true, false);
        wait_next_stage<L>(s, ns);
        barrier();
        if (s + 4 < ns) issue_stage<WB>(cur, cp, op, src(s + 4), tail(s + 4));
        // (after the last stage this reads a stale, unused buffer: no branch,
        // so the fragments carry no merge of old and new values)
        read_raw<WB>(raw, nxt, rp, 0);
        __builtin_amdgcn_sched_barrier(0);
        group_second<WB>(acc, p, f, sk);
        make_frags<WB>(f, raw, !NULLS || s + 1 < nr, !(odd && s + 1 == last));
        group_drain<WB>(acc, p, sk);
    };
    for (int s = 0; s < ns; s += 4) {
        step(s, b0, b1);
        if (s + 1 >= ns) break;
        step(s + 1, b1, b2);
        if (s + 2 >= ns) break;
        step(s + 2, b2, b3);
        if (s + 3 >= ns) break;
        step(s + 3, b3, b0);
    }
}

// ---------------------------------------------------------------- MXFP4 K loop
// The 4-bit float variant: E2M1 codes (stored in row pairs, so that a code
// copy reads whole 128-byte lines: a stage of two rows) in the same LDS ring,
// swizzle and copy pattern; E8M0 scale bytes instead of fp32 group scales.  The matrix unit applies the block scales itself (one
// v_mfma_scale_f32_32x32x64_f8f6f4 per group of 64 and 32 x 32 block), so the
// VALU does no per-group work.  K % 128 == 0: every stage holds two full
// groups, i.e. four k blocks of 32.
//
// The scale bytes are block-major, [K/32][P] with the row count rounded up
// to P (a multiple of 16): a stage's bytes of a tile are four runs of BT
// consecutive bytes, fetched in a few whole cache lines (row-major bytes
// would cost one memory request per row and stage, as many as the codes).
// Scale copies: one 256-byte transfer per wave and stage, lane l carrying 4
// consecutive rows of one k block.  WB = 2: wave w copies operand w / 2
// (weights, tokens), k blocks 2 (w % 2) + l / 32, rows 4 (l % 32) ..;
// WB = 1: wave w copies operand w % 2, k block l / 16, rows 4 (l % 16) ..;
// waves 2, 3 repeat waves 0, 1 (identical bytes to identical addresses), so
// that every wave issues the same number of copies per stage, which the
// counted waits rely on.  In LDS a stage holds [k block][BT rows] bytes per
// operand at SA_OFF / SB_OFF.  Row groups past the padded rows re-read the
// last one (never stored).
template <int WB>
struct MxLoads { static constexpr int L = 2 * WB + 1; };

struct MxScaleSrc {
    const uint8_t *base;   // the wave's operand, k block 0, first row of the tile
    uint32_t stage;        // bytes per stage: 4 P
    uint32_t off;          // the lane's offset: k block * P + row
    int dst;               // LDS offset of the wave's transfer within a stage
};

template <int WB>
__device__ __forceinline__ void issue_stage_mx(uint8_t *st, const CopyPlan<WB> &cp,
                                               const Operands &op, const MxScaleSrc &ss, int c) {
    using C = Cfg<WB>;
    const uint8_t *qws = op.qw0 + c * PAIRP;
    const uint8_t *qas = op.qa0 + c * PAIRP;
    const int wave = cp.wave;
#pragma unroll
    for (int i = 0; i < WB; ++i) {
        const int row = 16 * WB * wave + 16 * i;
        __builtin_amdgcn_global_load_lds(qws + cp.a_off[i], (lds_void *)(st + C::A_OFF + row * ROWP), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(qas + cp.b_off[i], (lds_void *)(st + C::B_OFF + row * ROWP), 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(ss.base + (int64_t)c * ss.stage + ss.off, (lds_void *)(st + ss.dst), 4,
                                     0, 0);
}

// One group's operands of the lane's blocks: 16 code bytes and the k block's
// scale byte each.
template <int WB>
struct MxFrag {
    u32x4 a[WB], b[WB];
    uint32_t ea[WB], eb[WB];
};

// rp.a_scale / b_scale: LDS offset of the lane's k block 0 (of the group)
// byte of its block-0 row; k block q adds q BT, block j adds 32 j.
template <int WB>
__device__ __forceinline__ void read_mx(MxFrag<WB> &f, const uint8_t *st, const ReadPlan &rp,
                                        int gi) {
    constexpr int BT = Cfg<WB>::BT;
#pragma unroll
    for (int blk = 0; blk < WB; ++blk) {
        f.a[blk] = *reinterpret_cast<const u32x4 *>(st + rp.a_code[gi] + blk * 32 * ROWP);
        f.b[blk] = *reinterpret_cast<const u32x4 *>(st + rp.b_code[gi] + blk * 32 * ROWP);
        f.ea[blk] = st[rp.a_scale + 2 * gi * BT + 32 * blk];
        f.eb[blk] = st[rp.b_scale + 2 * gi * BT + 32 * blk];
    }
}

// One group on every block of the wave.
template <int WB>
__device__ __forceinline__ void group_mx(f32x16 (&acc)[WB * WB], const MxFrag<WB> &f) {
#pragma unroll
    for (int t = 0; t < WB * WB; ++t) {
        const int bi = t / WB, bj = t % WB;
        acc[t] = mfma_mxfp4_32x32x64(f.a[bi], f.ea[bi], f.b[bj], f.eb[bj], acc[t]);
    }
}

// Stage s: group 1 of the stage is read while group 0 computes; after the
// barrier the buffer is refilled with stage s + 4 and the next stage's first
// group is read while group 1 computes.
template <int WB>
__device__ __forceinline__ void k_loop_mx(uint8_t *__restrict__ b0, uint8_t *__restrict__ b1,
                                          uint8_t *__restrict__ b2, uint8_t *__restrict__ b3,
                                          const CopyPlan<WB> &cp, const ReadPlan &rp,
                                          const Operands &op, const MxScaleSrc &ss, int ns,
                                          f32x16 (&acc)[WB * WB]) {
    constexpr int L = MxLoads<WB>::L;
    issue_stage_mx<WB>(b0, cp, op, ss, 0);
    if (ns > 1) issue_stage_mx<WB>(b1, cp, op, ss, 1);
    if (ns > 2) issue_stage_mx<WB>(b2, cp, op, ss, 2);
    if (ns > 3) issue_stage_mx<WB>(b3, cp, op, ss, 3);
    wait_stages<L>(ns < 4 ? ns - 1 : 3);
    barrier();
    MxFrag<WB> f0, f1;
    read_mx<WB>(f0, b0, rp, 0);

    auto step = [&](int s, uint8_t *cur, uint8_t *nxt) {
        read_mx<WB>(f1, cur, rp, 1);
        __builtin_amdgcn_sched_barrier(0);
        group_mx<WB>(acc, f0);
        wait_next_stage<L>(s, ns);
        barrier();
        if (s + 4 < ns) issue_stage_mx<WB>(cur, cp, op, ss, s + 4);
        // (after the last stage this reads a stale, unused buffer)
        read_mx<WB>(f0, nxt, rp, 0);
        __builtin_amdgcn_sched_barrier(0);
        group_mx<WB>(acc, f1);
    };
    for (int s = 0; s < ns; s += 4) {
        step(s, b0, b1);
        if (s + 1 >= ns) break;
        step(s + 1, b1, b2);
        if (s + 2 >= ns) break;
        step(s + 2, b2, b3);
        if (s + 3 >= ns) break;
        step(s + 3, b3, b0);
    }
}

}  // namespace

namespace {

// Fused QKV epilogue of a 128 x 128 tile (the "Bringing Nunchaku 4-bit
// inference to Diffusers" blog, the fused_qkv_norm_rottary listing: Q, K and
// V from one projection, norm_q / norm_k, then the rotary embedding, in one
// operator).  The tile lies in one section of [Q | K | V] (H D % 128 == 0).
// For Q and K: per token and head, rho = sqrt(mean(x^2) + eps) over the head's
// D columns (D = 128: the whole tile width, the two column-half waves swap
// their partial sums through LDS and both add them in the same order; D = 64:
// the wave's own 64 columns), v = x gamma / rho, then each adjacent pair
// (2p, 2p + 1) -- two consecutive values of the same lane -- turns by the
// caller's (cos, sin) of position s = m mod S.  V is only re-laid out.  The
// results go to [B, H, S, D] through an LDS staging of the tile, as 16-byte
// writes of eight consecutive d.
// LDS use of the QKV epilogue besides the output staging: the per-wave
// (cos, sin) regrouping areas (4 waves x 64 tokens x QKV_TP floats, inside
// the L2^T region) and the D = 128 sum-of-squares exchange (past the output
// staging).
constexpr int QKV_TP = 34;                                  // floats per token row
constexpr int QKV_XS_OFF = 2 * 128 * (SVDQ_MAX_RANK_DEV + 8) * 2;
static_assert(4 * 64 * QKV_TP * 4 <= 128 * (SVDQ_MAX_RANK_DEV + 8) * 2, "regrouping fits");
static_assert(QKV_XS_OFF + 2 * 2 * 2 * 32 * 4 <= (int)sizeof(Smem<2>), "exchange fits");

template <int WB>
__device__ __forceinline__ void
qkv_epilogue(f32x16 (&acc)[WB * WB], const u32x2 (&bb)[WB][4], const QkvArgs &qk,
             Smem<WB> &sm, int64_t M, int64_t m0, int64_t n0, int wn, int wm, int r32,
             int ks2) {
    constexpr int NB = WB * WB;
    const int D = qk.D;
    const int64_t HD = (int64_t)qk.H * D;
    const int sec = (int)(n0 / HD);
    const int64_t nsec = n0 - sec * HD;        // section column of the tile's left edge
    const int64_t S = qk.S;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
        const int bi = t / WB;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x2 b2 = bb[bi][q];
            acc[t][4 * q + 0] += bf16_lo(b2.x);
            acc[t][4 * q + 1] += bf16_hi(b2.x);
            acc[t][4 * q + 2] += bf16_lo(b2.y);
            acc[t][4 * q + 3] += bf16_hi(b2.y);
        }
    }
    // The tile goes out through LDS (as the plain store): staged in [m][n]
    // order past the L2^T rows, then written as 16-byte segments of 8
    // consecutive d of one token and head, eight lanes per 128-byte line,
    // non-temporal as the plain store.
    constexpr int BT = 64 * WB;
    constexpr int OP = 2 * BT + 16;                          // staged row pitch, bytes
    uint8_t *ost = reinterpret_cast<uint8_t *>(&sm) + BT * (SVDQ_MAX_RANK_DEV + 8) * 2;
    static_assert(BT * (SVDQ_MAX_RANK_DEV + 8) * 2 + BT * OP <= (int)sizeof(Smem<WB>),
                  "QKV output staging fits in LDS");
    auto stage = [&](int bi, int bj, int q, u32x2 out) {
        const int ml = wm * 32 * WB + 32 * bj + r32;
        const int nl = wn * 32 * WB + 32 * bi + 8 * q + 4 * ks2;
        *reinterpret_cast<u32x2 *>(ost + ml * OP + 2 * nl) = out;
    };
    if (sec == 2) {
#pragma unroll
        for (int bi = 0; bi < WB; ++bi) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int bj = 0; bj < WB; ++bj) {
                    const int t = bi * WB + bj;
                    u32x2 out;
                    out.x = pack_bf16x2(acc[t][4 * q], acc[t][4 * q + 1]);
                    out.y = pack_bf16x2(acc[t][4 * q + 2], acc[t][4 * q + 3]);
                    stage(bi, bj, q, out);
                }
            }
        }
    } else if constexpr (WB == 2) {   // quarter tiles are only ever V tiles (a head needs the full tile width)
    // The wave's (cos, sin) rows: its 64 tokens (m0 + 64 wm + tt) and its 32
    // pairs, starting at pair pb of the head, one 128-byte line per token and
    // table.  They are fetched as whole lines (lane l: token 8 j + l / 8,
    // pairs 4 (l % 8) .. + 3) and regrouped through LDS, instead of 8-byte
    // gathers that touch 32 lines per instruction.  Positions past M stay in
    // the table (s = m mod S); their rows are never stored.
    const int lane = 32 * ks2 + r32;
    const int half = D / 2;
    const int pb = (int)(((nsec + wn * 32 * WB) % D) / 2);
    const int64_t tok0 = m0 + wm * 32 * WB;
    u32x4 tc[8], tsn[8];
    {
        int64_t sp = (tok0 + (lane >> 3)) % S;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t at = sp * half + pb + 4 * (lane & 7);
            tc[j] = *reinterpret_cast<const u32x4 *>(qk.cos_t + at);
            tsn[j] = *reinterpret_cast<const u32x4 *>(qk.sin_t + at);
            sp += 8;
            if (sp >= S) sp = S >= 8 ? sp - S : sp % S;
        }
    }
    // sum of squares of each token over this wave's columns (and the partner
    // lane l ^ 32, which holds the other half of every 8-column group)
    float ss[WB];
#pragma unroll
    for (int bj = 0; bj < WB; ++bj) {
        float a = 0.0f;
#pragma unroll
        for (int bi = 0; bi < WB; ++bi)
#pragma unroll
            for (int i = 0; i < 16; ++i) a = fmaf(acc[bi * WB + bj][i], acc[bi * WB + bj][i], a);
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a),
                                                        false, false);
        ss[bj] = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    }
    __syncthreads();   // every wave is past its reads of the L2^T staging
    if (D == 128) {
        // past the output staging: [wn][wm][bj][32]
        float *xs = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(&sm) + QKV_XS_OFF);
        if (ks2 == 0) {
#pragma unroll
            for (int bj = 0; bj < WB; ++bj) xs[((wn * 2 + wm) * WB + bj) * 32 + r32] = ss[bj];
        }
        __syncthreads();
#pragma unroll
        for (int bj = 0; bj < WB; ++bj)
            ss[bj] = xs[((0 * 2 + wm) * WB + bj) * 32 + r32] + xs[((1 * 2 + wm) * WB + bj) * 32 + r32];
    }
    float inv[WB];
#pragma unroll
    for (int bj = 0; bj < WB; ++bj) inv[bj] = 1.0f / sqrtf(ss[bj] / (float)D + qk.eps);
    // regroup: the wave's own [64 tokens][QKV_TP floats] area of the L2^T
    // region (free now); cos first, then sin in the same place (one wave's
    // LDS accesses complete in order)
    float *tb = reinterpret_cast<float *>(&sm) + (wn * 2 + wm) * 64 * QKV_TP;
    f32x2 cs[WB][4][WB], sn[WB][4][WB];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32x4 v = t == 0 ? tc[j] : tsn[j];
            float *w = tb + (8 * j + (lane >> 3)) * QKV_TP + 4 * (lane & 7);
            *reinterpret_cast<u32x2 *>(w) = u32x2{v.x, v.y};
            *reinterpret_cast<u32x2 *>(w + 2) = u32x2{v.z, v.w};
        }
#pragma unroll
        for (int bi = 0; bi < WB; ++bi)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int bj = 0; bj < WB; ++bj) {
                    const f32x2 r = *reinterpret_cast<const f32x2 *>(
                        tb + (32 * bj + r32) * QKV_TP + 16 * bi + 4 * q + 2 * ks2);
                    if (t == 0) cs[bi][q][bj] = r;
                    else sn[bi][q][bj] = r;
                }
    }
    const uint16_t *gam = sec == 0 ? qk.gq : qk.gk;
#pragma unroll
    for (int bi = 0; bi < WB; ++bi) {
        u32x2 g4[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t nl = nsec + wn * 32 * WB + 32 * bi + 8 * q + 4 * ks2;
            g4[q] = *reinterpret_cast<const u32x2 *>(gam + (nl - (nl / D) * D));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float gv[4] = {bf16_lo(g4[q].x), bf16_hi(g4[q].x), bf16_lo(g4[q].y),
                                 bf16_hi(g4[q].y)};
#pragma unroll
            for (int bj = 0; bj < WB; ++bj) {
                const int t = bi * WB + bj;
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = acc[t][4 * q + j] * inv[bj] * gv[j];
                const float o0 = v[0] * cs[bi][q][bj].x - v[1] * sn[bi][q][bj].x;
                const float o1 = v[0] * sn[bi][q][bj].x + v[1] * cs[bi][q][bj].x;
                const float o2 = v[2] * cs[bi][q][bj].y - v[3] * sn[bi][q][bj].y;
                const float o3 = v[2] * sn[bi][q][bj].y + v[3] * cs[bi][q][bj].y;
                u32x2 out;
                out.x = pack_bf16x2(o0, o1);
                out.y = pack_bf16x2(o2, o3);
                stage(bi, bj, q, out);
            }
        }
    }
    }
    __syncthreads();
    uint16_t *dst = sec == 0 ? qk.Q : (sec == 1 ? qk.K : qk.V);
    constexpr int CH = BT / 8;                               // 16-byte segments of a row
    const int tid = threadIdx.x;
#pragma unroll
    for (int idx = tid; idx < BT * CH; idx += NTHR) {
        const int row = idx / CH, ch = idx % CH;
        const int64_t m = m0 + row;
        if (m >= M) continue;
        const int64_t nl = nsec + 8 * ch;
        const int64_t h = nl / D, d = nl - h * D;
        const int64_t b = m / S, sp = m - b * S;
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(ost + row * OP + 16 * ch),
                                    reinterpret_cast<u32x4 *>(dst + ((b * qk.H + h) * S + sp) * D + d));
    }
}

// MLP chain epilogue of a 128 x 128 tile (the "Bringing Nunchaku 4-bit
// inference to Diffusers" blog credits fused GELU/MLP paths for native speed;
// the model card's Nunchaku engine design fuses a layer's down-projection
// with its quantizer because both read the same input).  The tile is the
// MLP-up output; instead of storing it, the epilogue runs the next layer's
// activation step on it, so the [M, N] intermediate never reaches memory:
//   h  = bf16(act(acc + bias))              (the value the plain GEMM stores)
//   x^ = fl32(h fl32(1 / lambda[n]))        (smoothing of the next layer)
//   per token and group of 64 columns -- exactly one wave's columns, the
//   lane's 32 values and those of its v_permlane32_swap partner --
//   s = max|x^| / 7, code = rint(x^ fl32(1/s)) (within [-7, 7]): the same
//   quantizer as K1, stored as the next layer's codes and scales;
//   the tile's share of x^ L1 over its 128 columns: x^ as a bf16 hi/lo pair
//   on v_mfma_f32_32x32x16_bf16 (rows: the lane's tokens, which is the
//   operand layout the tile already has) against L1^T staged in LDS; the two
//   column-half waves add their partials in LDS in a fixed order and the sum
//   goes to the partial buffer [N/128][M][rn], reduced in a fixed order later.
template <int WB>
__device__ __forceinline__ void
mlp_epilogue(f32x16 (&acc)[WB * WB], const u32x2 (&bb)[WB][4], const MlpArgs &ma, int act,
             Smem<WB> &sm, int64_t M, int64_t N, int64_t m0, int64_t n0, int wn, int wm,
             int r32, int ks2, int tid) {
    static_assert(WB == 2, "the MLP epilogue works on 128 x 128 tiles");
    static_assert(sizeof(Smem<2>) >= 69632 + 512, "room for 1/lambda past the staging");
    constexpr int NB = WB * WB;
    const int64_t nw = n0 + 64 * wn;   // the wave's group of 64 columns
    // fl32(1 / lambda) of the tile's 128 columns, once each, in LDS beyond
    // every region the rank-r staging and the steps below use
    float *linv = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(&sm.u) + 69632);
    if (tid < 128) linv[tid] = 1.0f / ma.lam[n0 + tid];
    __syncthreads();
    // bias, activation, bf16 rounding, smoothing (x^ kept in acc)
#pragma unroll
    for (int bi = 0; bi < WB; ++bi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 inv4 = *reinterpret_cast<const f32x4 *>(linv + 64 * wn + 32 * bi + 8 * q + 4 * ks2);
            const u32x2 b2 = bb[bi][q];
            const float bv[4] = {bf16_lo(b2.x), bf16_hi(b2.x), bf16_lo(b2.y), bf16_hi(b2.y)};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float inv = inv4[j];
#pragma unroll
                for (int bj = 0; bj < WB; ++bj) {
                    float x = acc[bi * WB + bj][4 * q + j] + bv[j];
                    if (act == 1) x = gelu_erf(x);
                    const float h = bf16_lo(pack_bf16x2(x, 0.0f));
                    acc[bi * WB + bj][4 * q + j] = h * inv;
                }
            }
        }
    }
    // quantize each token's group; store codes and scales
    const int64_t kb = N / 2, G = N / kGroup;
#pragma unroll
    for (int bj = 0; bj < WB; ++bj) {
        const int64_t m = m0 + wm * 32 * WB + 32 * bj + r32;
        float amax = 0.0f;
#pragma unroll
        for (int bi = 0; bi < WB; ++bi)
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(acc[bi * WB + bj][i]));
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax), __float_as_uint(amax),
                                                        false, false);
        amax = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
        const float s = amax / 7.0f;
        float inv = 0.0f;
        if (s != 0.0f) {
            const float t = 1.0f / s;
            inv = __builtin_isfinite(t) ? t : 0.0f;
        }
        // Column 32 bi + 8 q + 4 ks2 + j of the wave's group is code
        // e = 8 (q % 2) + 4 ks2 + j of stored block 2 bi + q / 2, i.e. field
        // 2 (4 ks2 + j) + q % 2 of that block's image: lane ks2 = 0 holds
        // fields 0-7 (image bits 0-47) of each of the group's four blocks,
        // its partner l ^ 32 fields 8-15 (bits 48-95).  Each lane converts
        // its half as fields 0-7 (one FP6 conversion per block pair bi) and
        // a ks2 = 1 lane moves it up by 48 bits; the partners then swap the
        // halves of the pair the other one stores (lane ks2 stores pair
        // bi = ks2: blocks 2 ks2, 2 ks2 + 1, 16 bytes) and OR them in.
        uint32_t img[WB][6];
#pragma unroll
        for (int bi = 0; bi < WB; ++bi) {
            f32x16v a = {}, b = {};
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // |y| < 7.5: no clamp
                    a[8 * u + j] = code_eighths(acc[bi * WB + bj][4 * (2 * u) + j] * inv);
                    b[8 * u + j] = code_eighths(acc[bi * WB + bj][4 * (2 * u + 1) + j] * inv);
                }
            const i32x6 im = fp6_images(a, b);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t w0 = (uint32_t)im[3 * u], w1 = (uint32_t)im[3 * u + 1];
                img[bi][3 * u] = ks2 ? 0u : w0;
                img[bi][3 * u + 1] = ks2 ? (w0 << 16) : w1;
                img[bi][3 * u + 2] = ks2 ? __builtin_amdgcn_alignbit(w1, w0, 16) : 0u;
            }
        }
        u32x4 words;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            uint32_t full[3];
#pragma unroll
            for (int w = 0; w < 3; ++w) {
                const uint32_t give = ks2 ? img[0][3 * u + w] : img[1][3 * u + w];
                const auto sw = __builtin_amdgcn_permlane32_swap(give, give, false, false);
                const uint32_t got = sw[0] ^ sw[1] ^ give;           // the partner's half
                full[w] = got | (ks2 ? img[1][3 * u + w] : img[0][3 * u + w]);
            }
            const u32x2 st = fold_image(full[0], full[1], full[2]);
            words[2 * u] = st.x;
            words[2 * u + 1] = st.y;
        }
        if (m < M) {
            *reinterpret_cast<u32x4 *>(ma.qa + code_offset(m, kb, nw / 2 + 16 * ks2)) = words;
            if (ks2 == 0) ma.sa[scale_index(m, nw / kGroup, M)] = s;
        }
    }
    if (ma.rn == 0) return;
    // the tile's partial down-projection
    constexpr int LS = 128 + 4;                     // bf16 per staged L1^T row
    uint16_t *l1t = reinterpret_cast<uint16_t *>(&sm.u);                       // [32][LS]
    float *pl = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(&sm.u) + 16384);  // [8][32][33]
    __syncthreads();   // every wave is past the rank-r staging of this tile
    {
        const int n = tid & 127, c = tid >> 7;      // column, 16-rank half
        uint32_t v[8];
        if (16 * c < ma.rn) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(ma.L1 + (n0 + n) * (int64_t)ma.rn + 16 * c);
            const u32x4 a = src[0], b = src[1];
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = 0u;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            l1t[(16 * c + 2 * e) * LS + n] = (uint16_t)(v[e] & 0xFFFFu);
            l1t[(16 * c + 2 * e + 1) * LS + n] = (uint16_t)(v[e] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int bj = 0; bj < WB; ++bj) {
        f32x16 P = f32x16{};
#pragma unroll
        for (int bi = 0; bi < WB; ++bi) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                // columns 16c + 4 ks2 + 0..3 and 16c + 8 + 4 ks2 + 0..3 of block bi
                float xs[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) xs[e] = acc[bi * WB + bj][8 * c + e];
                u32x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t h = pack_bf16x2(xs[2 * e], xs[2 * e + 1]);
                    hi[e] = h;
                    lo[e] = pack_bf16x2(xs[2 * e] - bf16_lo(h), xs[2 * e + 1] - bf16_hi(h));
                }
                const int nl = 64 * wn + 32 * bi + 16 * c + 4 * ks2;
                const u32x2 b0 = *reinterpret_cast<const u32x2 *>(&l1t[r32 * LS + nl]);
                const u32x2 b1 = *reinterpret_cast<const u32x2 *>(&l1t[r32 * LS + nl + 8]);
                const u32x4 B = u32x4{b0.x, b0.y, b1.x, b1.y};
                P = mfma_bf16_32x32x16(hi, B, P);
                P = mfma_bf16_32x32x16(lo, B, P);
            }
        }
        float *dst = pl + ((wn * 2 + wm) * 2 + bj) * (32 * 33);
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[(8 * (j / 4) + 4 * ks2 + (j % 4)) * 33 + r32] = P[j];
    }
    __syncthreads();
    {
        const int tl = tid >> 1, half = tid & 1;      // token of the tile, 16-rank half
        const int wmi = tl >> 6, bji = (tl >> 5) & 1, row = tl & 31;
        const int64_t m = m0 + tl;
        if (m < M && 16 * half < ma.rn) {
            const float *a = pl + ((0 * 2 + wmi) * 2 + bji) * (32 * 33) + row * 33 + 16 * half;
            const float *b = pl + ((1 * 2 + wmi) * 2 + bji) * (32 * 33) + row * 33 + 16 * half;
            f32x4 *out = reinterpret_cast<f32x4 *>(ma.part + ((n0 / 128) * M + m) * ma.rn + 16 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                out[e] = f32x4{a[4 * e] + b[4 * e], a[4 * e + 1] + b[4 * e + 1],
                               a[4 * e + 2] + b[4 * e + 2], a[4 * e + 3] + b[4 * e + 3]};
        }
    }
}

// Output epilogues of a tile.  EPI_SUMS is the group-sum test hook: the K
// loop captures the exact sums of one group (TakeGroup) and the tile stores
// them as int32 instead of running the rescale and the epilogue.
enum { EPI_STORE = 0, EPI_QKV = 1, EPI_MLP = 2, EPI_SUMS = 3 };

struct SumsArgs {
    int32_t *S;             // [btm, btn, G]: S[i][j][g] of rows bm0 + i, columns bn0 + j
    int64_t bm0, bn0, btm, btn;
    int G, g;               // group count, the group this launch captures
};

// One output tile: 128 x 128 (WB = 2) or 64 x 64 (WB = 1) at (m0, n0).
// EPI_STORE: bias, activation, the [M, N] bf16 store; EPI_QKV: the fused QKV
// epilogue (epi -> QkvArgs); EPI_MLP: the next layer's activation step
// (epi -> MlpArgs).  The last two need WB = 2.  MXF: the operands are MXFP4
// (sa, sw point to E8M0 bytes [rows, K / 32]; K % 128 == 0); otherwise INT4
// with fp32 group scales [rows, K / 64].
//
// KS = 2 (k-split tiles, 512 threads, EPI_STORE, INT4): two halves of four
// waves each run the K loop of the same tile over the two halves of K, each
// in its own LDS ring (sm is the first of two Smem<WB>): half 0 the first
// 2 ceil(G/4) groups (whole stages), half 1 the rest; both run as many
// stages (half 1 pads with null stages), so that their barriers pair up.
// Half 1 then hands its partial sums to half 0 through LDS, and half 0
// runs the epilogue on acc0 + acc1.  For grids that leave compute units
// idle: two waves per SIMD instead of one, with no partial sums in memory.
template <int WB, int EPI = EPI_STORE, bool MXF = false, int KS = 1>
__device__ __forceinline__ void
tile_body(const uint8_t *__restrict__ qa, const void *__restrict__ sa,
          const uint8_t *__restrict__ qw, const void *__restrict__ sw,
          const float *__restrict__ xl1, const uint16_t *__restrict__ L2,
          const uint16_t *__restrict__ bias, int act, int64_t M, int64_t N, int64_t K, int r,
          uint16_t *__restrict__ Y, Smem<WB> &sm, int64_t m0, int64_t n0,
          const void *epi = nullptr) {
    static_assert(KS == 1 || (KS == 2 && EPI == EPI_STORE && !MXF), "k-split: plain INT4 tiles");
    using C = Cfg<WB>;
    constexpr int BT = C::BT, NB = C::NB;
    const int tid = KS == 2 ? (int)(threadIdx.x & (NTHR - 1)) : (int)threadIdx.x;
    const int half = KS == 2 ? (int)(threadIdx.x / NTHR) : 0;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wn = wave >> 1, wm = wave & 1;
    const int r32 = lane & 31, ks2 = lane >> 5;
    const int G = (int)(K / kGroup);
    const int kb = (int)(K / 2);
    const int ns = (G + GC - 1) / GC;          // stages; only the last may hold one group
    const bool odd = (G & 1) != 0;
    const int nlast = (int)((N - n0 < BT ? N - n0 : BT) - 1);
    const int mlast = (int)((M - m0 < BT ? M - m0 : BT) - 1);
    // k-split: this half's loop length, real stages and first stage
    int ksl = ns, ksr = ns, ks0 = 0;
    if constexpr (KS == 2) {
        const int gh = 2 * ((G + 3) / 4);
        ksl = gh / 2;
        ks0 = half ? ksl : 0;
        ksr = half ? (G - gh + 1) / 2 : ksl;
    }

    Operands op;
    op.qw0 = qw + n0 * (int64_t)kb + ks0 * PAIRP;
    op.qa0 = qa + m0 * (int64_t)kb + ks0 * PAIRP;
    if constexpr (MXF) {                       // block-major bytes [K/32][P]: column offset
        op.sw0 = static_cast<const uint8_t *>(sw) + n0;
        op.sa0 = static_cast<const uint8_t *>(sa) + m0;
    } else {                                   // stage-major fp32 pairs: 8 R bytes per stage
        op.sws = 8 * N;
        op.sas = 8 * M;
        op.sw0 = reinterpret_cast<const uint8_t *>(static_cast<const float *>(sw) + 2 * n0) +
                 ks0 * op.sws;
        op.sa0 = reinterpret_cast<const uint8_t *>(static_cast<const float *>(sa) + 2 * m0) +
                 ks0 * op.sas;
    }

    CopyPlan<WB> cp;
    cp.wave = __builtin_amdgcn_readfirstlane(wave);
#pragma unroll
    for (int i = 0; i < WB; ++i) {
        const int row = 16 * WB * wave + 16 * i + (lane >> 2);
        const int seg = (lane & 3) ^ swz(row);     // global segment landing in this lane's slot
        const int ra = min(row, nlast), rb = min(row, mlast);
        // row pairs (code_offset): a stage's chunk of rows 2p, 2p + 1 in one
        // 128-byte line; a one-group last stage is 32 bytes per row
        cp.a_off[i] = (uint32_t)((ra >> 1) * 2 * kb + 64 * (ra & 1) + 16 * seg);
        cp.b_off[i] = (uint32_t)((rb >> 1) * 2 * kb + 64 * (rb & 1) + 16 * seg);
        cp.a_tail[i] = (uint32_t)((ra >> 1) * 2 * kb + 32 * (ra & 1) + 16 * (seg & 1));
        cp.b_tail[i] = (uint32_t)((rb >> 1) * 2 * kb + 32 * (rb & 1) + 16 * (seg & 1));
    }
    MxScaleSrc ss{};
    if constexpr (MXF) {
        const bool tok = WB == 2 ? (wave >> 1) != 0 : (wave & 1) != 0;
        const int64_t P = tok ? mx_scale_rows(M) : mx_scale_rows(N);
        const int64_t r0 = tok ? m0 : n0;
        // k block and first of the lane's 4 rows; clamped so that the dword
        // stays inside the padded rows
        const int blk = WB == 2 ? 2 * (wave & 1) + (lane >> 5) : (lane >> 4);
        const int row4 = WB == 2 ? 4 * (lane & 31) : 4 * (lane & 15);
        const int64_t rmax = P - 4 - r0;
        const int rowc = (int)(row4 < rmax ? row4 : rmax);
        ss.base = tok ? op.sa0 : op.sw0;
        ss.stage = (uint32_t)(4 * P);
        ss.off = (uint32_t)(blk * P + rowc);
        ss.dst = (tok ? C::SB_OFF : C::SA_OFF) + (WB == 2 ? 256 * (wave & 1) : 0);
    } else {
        const int blk = WB == 2 ? wave : (wave & 1);
        const int row = 32 * blk + (lane >> 1);
        const int g = lane & 1;
        // a stage's two scales of a row are adjacent (stage-major pairs); the
        // pad of an odd count's last stage is zero, so the tail reads it too
        cp.s_off[0] = (uint32_t)(4 * (2 * min(row, nlast) + g));
        cp.s_off[1] = (uint32_t)(4 * (2 * min(row, mlast) + g));
        cp.s_tail[0] = cp.s_off[0];
        cp.s_tail[1] = cp.s_off[1];
    }

    ReadPlan rp;
    {
        // rows wn * 32 WB + 32 blk + r32 (and wm ...) all share swz(r32)
        const int x = swz(r32);
#pragma unroll
        for (int gi = 0; gi < GC; ++gi) {
            const int slot = (2 * gi + ks2) ^ x;
            rp.a_code[gi] = C::A_OFF + (wn * 32 * WB + r32) * ROWP + 16 * slot;
            rp.b_code[gi] = C::B_OFF + (wm * 32 * WB + r32) * ROWP + 16 * slot;
        }
        if constexpr (MXF) {                      // [k block][row] bytes, k block ks2 of group 0
            rp.a_scale = C::SA_OFF + ks2 * BT + wn * 32 * WB + r32;
            rp.b_scale = C::SB_OFF + ks2 * BT + wm * 32 * WB + r32;
            rp.b_scale1 = rp.b_scale;
        } else if (WB == 2) {                     // [row][group] fp32, group 0
            rp.a_scale = C::SA_OFF + (wn * 64 + lane) * GC * 4;
            rp.b_scale = C::SB_OFF + (wm * 64 + lane) * GC * 4;
            rp.b_scale1 = C::SB_OFF + (wm * 64 + (lane ^ 32)) * GC * 4;
        } else {                                  // group ks2 of the stage
            rp.a_scale = C::SA_OFF + (wn * 32 + r32) * GC * 4 + 4 * ks2;
            rp.b_scale = C::SB_OFF + (wm * 32 + r32) * GC * 4 + 4 * ks2;
            rp.b_scale1 = rp.b_scale;
        }
    }

    f32x16 acc[NB];
#pragma unroll
    for (int t = 0; t < NB; ++t) acc[t] = f32x16{};

    if constexpr (EPI == EPI_SUMS) {
        // the production K loop, with the sums of group sg.g kept instead of
        // rescaled; stored as exact int32 for the requested block
        const SumsArgs &sg = *static_cast<const SumsArgs *>(epi);
        const TakeGroup tg{sg.g};
        if (odd)
            k_loop<WB, true, TakeGroup>(sm.u.ring[0], sm.u.ring[1], sm.u.ring[2], sm.u.ring[3],
                                        cp, rp, op, ns, acc, tg);
        else
            k_loop<WB, false, TakeGroup>(sm.u.ring[0], sm.u.ring[1], sm.u.ring[2], sm.u.ring[3],
                                         cp, rp, op, ns, acc, tg);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int bi = t / WB, bj = t % WB;
            const int64_t mi = m0 + wm * 32 * WB + 32 * bj + r32 - sg.bm0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int64_t ni = n0 + wn * 32 * WB + 32 * bi + 8 * (i / 4) + 4 * ks2 + (i % 4) - sg.bn0;
                if (mi >= 0 && mi < sg.btm && ni >= 0 && ni < sg.btn)
                    sg.S[(mi * sg.btn + ni) * sg.G + sg.g] = (int32_t)acc[t][i];
            }
        }
        return;
    } else if constexpr (MXF)
        k_loop_mx<WB>(sm.u.ring[0], sm.u.ring[1], sm.u.ring[2], sm.u.ring[3], cp, rp, op, ss, ns,
                      acc);
    else if constexpr (KS == 2) {
        Smem<WB> &rs = (&sm)[half];
        // only half 1 can end on the one-group stage
        k_loop<WB, false, NoSink, true>(rs.u.ring[0], rs.u.ring[1], rs.u.ring[2], rs.u.ring[3], cp,
                                        rp, op, ksl, acc, NoSink{}, ksr, half == 1 && odd);
    } else if (odd)
        k_loop<WB, true>(sm.u.ring[0], sm.u.ring[1], sm.u.ring[2], sm.u.ring[3], cp, rp, op, ns,
                         acc);
    else
        k_loop<WB, false>(sm.u.ring[0], sm.u.ring[1], sm.u.ring[2], sm.u.ring[3], cp, rp, op, ns,
                          acc);
    __syncthreads();
    if constexpr (KS == 2) {
        // Half 1 leaves its partial sums in its own (now idle) ring, as
        // [t][q][thread] 16-byte pieces (elements 4q .. 4q + 3 of block t;
        // conflict-free 16-byte accesses), and retires after the barriers that
        // pair with half 0's; half 0 adds them and runs the epilogue alone.
        // The barriers half 1 skips to must match the EPI_STORE epilogue
        // below one for one: the exchange, the L2^T staging (r > 0) and the
        // output staging.
        static_assert(NB * 16 * NTHR * 4 <= (int)sizeof(Smem<WB>), "partials fit in a ring");
        f32x4 *xch = reinterpret_cast<f32x4 *>(&(&sm)[1]);
        if (half == 1) {
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    xch[(t * 4 + q) * NTHR + tid] =
                        f32x4{acc[t][4 * q], acc[t][4 * q + 1], acc[t][4 * q + 2], acc[t][4 * q + 3]};
            __syncthreads();            // the exchange
            if (r > 0) __syncthreads(); // the L2^T staging
            __syncthreads();            // the output staging
            return;
        }
        __syncthreads();                // the exchange
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 o = xch[(t * 4 + q) * NTHR + tid];
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[t][4 * q + j] += o[j];
            }
    }

    // ---- epilogue: rank-r up-projection on the same tile (bf16 MFMA, the
    // fp32 xl1 split into a bf16 hi/lo pair), then bias, activation, store.
    // Its global loads go out together so that their latencies overlap: the
    // lane's xl1 for the first 32 ranks, the bias of its columns, and the L2
    // rows the workgroup stages as L2^T in LDS.
    f32x4 xp[WB][2][2];                        // [bj][16-rank chunk][half]
    if (r > 0) {
#pragma unroll
        for (int bj = 0; bj < WB; ++bj) {
            const int64_t m = m0 + wm * 32 * WB + 32 * bj + r32;
            const int64_t mc = m < M ? m : M - 1;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                if (16 * c < r) {
                    const f32x4 *p = reinterpret_cast<const f32x4 *>(xl1 + mc * r + 16 * c + 8 * ks2);
                    xp[bj][c][0] = p[0];
                    xp[bj][c][1] = p[1];
                }
            }
        }
    }
    u32x2 bb[WB][4];
#pragma unroll
    for (int bi = 0; bi < WB; ++bi) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + wn * 32 * WB + 32 * bi + 8 * q + 4 * ks2;
            bb[bi][q] = (bias && n < N) ? *reinterpret_cast<const u32x2 *>(bias + n) : u32x2{0u, 0u};
        }
    }
    if (r > 0) {
        const int lstr = r + 8;   // bf16 elements per LDS row of L2^T
        uint16_t *l2t = sm.u.l2t;
        // Thread q stages rank rows [8 c, 8 c + 8) of column n = q % BT as one
        // 16-byte row segment of L2^T (consecutive lanes: consecutive n, so
        // both the global reads and the LDS writes are conflict-free).
        for (int q = tid; q < r * (BT / 8); q += NTHR) {
            const int n = q % BT;
            const int c = q / BT;
            uint32_t v[4] = {0u, 0u, 0u, 0u};
            if (n0 + n < N) {
                const uint16_t *src = L2 + (int64_t)(8 * c) * N + n0 + n;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = (uint32_t)src[(2 * e) * N] | ((uint32_t)src[(2 * e + 1) * N] << 16);
            }
            *reinterpret_cast<u32x4 *>(&l2t[n * lstr + 8 * c]) = u32x4{v[0], v[1], v[2], v[3]};
        }
        __syncthreads();
        // 16 ranks: L2^T rows from LDS (A), xl1 hi/lo of the lane's rows (B).
        auto chunk = [&](int c16, const f32x4 (&x)[WB][2]) {
            const int i0 = c16 + 8 * ks2;
            u32x4 AL[WB];
#pragma unroll
            for (int bi = 0; bi < WB; ++bi) {
                const int row = wn * 32 * WB + 32 * bi + r32;
                AL[bi] = *reinterpret_cast<const u32x4 *>(&l2t[row * lstr + i0]);
            }
#pragma unroll
            for (int bj = 0; bj < WB; ++bj) {
                const float xs[8] = {x[bj][0].x, x[bj][0].y, x[bj][0].z, x[bj][0].w,
                                     x[bj][1].x, x[bj][1].y, x[bj][1].z, x[bj][1].w};
                u32x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t h = pack_bf16x2(xs[2 * e], xs[2 * e + 1]);
                    hi[e] = h;
                    lo[e] = pack_bf16x2(xs[2 * e] - bf16_lo(h), xs[2 * e + 1] - bf16_hi(h));
                }
#pragma unroll
                for (int bi = 0; bi < WB; ++bi) {
                    acc[bi * WB + bj] = mfma_bf16_32x32x16(AL[bi], hi, acc[bi * WB + bj]);
                    acc[bi * WB + bj] = mfma_bf16_32x32x16(AL[bi], lo, acc[bi * WB + bj]);
                }
            }
        };
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            if (16 * c < r) {
                f32x4 x[WB][2];
#pragma unroll
                for (int bj = 0; bj < WB; ++bj) {
                    x[bj][0] = xp[bj][c][0];
                    x[bj][1] = xp[bj][c][1];
                }
                chunk(16 * c, x);
            }
        }
        for (int c16 = 32; c16 < r; c16 += 16) {
            f32x4 x[WB][2];
#pragma unroll
            for (int bj = 0; bj < WB; ++bj) {
                const int64_t m = m0 + wm * 32 * WB + 32 * bj + r32;
                const int64_t mc = m < M ? m : M - 1;
                const f32x4 *p = reinterpret_cast<const f32x4 *>(xl1 + mc * r + c16 + 8 * ks2);
                x[bj][0] = p[0];
                x[bj][1] = p[1];
            }
            chunk(c16, x);
        }
    }

    if constexpr (EPI == EPI_QKV) {
        qkv_epilogue<WB>(acc, bb, *static_cast<const QkvArgs *>(epi), sm, M, m0, n0, wn, wm, r32,
                         ks2);
        return;
    }
    if constexpr (EPI == EPI_MLP) {
        mlp_epilogue<WB>(acc, bb, *static_cast<const MlpArgs *>(epi), act, sm, M, N, m0, n0, wn,
                         wm, r32, ks2, tid);
        return;
    }
    // The tile goes out through LDS: staged in [m][n] order, then written as
    // 16-byte row segments, eight lanes per 128-byte line (a direct store
    // from the transposed tile would write 8 bytes into each of 32 rows per
    // instruction).  The stores are non-temporal: the output is written once
    // and not read here, so it should not displace from L2 the operands that
    // the XCD's other tiles still read.  The staging area lies past the L2^T rows that other
    // waves may still be reading for the rank-r step.
    // Block (bi, bj); element i of the lane is n = base + 8 (i / 4) +
    // 4 (lane / 32) + i % 4, m = base + lane % 32.
    constexpr int OP = 2 * BT + 16;                          // staged row pitch, bytes
    constexpr int OUT_OFF = BT * (SVDQ_MAX_RANK_DEV + 8) * 2;
    static_assert(OUT_OFF + BT * OP <= (int)sizeof(Smem<WB>), "output staging fits in LDS");
    uint8_t *ost = reinterpret_cast<uint8_t *>(&sm) + OUT_OFF;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
        const int bi = t / WB, bj = t % WB;
        const int ml = wm * 32 * WB + 32 * bj + r32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int nl = wn * 32 * WB + 32 * bi + 8 * q + 4 * ks2;
            const u32x2 b2 = bb[bi][q];
            const float bv[4] = {bf16_lo(b2.x), bf16_hi(b2.x), bf16_lo(b2.y), bf16_hi(b2.y)};
            float o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float x = acc[t][4 * q + j] + bv[j];
                if (act == 1) x = gelu_erf(x);
                o[j] = x;
            }
            u32x2 out;
            out.x = pack_bf16x2(o[0], o[1]);
            out.y = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<u32x2 *>(ost + ml * OP + 2 * nl) = out;
        }
    }
    __syncthreads();
    constexpr int CH = BT / 8;                               // 16-byte segments of a row
#pragma unroll
    for (int idx = tid; idx < BT * CH; idx += NTHR) {
        const int row = idx / CH, ch = idx % CH;
        const int64_t m = m0 + row, n = n0 + 8 * ch;
        if (m < M && n < N)
            __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(ost + row * OP + 16 * ch),
                                        reinterpret_cast<u32x4 *>(Y + m * N + n));
    }
}

}  // namespace

}  // namespace svdq
