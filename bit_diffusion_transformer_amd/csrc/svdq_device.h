// svdq_device.h -- device helpers shared by the gfx950 kernels of the
// SVDQuant W4A4 + low-rank linear layer (internal; not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

constexpr int kGroup = 64;   // quantization group along K

typedef int      i32x4 __attribute__((ext_vector_type(4)));
typedef float    f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16   bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16   bf16x2 __attribute__((ext_vector_type(2)));
typedef float    f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t d) { return __uint_as_float(d & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

// ---------------------------------------------------------------- MFMA

// 16x16 output tile, K = 64 int8 per call.  Lane l supplies, for row/column
// l % 16, 16 int8 of k-slot l / 16; the output lane l holds rows
// 4*(l/16) + j, j = 0..3, of column l % 16.
__device__ __forceinline__ i32x4 mfma_i8_16x16x64(i32x4 a, i32x4 b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// 16x16 output tile, K = 32 bf16 per call (8 per lane), fp32 accumulate; the
// output layout is the same as the int8 instruction's.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 16x16 output tile, K = 16 bf16 per call (4 per lane: k-slot l / 16 holds
// k = 4 (l / 16) .. + 3), fp32 accumulate; same output layout as above.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                     __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef float f32x32 __attribute__((ext_vector_type(32)));

// Two 32x32 fp32 outer products in one instruction (v_mfma_f32_32x32x1_2b_f32,
// K = 1, two blocks): lane l supplies a = A[row l % 32] and b = B[column
// l % 32] of block l / 32; element 16 q + i of the result is block q in the
// 32x32 output layout (element i of lane l: row 8 (i / 4) + 4 (l / 32) + i % 4,
// column l % 32, the layout of every 32x32 instruction used here).  With a
// zero accumulator each element is the fp32 product a b rounded once.
__device__ __forceinline__ f32x32 mfma_f32_outer2(float a, float b) {
    return __builtin_amdgcn_mfma_f32_32x32x1f32(a, b, f32x32{}, 0, 0, 0);
}

// 32x32 output tile, K = 16 bf16 per call (8 per lane, k-slot l / 32), fp32
// accumulate; same output layout.
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 32x32 output tile, K = 64 E2M1 (4-bit float) per call, each k block of 32
// scaled by its E8M0 byte (the matrix-core form of the OCP MX dot product).
// Lane l supplies, for row/column l % 32, the 32 codes of k block l / 32
// (16 bytes, element 2j in the low nibble of byte j) and that block's scale
// byte in bits 0-7 of sa / sb; fp32 accumulate; the 32x32 output layout.
__device__ __forceinline__ f32x16 mfma_mxfp4_32x32x64(u32x4 a, uint32_t sa, u32x4 b, uint32_t sb,
                                                      f32x16 c) {
    const i32x8 A = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const i32x8 B = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// ---------------------------------------------------------------- GELU

// GELU, erf form: 0.5 x (1 + erf(x / sqrt 2)), with erf from the rational
// approximation of Abramowitz and Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (after Hastings): for z >= 0,
//   erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2),
//   t = 1 / (1 + p z), |error| <= 1.5e-7,
// and erf(-z) = -erf(z); in fp32 with the hardware reciprocal and 2^x, the
// result is within about 3e-7 |x| of the exact GELU (far below a bf16 ulp of
// the output), for a fraction of the instructions of a full-precision erf.
// With z = |x| / sqrt 2 folded into the constants (p / sqrt 2; the a_i
// halved, so the polynomial gives h = (1 - erf(z)) / 2 directly;
// exp(-z^2) = 2^(x^2 (-log2(e) / 2))): GELU(x) = x - x h for x >= 0, x h
// otherwise.
__device__ __forceinline__ float gelu_erf(float x) {
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(fabsf(x), 0.23164188861846924f, 1.0f));
    float p = __builtin_fmaf(t, 0.5307027101516724f, -0.726576030254364f);
    p = __builtin_fmaf(t, p, 0.710706889629364f);
    p = __builtin_fmaf(t, p, -0.14224836230278015f);
    p = __builtin_fmaf(t, p, 0.1274147927761078f);
    const float e = __builtin_amdgcn_exp2f(x * x * -0.7213475108146667f);
    const float xh = x * (p * t * e);                        // x (1 - erf(z)) / 2
    return x >= 0.0f ? x - xh : xh;
}

// ---------------------------------------------------------------- 4-bit operands
// Stored layout of the INT4 codes (qa, qw): two per byte, code e of each block
// of 16 consecutive codes in nibble e of the block's 8 bytes (element 2j in
// the low nibble of byte j); a nibble holds |c_e| in its low three bits and
// the sign of c_((e - 1) mod 16) in its top bit.  One AND then gives the FP8
// (E4M3) bytes of the even codes and a funnel shift plus an AND those of the
// odd codes: the byte s000 0mmm is the E4M3 subnormal (-1)^s m 2^-9, so the
// codes enter the FP8 matrix instruction as exact multiples of 2^-9, and the
// instruction's block scale 2^9 on each operand makes its sums exact
// integers (|sum| <= 64 * 49).

// Two words of 8 two's-complement nibbles (codes 0-7 and 8-15 of a block,
// code e in nibble e mod 8, every code in [-7, 7]) -> the stored words.
__device__ __forceinline__ u32x2 store_code_words(uint32_t w0, uint32_t w1) {
    // nibble-wise two's complement -> sign | magnitude: a negative nibble t
    // (bit 3 set) becomes 8 | (16 - t), i.e. its bits flipped, plus one
    auto sign_mag = [](uint32_t w) {
        const uint32_t sg = w & 0x88888888u;
        const uint32_t one = sg >> 3;
        const uint32_t flip = (sg << 1) - one;       // 0xF in each negative nibble
        return (((w ^ flip) + one) & 0x77777777u) | sg;
    };
    const uint32_t s0 = sign_mag(w0), s1 = sign_mag(w1);
    // each nibble takes the sign bit of the nibble below it (cyclically over
    // the block's 16 nibbles)
    const uint32_t r0 = __builtin_amdgcn_alignbit(s0, s1, 28);
    const uint32_t r1 = __builtin_amdgcn_alignbit(s1, s0, 28);
    return u32x2{(r0 & 0x88888888u) | (s0 & 0x77777777u), (r1 & 0x88888888u) | (s1 & 0x77777777u)};
}

// The FP8 operand of 32 stored codes (two blocks, one 16-byte read).  The
// slot order (codes 0, 2, 4, 6 | 1, 3, 5, 7 | 8, 10, .. of each block) is the
// same for both GEMM operands, so the k pairing is preserved.
__device__ __forceinline__ i32x8 codes_to_fp8(u32x4 x) {
    constexpr uint32_t M = 0x87878787u;
    return i32x8{(int)(x.x & M), (int)(__builtin_amdgcn_alignbit(x.y, x.x, 4) & M),
                 (int)(x.y & M), (int)(__builtin_amdgcn_alignbit(x.x, x.y, 4) & M),
                 (int)(x.z & M), (int)(__builtin_amdgcn_alignbit(x.w, x.z, 4) & M),
                 (int)(x.w & M), (int)(__builtin_amdgcn_alignbit(x.z, x.w, 4) & M)};
}

// 32x32 output tile of exact per-group code sums S = sum_k qa qw over one
// group of 64: lane l supplies row l % 32 and 32 of the group's codes
// (k half l / 32) as FP8; the 32x32 output layout.  Scale bytes 127 + 9
// multiply each operand by 2^9.
__device__ __forceinline__ f32x16 mfma_codes_32x32x64(i32x8 a, i32x8 b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, f32x16{}, 0, 0, 0, 136, 0, 136);
}

// ---------------------------------------------------------------- quantizer

// Quantize one group of 64 values spread over the four lanes
// l, l^16, l^32, l^48 (16 consecutive values per lane).  Returns the group
// scale s = max|v| / 7 (every lane of the group gets it) and writes the
// lane's 16 codes (one block of the stored layout above) into `packed`.
// The code is rint(fl32(v * fl32(1/s))) clamped to [-7, 7]; a
// zero scale or a non-finite 1/s gives zero codes.  Division is IEEE
// correctly rounded (hipcc's default); no contraction is allowed here.
__device__ __forceinline__ float quantize_group16(const float (&v)[16], u32x2 &packed) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    // Max with the lanes l ^ 16 and l ^ 32: a permlane swap leaves, in the
    // two registers, the lane's own value and its partner's (in either
    // order), so their max is the pairwise max.
    {
        const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(amax),
                                                          __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
        const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(amax),
                                                          __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(p32[0]), __uint_as_float(p32[1]));
    }
    const float s = amax / 7.0f;
    float inv = 0.0f;
    if (s != 0.0f) {
        const float t = 1.0f / s;
        inv = __builtin_isfinite(t) ? t : 0.0f;
    }
    // No clamp is needed: with s = fl(amax / 7) and inv = fl(1 / s) finite
    // (s >= 2^-128, so s keeps at least 21 significant bits),
    // |v inv| <= amax inv <= 7 (1 + 2^-20) < 7.5, which rounds to at most 7.
    // rint via the 1.5*2^23 bias: y + 12582912 rounds (nearest even) to an
    // integer whose low 4 bits are the code's two's-complement nibble.  Funnel-shifting the nibbles in from the top
    // leaves element j in nibble j; store_code_words makes the stored form.
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float y = v[j] * inv;
        w0 = __builtin_amdgcn_alignbit(__float_as_uint(y + 12582912.0f), w0, 4);
    }
#pragma unroll
    for (int j = 8; j < 16; ++j) {
        const float y = v[j] * inv;
        w1 = __builtin_amdgcn_alignbit(__float_as_uint(y + 12582912.0f), w1, 4);
    }
    packed = store_code_words(w0, w1);
    return s;
}

// ---------------------------------------------------------------- MXFP4 quantizer

// Quantize the lane's 16 values of a 32-value block shared with lane l ^ 16
// (OCP MX v1.0, MXFP4): the block's scale X = 2^e with
// e = clamp(floor(log2 max|v|) - 2, -127, 127) (v_frexp_exp gives
// floor(log2) + 1 for normal and subnormal values), stored as the E8M0 byte
// e + 127 (0 for an all-zero block); each value becomes the E2M1 number
// nearest to v / X, ties to the even code, saturating at 6, a zero magnitude
// as code 0.  y = v / X is formed exactly (v_ldexp) and rounded by the
// hardware conversion v_cvt_scalef32_pk_fp4_f32 with scale 1: over every
// fp32 |y| <= 8 (every y here, since |v| / X < 8) it gives the same codes as
// rounding to nearest, ties to even, saturating at 6, except that a negative
// value that rounds to zero comes out as -0 (code 8), which is cleared
// afterwards.  Finite inputs only (a NaN gets a nonzero code).  The lane's 16 codes are
// packed element j in nibble j of packed (element 2j in the low nibble of
// byte j).
__device__ __forceinline__ uint32_t mx_quantize16(const float (&v)[16], u32x2 &packed) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    {
        const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(amax),
                                                          __float_as_uint(amax), false, false);
        amax = fmaxf(__uint_as_float(p16[0]), __uint_as_float(p16[1]));
    }
    int e = __builtin_amdgcn_frexp_expf(amax) - 3;
    e = e < -127 ? -127 : (e > 127 ? 127 : e);
    const bool zero = !(amax > 0.0f);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float y[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = __builtin_amdgcn_ldexpf(v[8 * h + j], -e);
        // values 2b, 2b + 1 -> byte b (low, high nibble); the byte index is an immediate
        w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], y[0], y[1], 1.0f, 0);
        w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], y[2], y[3], 1.0f, 1);
        w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], y[4], y[5], 1.0f, 2);
        w[h] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w[h], y[6], y[7], 1.0f, 3);
        // -0 (sign without magnitude) -> +0: a nibble keeps its sign bit
        // only when its magnitude is not zero (m + 7 reaches bit 3 iff m > 0)
        const uint32_t mag = w[h] & 0x77777777u;
        w[h] = mag | (w[h] & (mag + 0x77777777u) & 0x88888888u);
    }
    packed.x = w[0];
    packed.y = w[1];
    return zero ? 0u : (uint32_t)(e + 127);
}

}  // namespace svdq
