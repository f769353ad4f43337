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
// Stored layout of the INT4 codes (qa, qw): each block of 16 consecutive codes
// of a row takes 8 bytes (two little-endian words W0, W1).  Code e = 8h + i
// (h = 0, 1; i = 0..7) is field 2i + h of a 96-bit image (bits 6f .. 6f + 5
// for field f) holding the OCP FP6 E2M3 encoding of c / 8: |c| in bits 0-2,
// bits 3-4 zero, the sign in bit 5 (a zero code has none).  With the image
// words I0, I1, I2 (bits 0-31, 32-63, 64-95),
//   W0 = I0 | (I2 & kFree0),   W1 = I1 | (I2 & kFree1),
// where kFree0 / kFree1 are the always-zero bits 3-4 of the fields of I0 / I1
// (bit positions p with p mod 6 in {3, 4}); the two masks are disjoint and
// together cover every bit I2 can hold, so the fold loses nothing and one AND
// per word (two for I2) unfolds it.  The E2M3 subnormal m / 8 is exact, so the
// codes enter the FP6 matrix instruction as exact multiples of 1/8 and the
// instruction's block scale 2^3 on each operand makes its sums exact integers
// (|sum| <= 64 * 49).
constexpr uint32_t kFree0 = 0x18618618u, kFree1 = 0x86186186u;
constexpr uint32_t kKeep0 = ~kFree0, kKeep1 = ~kFree1;     // fields of I0 / I1

typedef float f32x16v __attribute__((ext_vector_type(16)));
typedef int i32x6 __attribute__((ext_vector_type(6)));

// The FP6 images of two 16-code blocks from 32 values that are exact
// multiples of 1/8 in [-7/8, 7/8] (v_cvt_scalef32_2xpk16_fp6_f32, scale 1:
// element j of a goes to field 2j, element j of b to field 2j + 1; so a block's
// codes 0-7 go in a, its codes 8-15 in b, the first block at j < 8).  Words
// 0-2 are the first block's image, words 3-5 the second's.
__device__ __forceinline__ i32x6 fp6_images(const f32x16v &a, const f32x16v &b) {
    return __builtin_bit_cast(i32x6, __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f));
}

// Fold one block's image words into the stored words.
__device__ __forceinline__ u32x2 fold_image(uint32_t i0, uint32_t i1, uint32_t i2) {
    return u32x2{(i2 & kFree0) | i0, (i2 & kFree1) | i1};
}

// c / 8 from a value y whose nearest integer (ties to even) is the code c:
// y + 1.5 * 2^23 rounds to 1.5 * 2^23 + c, and one fma scales that by 1/8 and
// removes the bias exactly (every term is a multiple of 1/8 far inside fp32's
// range); a zero code comes out as +0, never -0.
__device__ __forceinline__ float code_eighths(float y) {
    return __builtin_fmaf(y + 12582912.0f, 0.125f, -1572864.0f);
}

// Two words of 8 two's-complement nibbles (codes 0-7 and 8-15 of a block,
// code e in nibble e mod 8, every code in [-7, 7]) -> the stored words.
__device__ __forceinline__ u32x2 store_code_words(uint32_t w0, uint32_t w1) {
    f32x16v a = {}, b = {};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = (float)((int)(w0 << (28 - 4 * j)) >> 28) * 0.125f;
        b[j] = (float)((int)(w1 << (28 - 4 * j)) >> 28) * 0.125f;
    }
    const i32x6 img = fp6_images(a, b);
    return fold_image((uint32_t)img[0], (uint32_t)img[1], (uint32_t)img[2]);
}

// The FP6 operand of 32 stored codes (two blocks, one 16-byte read): the two
// images unfolded, 192 bits in six registers.  Field order is the same for
// both GEMM operands, so the k pairing is preserved.
__device__ __forceinline__ i32x8 codes_to_fp6(u32x4 x) {
    return i32x8{(int)(x.x & kKeep0), (int)(x.y & kKeep1), (int)((x.x & kFree0) | (x.y & kFree1)),
                 (int)(x.z & kKeep0), (int)(x.w & kKeep1), (int)((x.z & kFree0) | (x.w & kFree1)),
                 0, 0};
}

// 32x32 output tile of exact per-group code sums S = sum_k qa qw over one
// group of 64: lane l supplies row l % 32 and 32 of the group's codes
// (k half l / 32) as FP6 (E2M3); the 32x32 output layout.  Scale bytes 127 + 3
// multiply each operand by 2^3.
__device__ __forceinline__ f32x16 mfma_codes_32x32x64(i32x8 a, i32x8 b) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, f32x16{}, 2, 2, 0, 130, 0, 130);
}

// ---------------------------------------------------------------- quantizer

// Quantize one group of 64 values spread over the four lanes
// l, l^16, l^32, l^48 (16 consecutive values per lane).  Returns the group
// scale s = max|v| / 7 (every lane of the group gets it) and writes the
// lane's 16 codes (one block of the stored layout above) into `packed`.
// The code is rint(fl32(v * fl32(1/s))), always within [-7, 7]; a
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
    // Codes 0-7 of the block go to a, 8-15 to b (the stored field order).
    f32x16v a = {}, b = {};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = code_eighths(v[j] * inv);
        b[j] = code_eighths(v[8 + j] * inv);
    }
    const i32x6 img = fp6_images(a, b);
    packed = fold_image((uint32_t)img[0], (uint32_t)img[1], (uint32_t)img[2]);
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
