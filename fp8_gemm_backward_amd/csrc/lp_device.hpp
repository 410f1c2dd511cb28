// Device helpers shared by the lp kernels: vector types, scale decoding and
// element conversions built on gfx950's conversion instructions.
//
// Facts about the conversion instructions that the kernels rely on (each was
// checked on the hardware against an exact reference over every E2M1 / E4M3
// code and every E8M0 scale byte):
// * v_cvt_scalef32_pk_bf16_{fp4,fp8} multiply two codes by a power of two
//   taken from the EXPONENT FIELD of the fp32 scale operand (exponent field 0
//   is 2^-127, 0xFF is NaN) and round to bf16 exactly; their NaN result is
//   always 0xFFC0.
// * v_cvt_scalef32_pk_f32_{fp4,fp8} likewise use only the exponent field, so a
//   general fp32 block scale is applied with a separate fp32 multiply.
// * v_cvt_scalef32_pk_{fp8,fp4}_f32 divide by the scale's power of two and
//   round to nearest even; the FP8 form does not saturate (values beyond 464
//   become NaN), so inputs are clamped to +-448 first.
// * fp32 -> bf16 conversion (v_cvt_pk_bf16_f32) rounds to nearest even,
//   keeps subnormals and overflows to infinity.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lp {

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(short)))) short i16x2;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

enum Fmt : int { BF16 = 0, MXFP4 = 1, NVFP4 = 2, FP8_B128 = 3, MXFP8 = 4 };

// E8M0 scale byte -> fp32 whose exponent field the scaled conversions read
// (the mantissa is ignored by them).  Byte 0 becomes 0x00400000 (exponent
// field 0, read as 2^-127) and 0xFF becomes the quiet NaN 0x7FC00000.
__device__ __forceinline__ float e8m0_to_cvt_scale(uint32_t s) {
  return __builtin_bit_cast(float, (s << 23) | 0x00400000u);
}

// E8M0 scale byte -> its exact fp32 value 2^(s-127) (2^-127 is an fp32
// subnormal), NaN for 0xFF.  Used where the scale multiplies in fp32.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  uint32_t b = (s == 0xFFu) ? 0x7FC00000u : (s == 0u ? 0x00400000u : (s << 23));
  return __builtin_bit_cast(float, b);
}

__device__ __forceinline__ uint32_t bf16x2_bits(bf16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// Two fp32 -> packed bf16 pair, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times
// a power-of-two scale -> eight bf16 (four dwords, low half first).
__device__ __forceinline__ void fp4x8_to_bf16_pow2(uint32_t w, float cvt_scale, uint32_t out[4]) {
  out[0] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, cvt_scale, 0));
  out[1] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, cvt_scale, 1));
  out[2] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, cvt_scale, 2));
  out[3] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, cvt_scale, 3));
}

// Four E4M3 codes (one dword, byte j = element j) times a power-of-two scale
// -> four bf16 (two dwords).
__device__ __forceinline__ void fp8x4_to_bf16_pow2(uint32_t w, float cvt_scale, uint32_t out[2]) {
  out[0] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, cvt_scale, false));
  out[1] = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, cvt_scale, true));
}

// Eight E2M1 codes times a general fp32 multiplier S: exact code value in
// fp32, one fp32 multiply (RNE), then bf16 (RNE).
__device__ __forceinline__ void fp4x8_to_bf16_mul(uint32_t w, float S, uint32_t out[4]) {
  f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  out[0] = pack_bf16x2(v0[0] * S, v0[1] * S);
  out[1] = pack_bf16x2(v1[0] * S, v1[1] * S);
  out[2] = pack_bf16x2(v2[0] * S, v2[1] * S);
  out[3] = pack_bf16x2(v3[0] * S, v3[1] * S);
}

// Four E4M3 codes times a general fp32 multiplier S.
__device__ __forceinline__ void fp8x4_to_bf16_mul(uint32_t w, float S, uint32_t out[2]) {
  f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
  f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
  out[0] = pack_bf16x2(lo[0] * S, lo[1] * S);
  out[1] = pack_bf16x2(hi[0] * S, hi[1] * S);
}

// Replace any NaN among two packed bf16 by 0x7FC0 carrying the sign bit of
// the element's code (`sign_lo`, `sign_hi` are 0 or 1).
__device__ __forceinline__ uint32_t fix_nan_pair(uint32_t v, uint32_t sign_lo, uint32_t sign_hi) {
  uint32_t lo = v & 0xFFFFu, hi = v >> 16;
  bool nlo = (lo & 0x7F80u) == 0x7F80u && (lo & 0x7Fu) != 0u;
  bool nhi = (hi & 0x7F80u) == 0x7F80u && (hi & 0x7Fu) != 0u;
  lo = nlo ? (0x7FC0u | (sign_lo << 15)) : lo;
  hi = nhi ? (0x7FC0u | (sign_hi << 15)) : hi;
  return lo | (hi << 16);
}

}  // namespace lp
