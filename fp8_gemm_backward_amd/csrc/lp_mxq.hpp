// MX quantization of bf16 values, element by element (OCP MX scale rule,
// E4M3 / E2M1 elements, nearest even, saturating): the arithmetic shared
// by the standalone quantizers and the grad_X kernel that quantizes its
// weight operand itself.
//
// "perf: defer mxfp8 backward quantization": the backward quantizes with
// one E8M0 scale per 32 elements.  Per block: amax over |v| is taken on the
// bf16 bit patterns (integer max of the magnitude bits, which also flags
// NaN / infinity as >= 0x7F80); e = floor(log2 amax) - emax, clamped to
// [-127, 127], comes exactly from the exponent field (or the leading
// mantissa bit of a subnormal); each element is multiplied by 2^-e (exact),
// clamped to the format's maximum (saturation) and rounded to nearest even
// by the hardware conversion.
#pragma once

#include "lp_device.hpp"

namespace lp {

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// floor(log2 |v|) of a non-zero finite bf16 magnitude (bits & 0x7FFF).
__device__ __forceinline__ int floor_log2_bf16(uint32_t mag) {
  uint32_t e = mag >> 7;
  return e ? (int)e - 127 : (31 - __builtin_clz(mag)) - 133;
}

struct BlockScale {
  uint32_t byte;   // E8M0 scale byte
  float inv;       // 2^-e as fp32 (exact)
  bool bad;        // NaN or infinity in the block
};

template <bool kFp4>
__device__ __forceinline__ BlockScale block_scale(uint32_t amax_mag) {
  constexpr int kEmax = kFp4 ? 2 : 8;
  BlockScale s;
  s.bad = amax_mag >= 0x7F80u;
  int e = (amax_mag == 0u || s.bad) ? -127 : floor_log2_bf16(amax_mag) - kEmax;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  s.byte = s.bad ? 0xFFu : (uint32_t)(e + 127);
  s.inv = __builtin_bit_cast(float, (uint32_t)(127 - e) << 23);   // 127-e in [8, 254]
  return s;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Two scaled values -> two E4M3 codes (low byte first) in a 16-bit result.
__device__ __forceinline__ uint32_t to_e4m3x2(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  i16x2 old = {0, 0};
  i16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, a, b, 1.0f, false);
  return (uint32_t)(uint16_t)r[0];
}

// Two scaled values -> one byte of two E2M1 codes (first in the low nibble).
__device__ __forceinline__ uint32_t to_e2m1x2(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -6.0f, 6.0f);
  b = __builtin_amdgcn_fmed3f(b, -6.0f, 6.0f);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}

// E4M3 codes of bf16 pairs by the scaled bf16 conversion, without fp32
// arithmetic.  For a block scale byte b (not 0xFF) each magnitude is first
// clamped to 448 * 2^(b - 127), the largest that stays in range (the
// conversion does not saturate), on the bit patterns: a signed 16-bit min
// clamps positive values and leaves negative ones, an unsigned min against
// sign | threshold clamps negative ones.  The conversion then takes off the
// power of two in its scale operand's exponent field (b) and rounds to
// nearest even: the codes to_e4m3x2 gives for the elements times s.inv.
struct E4M3Scale {
  float sc;       // scale operand: exponent field b
  uint32_t thr;   // bf16 bits of 448 * 2^(b - 127), in both halves
};
__device__ __forceinline__ E4M3Scale e4m3_scale(uint32_t byte) {
  E4M3Scale q;
  q.sc = __builtin_bit_cast(float, byte << 23);
  q.thr = (((byte + 8u) << 7) | 0x60u) * 0x00010001u;   // b <= 246 for a finite block
  return q;
}
// The pair w (low element first) clamped and converted into the high
// (kHi) or low half of old (the other half kept).
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_scaled(uint32_t old, uint32_t w, const E4M3Scale& q) {
  typedef short s16x2v __attribute__((ext_vector_type(2)));
  typedef unsigned short u16x2v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
  const uint32_t pos = __builtin_bit_cast(
      uint32_t, __builtin_elementwise_min(__builtin_bit_cast(s16x2v, w), __builtin_bit_cast(s16x2v, q.thr)));
  const uint32_t c = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2v, pos),
                                                                          __builtin_bit_cast(u16x2v, q.thr | 0x80008000u)));
  const s16x2v r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(s16x2v, old),
                                                             __builtin_bit_cast(bf16x2v, c), q.sc, kHi);
  return __builtin_bit_cast(uint32_t, r);
}

// NaN codes of a bad block: E4M3 0x7F with each element's sign; E2M1 0.
__device__ __forceinline__ uint32_t nan_e4m3x2(uint32_t w) {
  return 0x7F7Fu | ((w >> 8) & 0x80u) | ((w >> 16) & 0x8000u);
}

__device__ __forceinline__ uint32_t pk_umax16(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

}  // namespace lp
