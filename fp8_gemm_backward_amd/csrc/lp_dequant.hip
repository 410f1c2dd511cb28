// Standalone dequantization to bf16 (HBM-bound, bit-exact).
//
// "Add Autograd Backward Support for FP4 GEMM Custom Ops": the backward
// dequantizes the saved packed FP4 operands to BF16; "Train adapters on top
// of FP8 weights", _dequantize_fp8_weight: E4M3 codes times their
// per-128x128-block fp32 inverse scale.
//
// Each thread decodes one 16-byte chunk of codes (32 FP4 or 16 FP8 elements)
// with a single vector load and writes 32 or 64 bytes of bf16 with vector
// stores; chunks never straddle a scale block.  The decoded value is
// bf16_rne(fp32_rne(code * S)); a NaN result is 0x7FC0 with the code's sign.
#include "lp_device.hpp"
#include "lp_internal.hpp"

namespace lp {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void store_bf16(u32x4* out, const uint32_t* o, int n16) {
#pragma unroll
  for (int j = 0; j < n16; ++j) out[j] = u32x4{o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
}

// Sign bits of the two E2M1 codes of byte `k` of a 16-byte chunk.
__device__ __forceinline__ uint32_t fp4_sign_lo(const u32x4& c, int k) { return (c[k >> 2] >> (8 * (k & 3) + 3)) & 1u; }
__device__ __forceinline__ uint32_t fp4_sign_hi(const u32x4& c, int k) { return (c[k >> 2] >> (8 * (k & 3) + 7)) & 1u; }
// Sign bit of E4M3 code `e` (0..15) of a 16-byte chunk.
__device__ __forceinline__ uint32_t fp8_sign(const u32x4& c, int e) { return (c[e >> 2] >> (8 * (e & 3) + 7)) & 1u; }

// MXFP4: chunk i covers elements [32i, 32i+32) = scale block i.
__global__ __launch_bounds__(kThreads) void dequant_mxfp4(const u32x4* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales,
                                                          u32x4* __restrict__ out, uint32_t nchunks) {
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= nchunks) return;
  u32x4 c = __builtin_nontemporal_load(codes + i);
  uint32_t s = scales[i];
  float cs = e8m0_to_cvt_scale(s);
  uint32_t o[16];
#pragma unroll
  for (int j = 0; j < 4; ++j) fp4x8_to_bf16_pow2(c[j], cs, o + 4 * j);
  if (s == 0xFFu) {
#pragma unroll
    for (int k = 0; k < 16; ++k) o[k] = fix_nan_pair(o[k], fp4_sign_lo(c, k), fp4_sign_hi(c, k));
  }
  store_bf16(out + 4 * (size_t)i, o, 4);
}

// NVFP4: chunk i covers elements [32i, 32i+32) = scale blocks 2i, 2i+1.
__global__ __launch_bounds__(kThreads) void dequant_nvfp4(const u32x4* __restrict__ codes,
                                                          const uint16_t* __restrict__ scales,
                                                          const float* __restrict__ tensor_scale,
                                                          u32x4* __restrict__ out, uint32_t nchunks) {
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= nchunks) return;
  u32x4 c = __builtin_nontemporal_load(codes + i);
  uint32_t sb = scales[i];
  float ts = *tensor_scale;
  f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sb, 1.0f, false);
  float S0 = sv[0] * ts, S1 = sv[1] * ts;
  uint32_t o[16];
  fp4x8_to_bf16_mul(c[0], S0, o + 0);
  fp4x8_to_bf16_mul(c[1], S0, o + 4);
  fp4x8_to_bf16_mul(c[2], S1, o + 8);
  fp4x8_to_bf16_mul(c[3], S1, o + 12);
#pragma unroll
  for (int k = 0; k < 16; ++k) o[k] = fix_nan_pair(o[k], fp4_sign_lo(c, k), fp4_sign_hi(c, k));
  store_bf16(out + 4 * (size_t)i, o, 4);
}

// MXFP8 with scale blocks along the columns: chunk i = elements [16i, 16i+16),
// scale block i/2.
__global__ __launch_bounds__(kThreads) void dequant_mxfp8_cols(const u32x4* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales,
                                                               u32x4* __restrict__ out, uint32_t nchunks) {
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= nchunks) return;
  u32x4 c = __builtin_nontemporal_load(codes + i);
  float cs = e8m0_to_cvt_scale(scales[i >> 1]);
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) fp8x4_to_bf16_pow2(c[j], cs, o + 2 * j);
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = fix_nan_pair(o[k], fp8_sign(c, 2 * k), fp8_sign(c, 2 * k + 1));
  store_bf16(out + 2 * (size_t)i, o, 2);
}

// MXFP8 with scale blocks along the rows: chunk i = 16 consecutive columns of
// one row; each column has its own scale byte scales[row/32][col].
__global__ __launch_bounds__(kThreads) void dequant_mxfp8_rows(const u32x4* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales,
                                                               u32x4* __restrict__ out, uint32_t nchunks,
                                                               FastDiv chunks_per_row, uint32_t cols) {
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= nchunks) return;
  uint32_t row = fdiv(i, chunks_per_row);               // over batch*rows
  uint32_t col = (i - row * chunks_per_row.d) * 16u;
  u32x4 c = __builtin_nontemporal_load(codes + i);
  u32x4 s = *reinterpret_cast<const u32x4*>(scales + (size_t)(row >> 5) * cols + col);
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[j], 1.0f, false);
    f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[j], 1.0f, true);
    uint32_t sw = s[j];
    o[2 * j] = pack_bf16x2(lo[0] * e8m0_to_f32(sw & 0xFFu), lo[1] * e8m0_to_f32((sw >> 8) & 0xFFu));
    o[2 * j + 1] = pack_bf16x2(hi[0] * e8m0_to_f32((sw >> 16) & 0xFFu), hi[1] * e8m0_to_f32(sw >> 24));
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = fix_nan_pair(o[k], fp8_sign(c, 2 * k), fp8_sign(c, 2 * k + 1));
  store_bf16(out + 2 * (size_t)i, o, 2);
}

// FP8 E4M3 with fp32 inverse scales per 128x128 block: chunk i = 16
// consecutive columns of one row (all inside one block).
__global__ __launch_bounds__(kThreads) void dequant_fp8_b128(const u32x4* __restrict__ codes,
                                                             const float* __restrict__ scales,
                                                             u32x4* __restrict__ out, uint32_t nchunks,
                                                             FastDiv chunks_per_row, FastDiv rows_per_batch,
                                                             uint32_t sblk_rows, uint32_t sblk_cols) {
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= nchunks) return;
  uint32_t grow = fdiv(i, chunks_per_row);              // row over batch*rows
  uint32_t col = (i - grow * chunks_per_row.d) * 16u;
  uint32_t b = fdiv(grow, rows_per_batch);
  uint32_t r = grow - b * rows_per_batch.d;
  float S = scales[((size_t)b * sblk_rows + (r >> 7)) * sblk_cols + (col >> 7)];
  u32x4 c = __builtin_nontemporal_load(codes + i);
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) fp8x4_to_bf16_mul(c[j], S, o + 2 * j);
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = fix_nan_pair(o[k], fp8_sign(c, 2 * k), fp8_sign(c, 2 * k + 1));
  store_bf16(out + 2 * (size_t)i, o, 2);
}

}  // namespace

hipError_t launch_dequant(const lp_qtensor& t, void* dst, hipStream_t stream) {
  const int64_t n = t.batch * t.rows * t.cols;
  if (n == 0) return hipSuccess;
  const int per_chunk = (t.fmt == LP_MXFP4 || t.fmt == LP_NVFP4) ? 32 : 16;
  const uint32_t nchunks = (uint32_t)(n / per_chunk);
  const dim3 grid((nchunks + kThreads - 1) / kThreads), block(kThreads);
  const u32x4* codes = static_cast<const u32x4*>(t.codes);
  u32x4* out = static_cast<u32x4*>(dst);
  switch (t.fmt) {
    case LP_MXFP4:
      dequant_mxfp4<<<grid, block, 0, stream>>>(codes, static_cast<const uint8_t*>(t.scales), out, nchunks);
      break;
    case LP_NVFP4:
      dequant_nvfp4<<<grid, block, 0, stream>>>(codes, static_cast<const uint16_t*>(t.scales), t.tensor_scale, out,
                                                nchunks);
      break;
    case LP_MXFP8:
      if (t.scale_axis == -1)
        dequant_mxfp8_cols<<<grid, block, 0, stream>>>(codes, static_cast<const uint8_t*>(t.scales), out, nchunks);
      else
        dequant_mxfp8_rows<<<grid, block, 0, stream>>>(codes, static_cast<const uint8_t*>(t.scales), out, nchunks,
                                                       make_fastdiv((uint32_t)(t.cols / 16)), (uint32_t)t.cols);
      break;
    case LP_FP8_B128:
      dequant_fp8_b128<<<grid, block, 0, stream>>>(
          codes, static_cast<const float*>(t.scales), out, nchunks, make_fastdiv((uint32_t)(t.cols / 16)),
          make_fastdiv((uint32_t)t.rows), (uint32_t)((t.rows + 127) / 128), (uint32_t)((t.cols + 127) / 128));
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lp
