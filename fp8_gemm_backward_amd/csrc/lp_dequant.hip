// Standalone dequantization to bf16 (HBM-bound, bit-exact).
//
// "Add Autograd Backward Support for FP4 GEMM Custom Ops": the backward
// dequantizes the saved packed FP4 operands to BF16; "Train adapters on top
// of FP8 weights", _dequantize_fp8_weight: E4M3 codes times their
// per-128x128-block fp32 inverse scale.
//
// The work unit is eight consecutive elements of a row (every format's
// scale blocks and rows are multiples of eight elements, so a unit never
// straddles one): four code bytes (E2M1) or eight (E4M3) in, sixteen bytes
// of bf16 out.  Lane i of a wave takes unit base + i, so every load and
// every store of a wave covers one contiguous span (256 B / 512 B of codes,
// 1 KiB of bf16).  Each thread handles kUnits units, spaced a workgroup
// apart, with all their loads issued before the first decode so that enough
// bytes are in flight to cover the HBM latency; codes and results are
// touched once, so loads and stores are nontemporal.  The decoded value is
// bf16_rne(fp32_rne(code * S)); a NaN result is 0x7FC0 with the code's sign.
#include "lp_device.hpp"
#include "lp_internal.hpp"

namespace lp {

namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 4;                       // units per thread
constexpr int kSpan = kThreads * kUnits;        // units per workgroup

// Sign bit of nibble-code e (0..7) of an E2M1 dword / of byte e (0..3) of an E4M3 dword.
__device__ __forceinline__ uint32_t fp4_sign(uint32_t w, int e) { return (w >> (4 * e + 3)) & 1u; }
__device__ __forceinline__ uint32_t fp8_sign(uint32_t w, int e) { return (w >> (8 * e + 7)) & 1u; }

// Eight E2M1 codes -> bf16 with the NaN results rewritten (only a NaN scale
// or a NaN/infinite multiplier makes one).
__device__ __forceinline__ u32x4 fix_fp4(const uint32_t o[4], uint32_t w) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) r[k] = fix_nan_pair(o[k], fp4_sign(w, 2 * k), fp4_sign(w, 2 * k + 1));
  return r;
}
__device__ __forceinline__ u32x4 fix_fp8(const uint32_t o[4], u32x2 w) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t d = w[k >> 1];
    const int e = 2 * (k & 1);
    r[k] = fix_nan_pair(o[k], fp8_sign(d, e), fp8_sign(d, e + 1));
  }
  return r;
}

// Unit index of load slot j of this thread, and whether it exists.
__device__ __forceinline__ uint32_t unit_of(int j) { return blockIdx.x * kSpan + j * kThreads + threadIdx.x; }

// MXFP4: unit u = codes dword u, scale byte u / 4.
__global__ __launch_bounds__(kThreads) void dequant_mxfp4(const uint32_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales,
                                                          u32x4* __restrict__ out, uint32_t nunits) {
  uint32_t c[kUnits], s[kUnits];
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    c[j] = u < nunits ? __builtin_nontemporal_load(codes + u) : 0u;
    s[j] = u < nunits ? scales[u >> 2] : 0u;
  }
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    if (u >= nunits) break;
    uint32_t o[4];
    fp4x8_to_bf16_pow2(c[j], e8m0_to_cvt_scale(s[j]), o);
    __builtin_nontemporal_store(s[j] == 0xFFu ? fix_fp4(o, c[j]) : u32x4{o[0], o[1], o[2], o[3]}, out + u);
  }
}

// NVFP4: unit u = codes dword u, E4M3 block-scale byte u / 2, times the
// fp32 tensor scale (one fp32 rounding per block).
__global__ __launch_bounds__(kThreads) void dequant_nvfp4(const uint32_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales,
                                                          const float* __restrict__ tensor_scale,
                                                          u32x4* __restrict__ out, uint32_t nunits) {
  uint32_t c[kUnits], s[kUnits];
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    c[j] = u < nunits ? __builtin_nontemporal_load(codes + u) : 0u;
    s[j] = u < nunits ? scales[u >> 1] : 0u;
  }
  const float ts = *tensor_scale;
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    if (u >= nunits) break;
    const float S = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(s[j], 1.0f, false)[0] * ts;
    uint32_t o[4];
    fp4x8_to_bf16_mul(c[j], S, o);
    __builtin_nontemporal_store(fix_fp4(o, c[j]), out + u);
  }
}

// MXFP8 with scale blocks along the columns: unit u = codes bytes [8u, 8u+8),
// scale byte u / 4.
__global__ __launch_bounds__(kThreads) void dequant_mxfp8_cols(const u32x2* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales,
                                                               u32x4* __restrict__ out, uint32_t nunits) {
  u32x2 c[kUnits];
  uint32_t s[kUnits];
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    c[j] = u < nunits ? __builtin_nontemporal_load(codes + u) : u32x2{0u, 0u};
    s[j] = u < nunits ? scales[u >> 2] : 0u;
  }
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    if (u >= nunits) break;
    const float cs = e8m0_to_cvt_scale(s[j]);
    uint32_t o[4];
    fp8x4_to_bf16_pow2(c[j][0], cs, o);
    fp8x4_to_bf16_pow2(c[j][1], cs, o + 2);
    __builtin_nontemporal_store(fix_fp8(o, c[j]), out + u);
  }
}

// MXFP8 with scale blocks along the rows: unit u = 8 consecutive columns of
// one row; column c of row r has its own scale byte scales[r / 32][c].
__global__ __launch_bounds__(kThreads) void dequant_mxfp8_rows(const u32x2* __restrict__ codes,
                                                               const uint8_t* __restrict__ scales,
                                                               u32x4* __restrict__ out, uint32_t nunits,
                                                               FastDiv units_per_row, uint32_t cols) {
  u32x2 c[kUnits], s[kUnits];
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    const uint32_t row = fdiv(u, units_per_row);         // over batch*rows
    const uint32_t col = (u - row * units_per_row.d) * 8u;
    c[j] = u < nunits ? __builtin_nontemporal_load(codes + u) : u32x2{0u, 0u};
    s[j] = u < nunits ? *reinterpret_cast<const u32x2*>(scales + (size_t)(row >> 5) * cols + col) : u32x2{0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    if (u >= nunits) break;
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[j][h], 1.0f, false);
      const f32x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c[j][h], 1.0f, true);
      const uint32_t sw = s[j][h];
      o[2 * h] = pack_bf16x2(lo[0] * e8m0_to_f32(sw & 0xFFu), lo[1] * e8m0_to_f32((sw >> 8) & 0xFFu));
      o[2 * h + 1] = pack_bf16x2(hi[0] * e8m0_to_f32((sw >> 16) & 0xFFu), hi[1] * e8m0_to_f32(sw >> 24));
    }
    __builtin_nontemporal_store(fix_fp8(o, c[j]), out + u);
  }
}

// FP8 E4M3 with fp32 inverse scales per 128x128 block: unit u = 8
// consecutive columns of one row (inside one block).
__global__ __launch_bounds__(kThreads) void dequant_fp8_b128(const u32x2* __restrict__ codes,
                                                             const float* __restrict__ scales,
                                                             u32x4* __restrict__ out, uint32_t nunits,
                                                             FastDiv units_per_row, FastDiv rows_per_batch,
                                                             uint32_t sblk_rows, uint32_t sblk_cols) {
  u32x2 c[kUnits];
  float S[kUnits];
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    const uint32_t grow = fdiv(u, units_per_row);        // row over batch*rows
    const uint32_t col = (u - grow * units_per_row.d) * 8u;
    const uint32_t b = fdiv(grow, rows_per_batch);
    const uint32_t r = grow - b * rows_per_batch.d;
    c[j] = u < nunits ? __builtin_nontemporal_load(codes + u) : u32x2{0u, 0u};
    S[j] = u < nunits ? scales[((size_t)b * sblk_rows + (r >> 7)) * sblk_cols + (col >> 7)] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = unit_of(j);
    if (u >= nunits) break;
    uint32_t o[4];
    fp8x4_to_bf16_mul(c[j][0], S[j], o);
    fp8x4_to_bf16_mul(c[j][1], S[j], o + 2);
    __builtin_nontemporal_store(fix_fp8(o, c[j]), out + u);
  }
}

}  // namespace

hipError_t launch_dequant(const lp_qtensor& t, void* dst, hipStream_t stream) {
  const int64_t n = t.batch * t.rows * t.cols;
  if (n == 0) return hipSuccess;
  const uint32_t nunits = (uint32_t)(n / 8);             // cols % 16 == 0, so n % 8 == 0
  const dim3 grid((nunits + kSpan - 1) / kSpan), block(kThreads);
  u32x4* out = static_cast<u32x4*>(dst);
  const auto* c32 = static_cast<const uint32_t*>(t.codes);
  const auto* c64 = static_cast<const u32x2*>(t.codes);
  const auto* s8 = static_cast<const uint8_t*>(t.scales);
  switch (t.fmt) {
    case LP_MXFP4:
      dequant_mxfp4<<<grid, block, 0, stream>>>(c32, s8, out, nunits);
      break;
    case LP_NVFP4:
      dequant_nvfp4<<<grid, block, 0, stream>>>(c32, s8, t.tensor_scale, out, nunits);
      break;
    case LP_MXFP8:
      if (t.scale_axis == -1)
        dequant_mxfp8_cols<<<grid, block, 0, stream>>>(c64, s8, out, nunits);
      else
        dequant_mxfp8_rows<<<grid, block, 0, stream>>>(c64, s8, out, nunits, make_fastdiv((uint32_t)(t.cols / 8)),
                                                       (uint32_t)t.cols);
      break;
    case LP_FP8_B128:
      dequant_fp8_b128<<<grid, block, 0, stream>>>(
          c64, static_cast<const float*>(t.scales), out, nunits, make_fastdiv((uint32_t)(t.cols / 8)),
          make_fastdiv((uint32_t)t.rows), (uint32_t)((t.rows + 127) / 128), (uint32_t)((t.cols + 127) / 128));
      break;
    case LP_FP8T_E4M3:
    case LP_FP8T_E5M2:
      return launch_tensor_dequant(t, dst, stream);
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lp
