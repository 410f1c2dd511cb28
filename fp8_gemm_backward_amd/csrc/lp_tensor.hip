// Per-tensor scaled FP8: quantization with amax recording, amax, scale from
// an amax history, and decoding (HBM-bound; quantization and decoding are
// bit-exact).
//
// "AstrAI fp8.py": every operand's scale is a quantization step
// scale = (amax / FP8_MAX) / 2^margin (at least 1e-12), FP8_MAX = 448 (E4M3)
// or 57344 (E5M2), taken over an amax history ring (delayed scaling) or the
// current amax (dynamic scaling); the backward quantizes its operands with
// those scales and records the gradient's amax for the ring.
//
// Quantization: t = x / scale (IEEE fp32 division), saturated to
// +-FP8_MAX (infinities included), then rounded to nearest even by the
// hardware conversion; NaN becomes 0x7F with the element's sign.  The scale
// is one value for the whole tensor, so the quotient is formed from its
// correctly rounded reciprocal y (one IEEE division per thread) with
// Markstein's correction: q ~ x y, r = x - s q (exact, one fma), t = q + r y
// rounded once, which is the correctly rounded x / s when q is within an ulp
// of it and nothing underflows or overflows (P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 34(1), 1990).  For 2^-80 <= s <= 2^100 every intermediate of a
// quotient that can round to a nonzero FP8 value is a normal number, and
// quotients beyond 2^20 (saturated in any case) are clamped before the
// correction, and the result takes x's sign (a zero quotient would lose it);
// other scales take the IEEE division.  amax is
// max |x| as the fp32 bit pattern of the largest bf16 magnitude: the bit
// patterns of non-negative floats order like the floats, NaN patterns above
// infinity, so an integer atomic max over them is max |x| with NaN winning.
//
// Atomic maxima on one address are serialised by the memory system (about
// 10 ns each, measured), so a kernel that records an amax runs at most one
// workgroup per compute unit, loops over the tensor, reduces across the
// workgroup in LDS and issues a single atomic.
#include "lp_device.hpp"
#include "lp_internal.hpp"

namespace lp {

namespace {

constexpr int kThreads = 256;
constexpr int kUnits = 4;                       // 8-element units per thread
constexpr int kSpan = kThreads * kUnits;
constexpr int kRedThreads = 1024;               // workgroup of the amax-recording kernels
constexpr int kRedBlocks = 256;                 // at most one per compute unit

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

__device__ __forceinline__ float fp8_max(bool e5m2) { return e5m2 ? 57344.0f : 448.0f; }

__device__ __forceinline__ uint32_t pk_umax16(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}

// Largest bf16 magnitude (as fp32 bits) of a unit's eight elements: a
// packed 16-bit maximum over the sign-cleared pairs, then the two halves.
__device__ __forceinline__ uint32_t unit_amax_bits(const u32x4& v) {
  const uint32_t m = pk_umax16(pk_umax16(v[0] & 0x7FFF7FFFu, v[1] & 0x7FFF7FFFu),
                               pk_umax16(v[2] & 0x7FFF7FFFu, v[3] & 0x7FFF7FFFu));
  const uint32_t lo = m & 0xFFFFu, hi = m >> 16;
  return (lo > hi ? lo : hi) << 16;
}

// Workgroup maximum (every thread calls), then one atomic per workgroup.
__device__ __forceinline__ void record_amax(uint32_t m, uint32_t* out) {
  __shared__ uint32_t s_max[kRedThreads / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, off);
    m = m > o ? m : o;
  }
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x / 64] = m;
  __syncthreads();
  if (threadIdx.x != 0) return;
  for (int w = 1; w < (int)(blockDim.x / 64); ++w) m = m > s_max[w] ? m : s_max[w];
  if (m != 0) __hip_atomic_fetch_max(out, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void zero_u32(uint32_t* p) { *p = 0u; }

// Units base + j NT + tid (j < kUnits) of src into v; zeros past the end.
template <int NT>
__device__ __forceinline__ void load_units(const u32x4* __restrict__ src, uint32_t nunits, uint32_t base,
                                           u32x4 (&v)[kUnits]) {
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = base + j * NT + threadIdx.x;
    v[j] = u < nunits ? __builtin_nontemporal_load(src + u) : u32x4{0u, 0u, 0u, 0u};
  }
}

// A workgroup's share of a grid-stride loop over spans of NT * kUnits
// units: body(v, base) for each span, with the next span's loads issued
// before the current span is processed.
template <int NT, class Body>
__device__ __forceinline__ void stride_loop(const u32x4* __restrict__ src, uint32_t nunits, Body body) {
  const uint32_t span = NT * kUnits, stride = gridDim.x * span;
  uint32_t base = blockIdx.x * span;
  if (base >= nunits) return;
  u32x4 cur[kUnits];
  load_units<NT>(src, nunits, base, cur);
  while (true) {
    const uint32_t next = base + stride;
    u32x4 nxt[kUnits];
    if (next < nunits) load_units<NT>(src, nunits, next, nxt);
    body(cur, base);
    if (next >= nunits) break;
#pragma unroll
    for (int j = 0; j < kUnits; ++j) cur[j] = nxt[j];
    base = next;
  }
}

__global__ __launch_bounds__(kRedThreads) void tensor_amax(const u32x4* __restrict__ src, uint32_t nunits,
                                                           uint32_t* __restrict__ amax) {
  uint32_t m = 0;
  stride_loop<kRedThreads>(src, nunits, [&](const u32x4 (&v)[kUnits], uint32_t) {
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      const uint32_t a = unit_amax_bits(v[j]);
      m = m > a ? m : a;
    }
  });
  record_amax(m, amax);
}

// x / s: with kFast, from y = RN(1 / s) as described above.
template <bool kFast>
__device__ __forceinline__ float quotient(float x, float s, float y) {
  if constexpr (kFast) {
    const float q = __builtin_amdgcn_fmed3f(x * y, -0x1p20f, 0x1p20f);
    const float r = __builtin_fmaf(-s, q, x);
    return __builtin_copysignf(__builtin_fmaf(r, y, q), x);       // q = -0 would give +0
  } else {
    return x / s;
  }
}

// Two elements -> two FP8 codes (low byte first).  NaN inputs are fixed by
// the caller.
template <bool kE5M2, bool kFast>
__device__ __forceinline__ uint32_t quant_pair(float a, float b, float s, float y) {
  const float mx = fp8_max(kE5M2);
  const float ca = __builtin_amdgcn_fmed3f(quotient<kFast>(a, s, y), -mx, mx);
  const float cb = __builtin_amdgcn_fmed3f(quotient<kFast>(b, s, y), -mx, mx);
  i16x2 old = {0, 0};
  if constexpr (kE5M2)
    return (uint32_t)(uint16_t)__builtin_amdgcn_cvt_scalef32_pk_bf8_f32(old, ca, cb, 1.0f, false)[0];
  else
    return (uint32_t)(uint16_t)__builtin_amdgcn_cvt_scalef32_pk_fp8_f32(old, ca, cb, 1.0f, false)[0];
}

// The NaN elements of a unit (8 bf16 in v) get code 0x7F with their sign.
__device__ __forceinline__ void fix_nan_codes(const u32x4& v, uint32_t o[2]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t h = (v[e / 2] >> (16 * (e & 1))) & 0xFFFFu;
    if ((h & 0x7FFFu) > 0x7F80u) {
      const uint32_t sh = 8 * (e & 3);
      o[e / 4] = (o[e / 4] & ~(0xFFu << sh)) | ((0x7Fu | ((h >> 8) & 0x80u)) << sh);
    }
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Unit u: 8 bf16 in (16 bytes), 8 codes out (8 bytes).  kAmax: the amax of
// the input goes to `amax` (one workgroup per compute unit at most, looping;
// else one pass of kSpan units per workgroup).
template <bool kE5M2, bool kAmax>
__global__ __launch_bounds__(kAmax ? kRedThreads : kThreads) void tensor_quant(
    const u32x4* __restrict__ src, uint32_t nunits, const float* __restrict__ scale, u32x2* __restrict__ codes,
    uint32_t* __restrict__ amax) {
  constexpr uint32_t NT_ = kAmax ? kRedThreads : kThreads;
  constexpr uint32_t span = NT_ * kUnits;
  const float s = *scale;
  const float y = 1.0f / s;
  uint32_t m = 0;
  auto pass = [&](auto fast) {
    constexpr bool kFast = decltype(fast)::value;
    auto body = [&](const u32x4 (&v)[kUnits], uint32_t base) {
#pragma unroll
      for (int j = 0; j < kUnits; ++j) {
        const uint32_t u = base + j * NT_ + threadIdx.x;
        if (u >= nunits) continue;
        const uint32_t a = unit_amax_bits(v[j]);
        if constexpr (kAmax) m = m > a ? m : a;
        uint32_t o[2];
#pragma unroll
        for (int k = 0; k < 4; k += 2) {
          const uint32_t lo = quant_pair<kE5M2, kFast>(bf16_lo(v[j][k]), bf16_hi(v[j][k]), s, y);
          const uint32_t hi = quant_pair<kE5M2, kFast>(bf16_lo(v[j][k + 1]), bf16_hi(v[j][k + 1]), s, y);
          o[k / 2] = lo | (hi << 16);
        }
        if (a > 0x7F800000u) fix_nan_codes(v[j], o);              // a NaN in the unit
        __builtin_nontemporal_store(u32x2{o[0], o[1]}, codes + u);
      }
    };
    if constexpr (kAmax) {
      stride_loop<NT_>(src, nunits, body);
    } else {                                                     // the grid covers every unit once
      u32x4 v[kUnits];
      load_units<NT_>(src, nunits, blockIdx.x * span, v);
      body(v, blockIdx.x * span);
    }
  };
  if (s >= 0x1p-80f && s <= 0x1p100f) pass(Flag<true>{});
  else pass(Flag<false>{});
  if constexpr (kAmax) record_amax(m, amax);
}

// scale = (max(history) / FP8_MAX) / 2^margin, at least 1e-12, NaN kept.
// One workgroup: a strided maximum per lane, then across the workgroup.  The
// running maximum starts at 0: a history whose maximum is at most 0 gives
// the floor either way.  `clear`, when not null, is a history slot that is
// zeroed after every entry has been read (the slot the next amax goes to).
__global__ __launch_bounds__(kThreads) void scale_from_history(const float* hist, int32_t len, bool e5m2,
                                                               int32_t margin, float* __restrict__ scale,
                                                               uint32_t* clear) {
  __shared__ float s_peak[kThreads / 64];
  __shared__ int s_nan[kThreads / 64];
  float peak = 0.0f;
  int nan = 0;
  for (int i = threadIdx.x; i < len; i += kThreads) {
    const float h = hist[i];
    nan |= __builtin_isnan(h) ? 1 : 0;
    peak = h > peak ? h : peak;                                  // false for NaN
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float o = __shfl_xor(peak, off);
    peak = o > peak ? o : peak;
    nan |= __shfl_xor(nan, off);
  }
  if (threadIdx.x % 64 == 0) {
    s_peak[threadIdx.x / 64] = peak;
    s_nan[threadIdx.x / 64] = nan;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  for (int w = 1; w < kThreads / 64; ++w) {
    peak = s_peak[w] > peak ? s_peak[w] : peak;
    nan |= s_nan[w];
  }
  float s = peak / fp8_max(e5m2);
  s = s / __builtin_ldexpf(1.0f, margin);
  *scale = nan ? __builtin_nanf("") : (s < 1e-12f ? 1e-12f : s);
  if (clear != nullptr) *clear = 0u;                             // every lane's reads are behind the barrier
}

// Decode: unit u = 8 codes -> 8 bf16, bf16_rne(fp32_rne(code * scale)), a
// NaN result 0x7FC0 with the code's sign.
template <bool kE5M2>
__global__ __launch_bounds__(kThreads) void tensor_dequant(const u32x2* __restrict__ codes, uint32_t nunits,
                                                           const float* __restrict__ scale, u32x4* __restrict__ out) {
  u32x2 c[kUnits];
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = blockIdx.x * kSpan + j * kThreads + threadIdx.x;
    c[j] = u < nunits ? __builtin_nontemporal_load(codes + u) : u32x2{0u, 0u};
  }
  const float S = *scale;
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = blockIdx.x * kSpan + j * kThreads + threadIdx.x;
    if (u >= nunits) break;
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t w = c[j][h];
      f32x2 lo, hi;
      if constexpr (kE5M2) {
        lo = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, 1.0f, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(w, 1.0f, true);
      } else {
        lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, true);
      }
      o[2 * h] = fix_nan_pair(pack_bf16x2(lo[0] * S, lo[1] * S), (w >> 7) & 1u, (w >> 15) & 1u);
      o[2 * h + 1] = fix_nan_pair(pack_bf16x2(hi[0] * S, hi[1] * S), (w >> 23) & 1u, w >> 31);
    }
    __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, out + u);
  }
}

dim3 grid_of(uint32_t nunits) { return dim3((nunits + kSpan - 1) / kSpan); }

// Grid of a kernel that records an amax.
dim3 red_grid_of(uint32_t nunits) {
  const uint32_t b = (nunits + kRedThreads * kUnits - 1) / (kRedThreads * kUnits);
  return dim3(b < (uint32_t)kRedBlocks ? b : (uint32_t)kRedBlocks);
}

}  // namespace

hipError_t launch_tensor_amax(const void* src, int64_t n, float* amax, hipStream_t stream) {
  uint32_t* a = reinterpret_cast<uint32_t*>(amax);
  zero_u32<<<1, 1, 0, stream>>>(a);
  const uint32_t nunits = (uint32_t)(n / 8);
  if (nunits > 0) tensor_amax<<<red_grid_of(nunits), kRedThreads, 0, stream>>>(static_cast<const u32x4*>(src), nunits, a);
  return hipGetLastError();
}

// The quantization proper; `amax`, when not null, must already be zero.
static hipError_t quant_kernels(const void* src, int64_t n, int fmt, const float* scale, void* codes, float* amax,
                                hipStream_t stream) {
  uint32_t* a = reinterpret_cast<uint32_t*>(amax);
  const uint32_t nunits = (uint32_t)(n / 8);
  if (nunits == 0) return hipGetLastError();
  auto s = static_cast<const u32x4*>(src);
  auto c = static_cast<u32x2*>(codes);
  const bool e5 = fmt == LP_FP8T_E5M2;
  if (a != nullptr) {
    if (e5) tensor_quant<true, true><<<red_grid_of(nunits), kRedThreads, 0, stream>>>(s, nunits, scale, c, a);
    else tensor_quant<false, true><<<red_grid_of(nunits), kRedThreads, 0, stream>>>(s, nunits, scale, c, a);
  } else {
    if (e5) tensor_quant<true, false><<<grid_of(nunits), kThreads, 0, stream>>>(s, nunits, scale, c, a);
    else tensor_quant<false, false><<<grid_of(nunits), kThreads, 0, stream>>>(s, nunits, scale, c, a);
  }
  return hipGetLastError();
}

hipError_t launch_tensor_quant(const void* src, int64_t n, int fmt, const float* scale, void* codes, float* amax,
                               hipStream_t stream) {
  if (amax != nullptr) zero_u32<<<1, 1, 0, stream>>>(reinterpret_cast<uint32_t*>(amax));
  return quant_kernels(src, n, fmt, scale, codes, amax, stream);
}

hipError_t launch_scale_from_history(const float* hist, int32_t len, int fmt, int32_t margin, float* scale,
                                     hipStream_t stream) {
  scale_from_history<<<1, kThreads, 0, stream>>>(hist, len, fmt == LP_FP8T_E5M2, margin, scale, nullptr);
  return hipGetLastError();
}

hipError_t launch_tensor_quant_delayed(const void* src, int64_t n, int fmt, float* hist, int32_t len, int32_t slot,
                                       int32_t margin, void* codes, float* scale, hipStream_t stream) {
  uint32_t* rec = reinterpret_cast<uint32_t*>(hist + slot);
  scale_from_history<<<1, kThreads, 0, stream>>>(hist, len, fmt == LP_FP8T_E5M2, margin, scale, rec);
  return quant_kernels(src, n, fmt, scale, codes, hist + slot, stream);
}

hipError_t launch_tensor_dequant(const lp_qtensor& t, void* dst, hipStream_t stream) {
  const uint32_t nunits = (uint32_t)(t.batch * t.rows * t.cols / 8);
  if (nunits == 0) return hipSuccess;
  auto c = static_cast<const u32x2*>(t.codes);
  auto o = static_cast<u32x4*>(dst);
  if (t.fmt == LP_FP8T_E5M2)
    tensor_dequant<true><<<grid_of(nunits), kThreads, 0, stream>>>(c, nunits, t.tensor_scale, o);
  else
    tensor_dequant<false><<<grid_of(nunits), kThreads, 0, stream>>>(c, nunits, t.tensor_scale, o);
  return hipGetLastError();
}

}  // namespace lp
