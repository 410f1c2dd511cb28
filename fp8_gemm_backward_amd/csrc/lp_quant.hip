// Dynamic MX quantization of bf16 (HBM-bound, bit-exact).
//
// "perf: defer mxfp8 backward quantization", MXFP8GMMFunction.op_dx and
// MXFP8MatMul.backward: the backward re-quantizes the gradient along its
// last axis and the weight along its reduction axis, one E8M0 scale per 32
// elements (group_sizes [1, 1, 32]).
//
// The element arithmetic (block amax, E8M0 scale, saturating nearest-even
// conversion) is in lp_mxq.hpp.
#include <type_traits>

#include "lp_device.hpp"
#include "lp_internal.hpp"
#include "lp_mxq.hpp"

namespace lp {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxQuantGroups = 1024;          // groups of a grouped weight (the API's limit)
constexpr uint32_t kRowsGroupsGrid = 2048;     // workgroups of the filtered-group quantizer

// Axis -1: the work unit is eight consecutive elements (16 bytes of bf16);
// the four lanes of a quad hold one 32-element block and take its amax
// with two DPP exchanges inside the quad.  Lane i of a wave takes unit
// base + i, so every load and code store of a wave covers one contiguous
// span; each thread handles kUnits units, spaced a workgroup apart, with
// all loads issued first; codes are written with nontemporal stores.
constexpr int kUnits = 4;
constexpr int kSpan = kThreads * kUnits;

__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  return v;
}

template <bool kFp4>
__global__ __launch_bounds__(kThreads) void mx_quant_cols(const u32x4* __restrict__ src,
                                                          std::conditional_t<kFp4, uint32_t, u32x2>* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, uint32_t nunits) {
  u32x4 v[kUnits];
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = blockIdx.x * kSpan + j * kThreads + threadIdx.x;
    v[j] = u < nunits ? __builtin_nontemporal_load(src + u) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = blockIdx.x * kSpan + j * kThreads + threadIdx.x;
    uint32_t amax = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t w = v[j][k] & 0x7FFF7FFFu;
      amax = umax(amax, umax(w & 0xFFFFu, w >> 16));
    }
    amax = quad_max(amax);                                 // all four lanes of the quad agree
    if (u >= nunits) continue;                             // whole quads drop out together
    const BlockScale s = block_scale<kFp4>(amax);
    if ((threadIdx.x & 3) == 0) scales[u >> 2] = (uint8_t)s.byte;
    if constexpr (!kFp4) {
      const E4M3Scale q = e4m3_scale(s.byte);
      uint32_t o[2];
#pragma unroll
      for (int k = 0; k < 4; k += 2) {
        const uint32_t w0 = v[j][k], w1 = v[j][k + 1];
        const uint32_t c = e4m3x2_scaled<true>(e4m3x2_scaled<false>(w0, w0, q), w1, q);
        o[k / 2] = s.bad ? (nan_e4m3x2(w0) | (nan_e4m3x2(w1) << 16)) : c;
      }
      __builtin_nontemporal_store(u32x2{o[0], o[1]}, codes + u);
    } else {
      uint32_t o = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) o |= to_e2m1x2(bf16_lo(v[j][k]) * s.inv, bf16_hi(v[j][k]) * s.inv) << (8 * k);
      __builtin_nontemporal_store(s.bad ? 0u : o, codes + u);
    }
  }
}

// Axis -2: thread i owns a strip of 32 rows x 8 columns; every column is its
// own scale block, so the amax is lane-local and consecutive lanes read
// consecutive 16-byte column chunks of each row.
template <bool kFp4>
__global__ __launch_bounds__(kThreads) void mx_quant_rows(const uint16_t* __restrict__ src,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales, uint32_t nstrips,
                                                          FastDiv strips_per_row, uint32_t cols) {
  uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= nstrips) return;
  uint32_t rb = fdiv(i, strips_per_row);                 // block of 32 rows over batch*rows
  uint32_t c0 = (i - rb * strips_per_row.d) * 8u;
  const uint16_t* base = src + (size_t)rb * 32u * cols + c0;
  u32x4 v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) v[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (size_t)r * cols));
  uint32_t amax[4] = {0, 0, 0, 0};   // packed pairs of column maxima
#pragma unroll
  for (int r = 0; r < 32; ++r)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t w = v[r][k] & 0x7FFF7FFFu;
      amax[k] = umax(amax[k] & 0xFFFFu, w & 0xFFFFu) | (umax(amax[k] >> 16, w >> 16) << 16);
    }
  BlockScale s[8];
  uint32_t sbytes[2] = {0, 0};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    s[c] = block_scale<kFp4>((amax[c >> 1] >> (16 * (c & 1))) & 0xFFFFu);
    sbytes[c >> 2] |= s[c].byte << (8 * (c & 3));
  }
  *reinterpret_cast<u32x2*>(scales + (size_t)rb * cols + c0) = u32x2{sbytes[0], sbytes[1]};
  uint8_t* out = codes + (size_t)rb * 32u * (kFp4 ? cols / 2 : cols) + (kFp4 ? c0 / 2 : c0);
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    if constexpr (!kFp4) {
      uint32_t o[2];
#pragma unroll
      for (int k = 0; k < 4; k += 2) {
        uint32_t w0 = v[r][k], w1 = v[r][k + 1];
        int c = 2 * k;
        uint32_t p0 = to_e4m3x2(bf16_lo(w0) * s[c].inv, bf16_hi(w0) * s[c + 1].inv);
        uint32_t p1 = to_e4m3x2(bf16_lo(w1) * s[c + 2].inv, bf16_hi(w1) * s[c + 3].inv);
        uint32_t b0 = s[c].bad ? (0x7Fu | ((w0 >> 8) & 0x80u)) : (p0 & 0xFFu);
        uint32_t b1 = s[c + 1].bad ? (0x7Fu | ((w0 >> 24) & 0x80u)) : (p0 >> 8);
        uint32_t b2 = s[c + 2].bad ? (0x7Fu | ((w1 >> 8) & 0x80u)) : (p1 & 0xFFu);
        uint32_t b3 = s[c + 3].bad ? (0x7Fu | ((w1 >> 24) & 0x80u)) : (p1 >> 8);
        o[k / 2] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
      }
      *reinterpret_cast<u32x2*>(out + (size_t)r * cols) = u32x2{o[0], o[1]};
    } else {
      uint32_t o = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t w = v[r][k];
        int c = 2 * k;
        uint32_t b = to_e2m1x2(bf16_lo(w) * s[c].inv, bf16_hi(w) * s[c + 1].inv);
        uint32_t lo = s[c].bad ? 0u : (b & 0xFu);
        uint32_t hi = s[c + 1].bad ? 0u : (b >> 4);
        o |= (lo | (hi << 4)) << (8 * k);
      }
      *reinterpret_cast<uint32_t*>(out + (size_t)r * (cols / 2)) = o;
    }
  }
}

// Tiled form for cols % 32 == 0, used for axis -2 and for both axes at once
// ("perf: defer mxfp8 backward quantization", MXFP8MatMul.backward,
// npu_dynamic_mx_quant_with_dual_axis: one read of the bf16 tensor, two
// quantized copies).  Sixteen lanes own a 32 x 32 tile, lane l = c + 4 r
// holding rows 8 r .. 8 r + 7 and columns 8 c .. 8 c + 7 (16 bytes a row),
// and the four 16-lane groups of a wave own consecutive tiles of a row of
// tiles, so that each load covers 256 contiguous bytes of four rows.  A
// column's amax over the tile's 32 rows combines the four lanes with its
// column strip (DPP row rotations by 4 and 8); a row's amax over 32 columns
// combines the lanes of a quad (quad permutations).  Four times as many
// threads as a 32 x 8 strip per thread, and a quarter of the registers.
// One 32 x 32 tile (index `tile` over batch * rows / 32 row blocks of
// tiles_per_row tiles each) by the 16 lanes of the calling lane group.
template <bool kFp4, bool kDual>
__device__ __forceinline__ void quant_tile32(const uint16_t* __restrict__ src, uint8_t* __restrict__ codes_c,
                                             uint8_t* __restrict__ scales_c, uint8_t* __restrict__ codes_r,
                                             uint8_t* __restrict__ scales_r, uint32_t tile, FastDiv tiles_per_row,
                                             uint32_t cols) {
  const uint32_t l16 = threadIdx.x & 15, ci = l16 & 3, ri = l16 >> 2;
  const uint32_t rb = fdiv(tile, tiles_per_row);         // block of 32 rows over batch*rows
  const uint32_t tc = tile - rb * tiles_per_row.d;       // block of 32 columns
  const uint32_t c0 = 32u * tc + 8u * ci;
  const size_t row0 = (size_t)rb * 32u + 8u * ri;
  const uint16_t* base = src + row0 * cols + c0;
  u32x4 v[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) v[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (size_t)r * cols));

  // Blocks along the rows (axis -2): column maxima over this lane's 8 rows,
  // then over the 4 lanes of the column strip.
  uint32_t cm[4] = {0, 0, 0, 0};
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int k = 0; k < 4; ++k) cm[k] = pk_umax16(cm[k], v[r][k] & 0x7FFF7FFFu);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    cm[k] = pk_umax16(cm[k], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cm[k], 0x124, 0xF, 0xF, false));  // row_ror:4
    cm[k] = pk_umax16(cm[k], (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cm[k], 0x128, 0xF, 0xF, false));  // row_ror:8
  }
  BlockScale s[8];
  uint32_t sbytes[2] = {0, 0};
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    s[c] = block_scale<kFp4>((cm[c >> 1] >> (16 * (c & 1))) & 0xFFFFu);
    sbytes[c >> 2] |= s[c].byte << (8 * (c & 3));
  }
  if (ri == 0) *reinterpret_cast<u32x2*>(scales_r + (size_t)rb * cols + c0) = u32x2{sbytes[0], sbytes[1]};
  const size_t row_bytes = kFp4 ? cols / 2 : cols;
  uint8_t* out_r = codes_r + row0 * row_bytes + (kFp4 ? c0 / 2 : c0);
  if constexpr (!kFp4) {
    // E4M3 along the rows, two rows at a time: column c's elements of rows
    // r and r + 1 form one pair under column c's scale, so each conversion
    // takes one scale; byte permutes then regroup the codes by row.  A block
    // with a NaN or an infinity (any in the wave: a uniform branch) gets the
    // NaN codes afterwards.
    E4M3Scale q[8];
    uint32_t badc = 0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      q[c] = e4m3_scale(s[c].byte);
      badc |= (s[c].bad ? 1u : 0u) << c;
    }
    const bool anybad = __builtin_amdgcn_ballot_w64(badc != 0) != 0;
#pragma unroll
    for (int r = 0; r < 8; r += 2) {
      uint32_t x[4];                      // x[k]: bytes (r, 2k), (r+1, 2k), (r, 2k+1), (r+1, 2k+1)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t pe = __builtin_amdgcn_perm(v[r + 1][k], v[r][k], 0x05040100u);   // column 2k, rows r, r+1
        const uint32_t po = __builtin_amdgcn_perm(v[r + 1][k], v[r][k], 0x07060302u);   // column 2k+1
        x[k] = e4m3x2_scaled<false>(pe, pe, q[2 * k]);
        x[k] = e4m3x2_scaled<true>(x[k], po, q[2 * k + 1]);
        if (__builtin_expect(anybad, false)) {
          if ((badc >> (2 * k)) & 1u) x[k] = (x[k] & 0xFFFF0000u) | nan_e4m3x2(pe);
          if ((badc >> (2 * k + 1)) & 1u) x[k] = (x[k] & 0xFFFFu) | (nan_e4m3x2(po) << 16);
        }
      }
      const u32x2 lo = {__builtin_amdgcn_perm(x[1], x[0], 0x06040200u), __builtin_amdgcn_perm(x[3], x[2], 0x06040200u)};
      const u32x2 hi = {__builtin_amdgcn_perm(x[1], x[0], 0x07050301u), __builtin_amdgcn_perm(x[3], x[2], 0x07050301u)};
      __builtin_nontemporal_store(lo, reinterpret_cast<u32x2*>(out_r + (size_t)r * row_bytes));
      __builtin_nontemporal_store(hi, reinterpret_cast<u32x2*>(out_r + (size_t)(r + 1) * row_bytes));
    }
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      uint32_t o = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w = v[r][k];
        const int c = 2 * k;
        const uint32_t b = to_e2m1x2(bf16_lo(w) * s[c].inv, bf16_hi(w) * s[c + 1].inv);
        const uint32_t lo = s[c].bad ? 0u : (b & 0xFu);
        const uint32_t hi = s[c + 1].bad ? 0u : (b >> 4);
        o |= (lo | (hi << 4)) << (8 * k);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<uint32_t*>(out_r + (size_t)r * row_bytes));
    }
  }
  if constexpr (kDual) {
    // Blocks along the columns (axis -1): each of the 8 rows over the quad.
    uint8_t* out_c = codes_c + row0 * row_bytes + (kFp4 ? c0 / 2 : c0);
    uint8_t* sc_c = scales_c + row0 * (cols / 32) + tc;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      uint32_t m = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) m = pk_umax16(m, v[r][k] & 0x7FFF7FFFu);
      m = umax(m & 0xFFFFu, m >> 16);
      const BlockScale sr = block_scale<kFp4>(quad_max(m));
      if (ci == (uint32_t)(r >> 1)) sc_c[(size_t)r * (cols / 32)] = (uint8_t)sr.byte;   // two rows per lane
      if constexpr (!kFp4) {
        // E4M3 along the columns: the row's one scale for all eight values.
        const E4M3Scale q = e4m3_scale(sr.byte);
        uint32_t o[2];
#pragma unroll
        for (int k = 0; k < 4; k += 2) {
          const uint32_t w0 = v[r][k], w1 = v[r][k + 1];
          const uint32_t c = e4m3x2_scaled<true>(e4m3x2_scaled<false>(w0, w0, q), w1, q);
          o[k / 2] = sr.bad ? (nan_e4m3x2(w0) | (nan_e4m3x2(w1) << 16)) : c;
        }
        __builtin_nontemporal_store(u32x2{o[0], o[1]}, reinterpret_cast<u32x2*>(out_c + (size_t)r * row_bytes));
      } else {
        uint32_t o = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) o |= to_e2m1x2(bf16_lo(v[r][k]) * sr.inv, bf16_hi(v[r][k]) * sr.inv) << (8 * k);
        __builtin_nontemporal_store(sr.bad ? 0u : o, reinterpret_cast<uint32_t*>(out_c + (size_t)r * row_bytes));
      }
    }
  }
}

template <bool kFp4, bool kDual>
__global__ __launch_bounds__(kThreads) void mx_quant_tile(const uint16_t* __restrict__ src,
                                                          uint8_t* __restrict__ codes_c, uint8_t* __restrict__ scales_c,
                                                          uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
                                                          uint32_t ntiles, FastDiv tiles_per_row, uint32_t cols) {
  const uint32_t tile = (blockIdx.x * kThreads + threadIdx.x) >> 4;
  if (tile >= ntiles) return;                            // whole 16-lane groups
  quant_tile32<kFp4, kDual>(src, codes_c, scales_c, codes_r, scales_r, tile, tiles_per_row, cols);
}

// MXFP8 quantization along the rows (-2) of a grouped weight [G][N][K], for
// the groups with more than min_rows rows only (the others quantize their
// weight inside the grad_X product).  The first wave lists those groups in
// LDS from the int32 cumulative ends, with the kernels' clamping
// (end_g = min(max(0, o_0 .. o_g), M)); the workgroups then stride over the
// listed groups' tiles, 16 tiles (one per 16 lanes) per step.  A grid that
// covered every group's tiles and let the unlisted ones exit spent most of
// its time dispatching workgroups that do nothing.
__global__ __launch_bounds__(kThreads) void mx_quant_rows_groups(const uint16_t* __restrict__ src,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales,
                                                                 const int32_t* __restrict__ offsets, int32_t M,
                                                                 int32_t groups, int32_t min_rows,
                                                                 uint32_t tiles_per_group, FastDiv tiles_per_row,
                                                                 uint32_t cols) {
  __shared__ int32_t s_list[kMaxQuantGroups];
  __shared__ int32_t s_n;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0, n = 0;                                  // end of the previous chunk's last group; listed so far
    for (int base = 0; base < groups; base += 64) {
      const int j = base + lane;
      int m = j < groups ? offsets[j] : 0;
      m = m > 0 ? m : 0;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {                   // inclusive running maximum across the lanes
        const int up = __shfl_up(m, d);
        if (lane >= d) m = up > m ? up : m;
      }
      int end = m > carry ? m : carry;
      end = end < M ? end : M;
      int prev = __shfl_up(end, 1);
      if (lane == 0) prev = carry < M ? carry : M;
      const bool listed = j < groups && end - prev > min_rows;
      const uint64_t mask = __ballot(listed);
      if (listed) s_list[n + __popcll(mask & ((1ull << lane) - 1))] = j;
      n += __popcll(mask);
      carry = __shfl(end, 63);
    }
    if (lane == 0) s_n = n;
  }
  __syncthreads();
  const uint32_t steps = (tiles_per_group + kThreads / 16 - 1) / (kThreads / 16);   // steps per group
  const uint32_t total = (uint32_t)s_n * steps;
  for (uint32_t c = blockIdx.x; c < total; c += gridDim.x) {
    const uint32_t li = c / steps;
    const uint32_t t = (c - li * steps) * (kThreads / 16) + (threadIdx.x >> 4);
    if (t < tiles_per_group)
      quant_tile32<false, false>(src, nullptr, nullptr, codes, scales, (uint32_t)s_list[li] * tiles_per_group + t,
                                 tiles_per_row, cols);
  }
}

}  // namespace

hipError_t launch_mx_quant_rows_groups(const void* src, int64_t groups, int64_t rows, int64_t cols,
                                       const int32_t* offsets, int64_t M, int64_t min_rows, void* codes, void* scales,
                                       hipStream_t stream) {
  if (groups * rows * cols == 0) return hipSuccess;
  const uint32_t tpr = (uint32_t)(cols / 32);
  const uint32_t tpg = (uint32_t)(rows / 32) * tpr;
  // Enough workgroups to keep every compute unit streaming; each strides
  // over the listed groups' tiles.
  const uint64_t steps = (uint64_t)groups * ((tpg + kThreads / 16 - 1) / (kThreads / 16));
  const dim3 grid((uint32_t)(steps < kRowsGroupsGrid ? steps : kRowsGroupsGrid)), block(kThreads);
  mx_quant_rows_groups<<<grid, block, 0, stream>>>(static_cast<const uint16_t*>(src), static_cast<uint8_t*>(codes),
                                                   static_cast<uint8_t*>(scales), offsets, (int32_t)M,
                                                   (int32_t)groups, (int32_t)min_rows, tpg, make_fastdiv(tpr),
                                                   (uint32_t)cols);
  return hipGetLastError();
}

hipError_t launch_mx_quant(const void* src, int64_t batch, int64_t rows, int64_t cols, int axis, int dst_fmt,
                           void* codes, void* scales, hipStream_t stream) {
  const int64_t n = batch * rows * cols;
  if (n == 0) return hipSuccess;
  const bool fp4 = dst_fmt == LP_MXFP4;
  if (axis == -1) {
    const uint32_t nunits = (uint32_t)(n / 8);
    const dim3 grid((nunits + kSpan - 1) / kSpan), block(kThreads);
    auto s = static_cast<const u32x4*>(src);
    auto sc = static_cast<uint8_t*>(scales);
    if (fp4)
      mx_quant_cols<true><<<grid, block, 0, stream>>>(s, static_cast<uint32_t*>(codes), sc, nunits);
    else
      mx_quant_cols<false><<<grid, block, 0, stream>>>(s, static_cast<u32x2*>(codes), sc, nunits);
  } else if (cols % 32 == 0) {
    const uint32_t tpr = (uint32_t)(cols / 32);
    const uint32_t ntiles = (uint32_t)(batch * (rows / 32) * tpr);
    const dim3 grid((ntiles * 16 + kThreads - 1) / kThreads), block(kThreads);
    auto s = static_cast<const uint16_t*>(src);
    auto c = static_cast<uint8_t*>(codes);
    auto sc = static_cast<uint8_t*>(scales);
    if (fp4)
      mx_quant_tile<true, false><<<grid, block, 0, stream>>>(s, nullptr, nullptr, c, sc, ntiles, make_fastdiv(tpr),
                                                              (uint32_t)cols);
    else
      mx_quant_tile<false, false><<<grid, block, 0, stream>>>(s, nullptr, nullptr, c, sc, ntiles, make_fastdiv(tpr),
                                                               (uint32_t)cols);
  } else {
    const uint32_t spr = (uint32_t)(cols / 8);
    const uint32_t nstrips = (uint32_t)(batch * (rows / 32) * spr);
    const dim3 grid((nstrips + kThreads - 1) / kThreads), block(kThreads);
    auto s = static_cast<const uint16_t*>(src);
    auto c = static_cast<uint8_t*>(codes);
    auto sc = static_cast<uint8_t*>(scales);
    if (fp4)
      mx_quant_rows<true><<<grid, block, 0, stream>>>(s, c, sc, nstrips, make_fastdiv(spr), (uint32_t)cols);
    else
      mx_quant_rows<false><<<grid, block, 0, stream>>>(s, c, sc, nstrips, make_fastdiv(spr), (uint32_t)cols);
  }
  return hipGetLastError();
}

hipError_t launch_mx_quant_dual(const void* src, int64_t batch, int64_t rows, int64_t cols, int dst_fmt,
                                void* codes_c, void* scales_c, void* codes_r, void* scales_r, hipStream_t stream) {
  const int64_t n = batch * rows * cols;
  if (n == 0) return hipSuccess;
  const uint32_t tpr = (uint32_t)(cols / 32);
  const uint32_t ntiles = (uint32_t)(batch * (rows / 32) * tpr);
  const dim3 grid((ntiles * 16 + kThreads - 1) / kThreads), block(kThreads);
  auto s = static_cast<const uint16_t*>(src);
  auto cc = static_cast<uint8_t*>(codes_c);
  auto scc = static_cast<uint8_t*>(scales_c);
  auto cr = static_cast<uint8_t*>(codes_r);
  auto scr = static_cast<uint8_t*>(scales_r);
  if (dst_fmt == LP_MXFP4)
    mx_quant_tile<true, true><<<grid, block, 0, stream>>>(s, cc, scc, cr, scr, ntiles, make_fastdiv(tpr), (uint32_t)cols);
  else
    mx_quant_tile<false, true><<<grid, block, 0, stream>>>(s, cc, scc, cr, scr, ntiles, make_fastdiv(tpr), (uint32_t)cols);
  return hipGetLastError();
}

}  // namespace lp
