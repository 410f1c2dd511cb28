// Internal interface between the C-ABI layer (lp_api.hip) and the kernel
// translation units.  Not installed; callers use include/lp.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lp.h"

namespace lp {

// Unsigned division by a divisor fixed at launch (Granlund & Montgomery,
// "Division by invariant integers using multiplication", round-up variant):
// q = (umulhi(n, magic) + n) >> shift, exact for n, d < 2^31.
struct FastDiv {
  uint32_t d, magic, shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shift = s;
  f.magic = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  uint32_t t = __umulhi(n, f.magic);
  return (t + n) >> f.shift;
}

// Launchers; each returns hipSuccess or the launch error.  Arguments were
// validated by the caller.
hipError_t launch_dequant(const lp_qtensor& src, void* dst, hipStream_t stream);
hipError_t launch_mx_quant(const void* src, int64_t batch, int64_t rows, int64_t cols, int axis,
                           int dst_fmt, void* codes, void* scales, hipStream_t stream);
hipError_t launch_mx_quant_dual(const void* src, int64_t batch, int64_t rows, int64_t cols, int dst_fmt,
                                void* codes_c, void* scales_c, void* codes_r, void* scales_r, hipStream_t stream);
// Per-tensor scaled FP8 (lp_tensor.hip).  n is a multiple of 8; amax may be
// null in launch_tensor_quant.
hipError_t launch_tensor_amax(const void* src, int64_t n, float* amax, hipStream_t stream);
hipError_t launch_tensor_quant(const void* src, int64_t n, int fmt, const float* scale, void* codes, float* amax,
                               hipStream_t stream);
hipError_t launch_scale_from_history(const float* hist, int32_t len, int fmt, int32_t margin, float* scale,
                                     hipStream_t stream);
hipError_t launch_tensor_dequant(const lp_qtensor& t, void* dst, hipStream_t stream);
// Scale from hist (then hist[slot] cleared), quantization with that scale,
// the input's amax into hist[slot].
hipError_t launch_tensor_quant_delayed(const void* src, int64_t n, int fmt, float* hist, int32_t len, int32_t slot,
                                       int32_t margin, void* codes, float* scale, hipStream_t stream);

// One backward contraction (grad_X or grad_W) over `groups` groups.
//   dx: C[m][k] = sum_n grad[m][n] * W[g][n][k]  (groups partition the rows m)
//   dw: C[g][n][k] = sum_m grad[m][n] * X[m][k]  (groups partition the sum over m)
// offsets == nullptr means one group spanning all M rows.
struct GemmCall {
  bool dw;
  const lp_qtensor* grad;
  const lp_qtensor* other;  // W for dx, X for dw
  const int32_t* offsets;
  int32_t groups;
  int64_t M, N, K;
  void* out;
  void* ws;                 // workspace for split contractions, or nullptr
  size_t ws_bytes;
  int32_t fuse_rows = 0;    // grouped dX: groups of at most this many rows are
  int32_t fuse_side = 0;    // left out (1) or the only ones (2); 0: all groups
};
hipError_t launch_gemm(const GemmCall& call, hipStream_t stream);

// Forward y[m][n] = sum_k x[m][k] w[g][n][k] (groups partition the rows m;
// offsets == nullptr: one group).  x and w are both MXFP4 or both MXFP8,
// scaled along k.
hipError_t launch_fwd(const lp_qtensor& x, const lp_qtensor& w, const int32_t* offsets, int32_t groups, void* y,
                      hipStream_t stream);

// grad_X then grad_W of one call (same gradient); per-tensor FP8 operands
// run both in one launch.
hipError_t launch_gemm_pair(const GemmCall& dx, const GemmCall& dw, hipStream_t stream);

// Workspace bytes the contraction would use to split its contraction
// (0: it does not split).
size_t gemm_workspace_bytes(const GemmCall& call);

// grad_X of the deferred MXFP8 recipe: grad (MXFP8, scales along -1)
// [M][N] times the bf16 weight w [G][N][K] quantized to MXFP8 along N.
// Groups of at most fuse_rows rows quantize their weight inside the
// product; the others' weights are first quantized into w_codes / w_scales
// ([G][N][K], [G][N/32][K]; unused when fuse_rows >= M).
hipError_t launch_grouped_dx_deferred(const lp_qtensor& grad, const void* w, int64_t K, const int32_t* offsets,
                                      int32_t groups, int64_t fuse_rows, void* w_codes, void* w_scales,
                                      void* grad_x, hipStream_t stream);
// MXFP8 quantization along the rows of w [G][N][K] for the groups of more
// than min_rows rows (lp_quant.hip).
hipError_t launch_mx_quant_rows_groups(const void* src, int64_t groups, int64_t rows, int64_t cols,
                                       const int32_t* offsets, int64_t M, int64_t min_rows, void* codes, void* scales,
                                       hipStream_t stream);

}  // namespace lp
