// C-ABI entry points: argument checking, then one launch per contraction.
// Every rule checked here is stated next to the entry point in lp.h.
#include <stdint.h>

#include <mutex>

#include "lp_internal.hpp"

namespace {

constexpr int64_t kMaxUnits = (int64_t)1 << 31;    // kernels index 8-element units in 32 bits
constexpr int64_t kMaxDim = ((int64_t)1 << 31) - 1;
constexpr int64_t kMaxTiles = (int64_t)1 << 30;    // output tiles of one launch, counted in 32 bits
// Products: a tile's 256 rows of any operand span fewer than 2^31 bytes (the
// kernels address them with 32-bit offsets and buffer windows), and the
// contraction of grad_W (the token rows) runs a few slabs past its end in
// 32-bit arithmetic.
constexpr int64_t kMaxProductCols = (int64_t)1 << 22;
constexpr int64_t kMaxProductRows = (int64_t)1 << 30;

// Element count of a [b][r][c] tensor (each size in [0, kMaxDim]) into *n;
// false when it reaches 8 kMaxUnits.  r c stays below 2^62, and the product
// with b is only formed once it is known to fit.
bool count_ok(int64_t b, int64_t r, int64_t c, int64_t* n) {
  const int64_t rc = r * c;
  if (rc != 0 && b > (8 * kMaxUnits - 1) / rc) return false;
  *n = b * rc;
  return true;
}

// Output tiles of a result with `cols` columns whose rows make at most
// `row_tiles` row tiles of 128, an upper bound for every tile shape the
// kernels use (at least 128 x 128): the launches count them in 32 bits.
// row_tiles < 2^35 here, so the product cannot overflow.
bool tiles_ok(int64_t row_tiles, int64_t cols) { return row_tiles * (cols / 128 + 1) <= kMaxTiles; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool is_fp4(int f) { return f == LP_MXFP4 || f == LP_NVFP4; }
bool is_fp8t(int f) { return f == LP_FP8T_E4M3 || f == LP_FP8T_E5M2; }
bool has_tensor_scale(int f) { return f == LP_NVFP4 || is_fp8t(f); }
bool has_block_scales(int f) { return f != LP_BF16 && !is_fp8t(f); }

// Shape, pointer and alignment checks of one operand tensor.
lp_status check_tensor(const lp_qtensor* t) {
  if (t == nullptr) return LP_ERR_NULL;
  if (t->fmt < LP_BF16 || t->fmt > LP_FP8T_E5M2) return LP_ERR_FORMAT;
  if (t->batch < 0 || t->rows < 0 || t->cols < 0) return LP_ERR_SHAPE;
  if (t->rows > kMaxDim || t->cols > kMaxDim || t->batch > kMaxDim) return LP_ERR_SHAPE;
  const int axis = has_block_scales(t->fmt) ? t->scale_axis : -1;
  if (axis != -1 && axis != -2) return LP_ERR_FORMAT;
  if (axis == -2 && t->fmt != LP_MXFP8) return LP_ERR_FORMAT;
  if (t->cols % 16) return LP_ERR_SHAPE;
  if ((t->fmt == LP_MXFP4 || (t->fmt == LP_MXFP8 && axis == -1)) && t->cols % 32) return LP_ERR_SHAPE;
  if (t->fmt == LP_MXFP8 && axis == -2 && t->rows % 32) return LP_ERR_SHAPE;
  int64_t n = 0;
  if (!count_ok(t->batch, t->rows, t->cols, &n)) return LP_ERR_SHAPE;
  if (n == 0) return LP_OK;
  if (t->codes == nullptr) return LP_ERR_NULL;
  if (has_block_scales(t->fmt) && t->scales == nullptr) return LP_ERR_NULL;
  if (has_tensor_scale(t->fmt) && t->tensor_scale == nullptr) return LP_ERR_NULL;
  if (!aligned(t->codes, 16)) return LP_ERR_ALIGN;
  if (has_block_scales(t->fmt) && !aligned(t->scales, 16)) return LP_ERR_ALIGN;
  if (has_tensor_scale(t->fmt) && !aligned(t->tensor_scale, 4)) return LP_ERR_ALIGN;
  return LP_OK;
}

lp_status hip_status(hipError_t e) { return e == hipSuccess ? LP_OK : LP_ERR_HIP; }

// Checks shared by the linear and grouped backward.  `groups` is 0 for the
// dense linear (then w->batch must be 1).
lp_status check_bwd(const lp_qtensor* grad, const lp_qtensor* x, const lp_qtensor* w, void* grad_x, void* grad_w,
                    int64_t groups) {
  lp_status st = check_tensor(grad);
  if (st != LP_OK) return st;
  if (grad->batch != 1) return LP_ERR_SHAPE;
  // grad_out: bf16 for every product; MXFP8 along its columns (the dX
  // contraction) for dX only; MXFP8 along its rows (the dW contraction) for a
  // dense dW of an MXFP8 input scaled along its rows, only; per-tensor FP8
  // for both products, with per-tensor FP8 operands only.
  const bool g_mx_cols = grad->fmt == LP_MXFP8 && grad->scale_axis == -1;
  const bool g_mx_rows = grad->fmt == LP_MXFP8 && grad->scale_axis == -2;
  const bool g_t = is_fp8t(grad->fmt);
  if (grad->fmt != LP_BF16 && !g_mx_cols && !g_mx_rows && !g_t) return LP_ERR_FORMAT;
  if (g_mx_rows && (grad_x != nullptr || groups != 0)) return LP_ERR_FORMAT;
  const int64_t M = grad->rows, N = grad->cols;
  int64_t K = -1;
  if (grad_x != nullptr) {
    if ((st = check_tensor(w)) != LP_OK) return st;
    if (is_fp8t(w->fmt) != g_t) return LP_ERR_FORMAT;
    if (w->batch != (groups ? groups : 1) || w->rows != N) return LP_ERR_SHAPE;
    K = w->cols;
  }
  if (grad_w != nullptr) {
    if (g_mx_cols) return LP_ERR_FORMAT;              // its scales do not run along the dW contraction
    if ((st = check_tensor(x)) != LP_OK) return st;
    if (is_fp8t(x->fmt) != g_t) return LP_ERR_FORMAT;
    if (g_mx_rows && !(x->fmt == LP_MXFP8 && x->scale_axis == -2)) return LP_ERR_FORMAT;
    if (x->batch != 1 || x->rows != M) return LP_ERR_SHAPE;
    if (K >= 0 && x->cols != K) return LP_ERR_SHAPE;
    K = x->cols;
  }
  for (const lp_qtensor* t : {grad_x ? w : nullptr, grad_w ? x : nullptr}) {
    if (t != nullptr && is_fp4(t->fmt) && t->cols % 32) return LP_ERR_SHAPE;
  }
  if (M >= kMaxProductRows || N >= kMaxProductCols || K >= kMaxProductCols) return LP_ERR_SHAPE;
  const int64_t G = groups ? groups : 1;
  if (grad_x != nullptr && !tiles_ok(M / 128 + G + 1, K)) return LP_ERR_SHAPE;   // a partial tile per group
  if (grad_w != nullptr && !tiles_ok(G * (N / 128 + 1), K)) return LP_ERR_SHAPE;
  if (grad_x != nullptr && M * K > 0 && !aligned(grad_x, 16)) return LP_ERR_ALIGN;
  if (grad_w != nullptr && N * K > 0 && !aligned(grad_w, 16)) return LP_ERR_ALIGN;
  return LP_OK;
}

}  // namespace

extern "C" {

lp_status lp_dequant(const lp_qtensor* src, void* dst, void* stream) {
  lp_status st = check_tensor(src);
  if (st != LP_OK) return st;
  if (src->fmt == LP_BF16) return LP_ERR_FORMAT;
  if (src->batch == 0 || src->rows == 0 || src->cols == 0) return LP_OK;
  if (dst == nullptr) return LP_ERR_NULL;
  if (!aligned(dst, 16)) return LP_ERR_ALIGN;
  return hip_status(lp::launch_dequant(*src, dst, static_cast<hipStream_t>(stream)));
}

lp_status lp_mx_quant(const void* src, int64_t batch, int64_t rows, int64_t cols, int32_t axis, int32_t dst_fmt,
                      void* codes, void* scales, void* stream) {
  if (batch < 0 || rows < 0 || cols < 0 || batch > kMaxDim || rows > kMaxDim || cols > kMaxDim) return LP_ERR_SHAPE;
  if (axis != -1 && axis != -2) return LP_ERR_FORMAT;
  if (dst_fmt != LP_MXFP8 && dst_fmt != LP_MXFP4) return LP_ERR_FORMAT;
  if (axis == -1 && cols % 32) return LP_ERR_SHAPE;
  if (axis == -2 && (rows % 32 || cols % 8)) return LP_ERR_SHAPE;
  int64_t n = 0;
  if (!count_ok(batch, rows, cols, &n)) return LP_ERR_SHAPE;
  if (n == 0) return LP_OK;
  if (src == nullptr || codes == nullptr || scales == nullptr) return LP_ERR_NULL;
  if (!aligned(src, 16) || !aligned(codes, 16) || !aligned(scales, 16)) return LP_ERR_ALIGN;
  return hip_status(lp::launch_mx_quant(src, batch, rows, cols, axis, dst_fmt, codes, scales,
                                        static_cast<hipStream_t>(stream)));
}

lp_status lp_mx_quant_dual(const void* src, int64_t batch, int64_t rows, int64_t cols, int32_t dst_fmt,
                           void* codes_cols, void* scales_cols, void* codes_rows, void* scales_rows, void* stream) {
  if (batch < 0 || rows < 0 || cols < 0 || batch > kMaxDim || rows > kMaxDim || cols > kMaxDim) return LP_ERR_SHAPE;
  if (dst_fmt != LP_MXFP8 && dst_fmt != LP_MXFP4) return LP_ERR_FORMAT;
  if (rows % 32 || cols % 32) return LP_ERR_SHAPE;
  int64_t n = 0;
  if (!count_ok(batch, rows, cols, &n)) return LP_ERR_SHAPE;
  if (n == 0) return LP_OK;
  if (src == nullptr || codes_cols == nullptr || scales_cols == nullptr || codes_rows == nullptr ||
      scales_rows == nullptr)
    return LP_ERR_NULL;
  if (!aligned(src, 16) || !aligned(codes_cols, 16) || !aligned(scales_cols, 16) || !aligned(codes_rows, 16) ||
      !aligned(scales_rows, 16))
    return LP_ERR_ALIGN;
  return hip_status(lp::launch_mx_quant_dual(src, batch, rows, cols, dst_fmt, codes_cols, scales_cols, codes_rows,
                                             scales_rows, static_cast<hipStream_t>(stream)));
}

lp_status lp_tensor_amax(const void* src, int64_t n, float* amax, void* stream) {
  if (n < 0 || n % 8 || n / 8 >= kMaxUnits) return LP_ERR_SHAPE;
  if (amax == nullptr || (n > 0 && src == nullptr)) return LP_ERR_NULL;
  if (!aligned(amax, 4) || !aligned(src, 16)) return LP_ERR_ALIGN;
  return hip_status(lp::launch_tensor_amax(src, n, amax, static_cast<hipStream_t>(stream)));
}

lp_status lp_tensor_quant(const void* src, int64_t n, int32_t dst_fmt, const float* scale, void* codes, float* amax,
                          void* stream) {
  if (!is_fp8t(dst_fmt)) return LP_ERR_FORMAT;
  if (n < 0 || n % 8 || n / 8 >= kMaxUnits) return LP_ERR_SHAPE;
  if (n > 0 && (src == nullptr || codes == nullptr || scale == nullptr)) return LP_ERR_NULL;
  if (amax != nullptr && amax == scale) return LP_ERR_SHAPE;     // the amax would clear the scale first
  if (!aligned(src, 16) || !aligned(codes, 16) || !aligned(scale, 4) || !aligned(amax, 4)) return LP_ERR_ALIGN;
  return hip_status(lp::launch_tensor_quant(src, n, dst_fmt, scale, codes, amax, static_cast<hipStream_t>(stream)));
}

lp_status lp_scale_from_history(const float* history, int32_t len, int32_t fmt, int32_t margin, float* scale,
                                void* stream) {
  if (!is_fp8t(fmt)) return LP_ERR_FORMAT;
  if (len < 1 || len > 65536 || margin < -64 || margin > 64) return LP_ERR_SHAPE;
  if (history == nullptr || scale == nullptr) return LP_ERR_NULL;
  if (!aligned(history, 4) || !aligned(scale, 4)) return LP_ERR_ALIGN;
  return hip_status(lp::launch_scale_from_history(history, len, fmt, margin, scale, static_cast<hipStream_t>(stream)));
}

lp_status lp_tensor_quant_delayed(const void* src, int64_t n, int32_t dst_fmt, float* history, int32_t len,
                                  int32_t slot, int32_t margin, void* codes, float* scale, void* stream) {
  if (!is_fp8t(dst_fmt)) return LP_ERR_FORMAT;
  if (n < 0 || n % 8 || n / 8 >= kMaxUnits) return LP_ERR_SHAPE;
  if (len < 1 || len > 65536 || slot < 0 || slot >= len || margin < -64 || margin > 64) return LP_ERR_SHAPE;
  if (history == nullptr || scale == nullptr || (n > 0 && (src == nullptr || codes == nullptr))) return LP_ERR_NULL;
  if (scale >= history && scale < history + len) return LP_ERR_SHAPE;   // the scale must not live in the ring
  if (!aligned(src, 16) || !aligned(codes, 16) || !aligned(history, 4) || !aligned(scale, 4)) return LP_ERR_ALIGN;
  return hip_status(lp::launch_tensor_quant_delayed(src, n, dst_fmt, history, len, slot, margin, codes, scale,
                                                    static_cast<hipStream_t>(stream)));
}

static lp_status run_bwd(const lp_qtensor* grad, const lp_qtensor* x, const lp_qtensor* w, const int32_t* offsets,
                         int64_t groups, void* grad_x, void* grad_w, void* ws, size_t ws_bytes, void* stream) {
  const int64_t M = grad->rows, N = grad->cols;
  const int64_t K = grad_x ? w->cols : x->cols;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t G = (int32_t)(groups ? groups : 1);
  if (grad_x != nullptr && M * K > 0 && grad_w != nullptr && N * K > 0 && ws == nullptr) {
    lp::GemmCall cx{false, grad, w, offsets, G, M, N, K, grad_x, nullptr, 0};
    lp::GemmCall cw{true, grad, x, offsets, G, M, N, K, grad_w, nullptr, 0};
    return lp::launch_gemm_pair(cx, cw, s) == hipSuccess ? LP_OK : LP_ERR_HIP;
  }
  // dX and dW run one after the other on the stream, so they can share the workspace.
  if (grad_x != nullptr && M * K > 0) {
    lp::GemmCall c{false, grad, w, offsets, (int32_t)(groups ? groups : 1), M, N, K, grad_x, ws, ws_bytes};
    hipError_t e = lp::launch_gemm(c, s);
    if (e != hipSuccess) return LP_ERR_HIP;
  }
  if (grad_w != nullptr && N * K > 0) {
    lp::GemmCall c{true, grad, x, offsets, (int32_t)(groups ? groups : 1), M, N, K, grad_w, ws, ws_bytes};
    hipError_t e = lp::launch_gemm(c, s);
    if (e != hipSuccess) return LP_ERR_HIP;
  }
  return LP_OK;
}

lp_status lp_linear_bwd(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w, void* grad_x,
                        void* grad_w, void* stream) {
  if (grad_x == nullptr && grad_w == nullptr) return LP_OK;
  lp_status st = check_bwd(grad_out, x, w, grad_x, grad_w, 0);
  if (st != LP_OK) return st;
  return run_bwd(grad_out, x, w, nullptr, 0, grad_x, grad_w, nullptr, 0, stream);
}

lp_status lp_linear_bwd_workspace(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w,
                                  const void* grad_x, const void* grad_w, size_t* bytes) {
  if (bytes == nullptr) return LP_ERR_NULL;
  *bytes = 0;
  if (grad_x == nullptr && grad_w == nullptr) return LP_OK;
  // Only the shapes matter here: stand-in output pointers pass the checks.
  void* gx = grad_x ? reinterpret_cast<void*>(uintptr_t{256}) : nullptr;
  void* gw = grad_w ? reinterpret_cast<void*>(uintptr_t{256}) : nullptr;
  lp_status st = check_bwd(grad_out, x, w, gx, gw, 0);
  if (st != LP_OK) return st;
  const int64_t M = grad_out->rows, N = grad_out->cols;
  const int64_t K = grad_x ? w->cols : x->cols;
  size_t need = 0;
  if (grad_x != nullptr && M * K > 0) {
    lp::GemmCall c{false, grad_out, w, nullptr, 1, M, N, K, nullptr, nullptr, 0};
    need = lp::gemm_workspace_bytes(c);
  }
  if (grad_w != nullptr && N * K > 0) {
    lp::GemmCall c{true, grad_out, x, nullptr, 1, M, N, K, nullptr, nullptr, 0};
    const size_t b = lp::gemm_workspace_bytes(c);
    need = b > need ? b : need;
  }
  *bytes = need;
  return LP_OK;
}

lp_status lp_linear_bwd_ws(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w, void* grad_x,
                           void* grad_w, void* workspace, size_t workspace_bytes, void* stream) {
  if (grad_x == nullptr && grad_w == nullptr) return LP_OK;
  lp_status st = check_bwd(grad_out, x, w, grad_x, grad_w, 0);
  if (st != LP_OK) return st;
  if (workspace == nullptr) workspace_bytes = 0;
  if (workspace != nullptr && !aligned(workspace, 256)) return LP_ERR_ALIGN;
  return run_bwd(grad_out, x, w, nullptr, 0, grad_x, grad_w, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- no-allocation variant
// The split-contraction workspace of lp_linear_bwd_noalloc: a file-scope
// device array, one copy per GPU the library runs on, held until the process
// ends.  A split plan uses at most 256 partial tiles of 256 x 256 fp32
// (64 MiB: splitting only happens when the output has fewer tiles than the
// GPU has compute units, and a tile splits at most 256 / tiles ways) plus
// one u32 counter per tile (at most 64 tiles: 256 bytes); the array adds
// 4 KiB of headroom for the counters.  Host code never passes `scratch`
// itself to a kernel (in host code the name is a stand-in, not a device
// address): it uses the address hipGetSymbolAddress returns for the current
// device.
namespace {

constexpr size_t kScratchBytes = ((size_t)64 << 20) + 4096;
constexpr size_t kScratchCounterBytes = 4096;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch`, looked up once per device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

// Zero n words: the per-tile counters must start at zero.  A kernel rather
// than hipMemsetAsync, so that the call can be captured in a graph.
__global__ void clear_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

extern "C" {

lp_status lp_linear_bwd_noalloc(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w,
                                void* grad_x, void* grad_w, void* stream) {
  size_t need = 0;
  lp_status st = lp_linear_bwd_workspace(grad_out, x, w, grad_x, grad_w, &need);
  if (st != LP_OK) return st;
  if (grad_x == nullptr && grad_w == nullptr) return LP_OK;
  if ((st = check_bwd(grad_out, x, w, grad_x, grad_w, 0)) != LP_OK) return st;
  if (need > kScratchBytes) return LP_ERR_SHAPE;
  void* ws = nullptr;
  if (need > 0) {
    if (scratch_address(&ws) != hipSuccess) return LP_ERR_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    constexpr int kWords = (int)(kScratchCounterBytes / 4);
    clear_words<<<dim3(kWords / 256), dim3(256), 0, s>>>(static_cast<uint32_t*>(ws), kWords);
    if (hipGetLastError() != hipSuccess) return LP_ERR_HIP;
  }
  return run_bwd(grad_out, x, w, nullptr, 0, grad_x, grad_w, ws, need > 0 ? kScratchBytes : 0, stream);
}

}  // extern "C"

extern "C" {

// Checks of the forward: x [M][K] and w [G][N][K], both MXFP4 or both MXFP8
// scaled along k (K % 128 for MXFP4, K % 64 for MXFP8), both NVFP4 (K % 32),
// or a bf16 x with a bf16 or block-FP8 weight (K % 16); N % 16.
static lp_status check_fwd(const lp_qtensor* x, const lp_qtensor* w, void* y, int64_t groups) {
  lp_status st = check_tensor(x);
  if (st != LP_OK) return st;
  if ((st = check_tensor(w)) != LP_OK) return st;
  const bool mx = (x->fmt == LP_MXFP4 || x->fmt == LP_MXFP8) && w->fmt == x->fmt;
  const bool nv = x->fmt == LP_NVFP4 && w->fmt == LP_NVFP4;
  const bool b16 = x->fmt == LP_BF16 && (w->fmt == LP_BF16 || w->fmt == LP_FP8_B128 || w->fmt == LP_NVFP4);
  if (!mx && !nv && !b16) return LP_ERR_FORMAT;
  if ((mx || nv) && (x->scale_axis != -1 || w->scale_axis != -1)) return LP_ERR_FORMAT;
  if (w->fmt == LP_NVFP4 && w->scale_axis != -1) return LP_ERR_FORMAT;
  if (x->batch != 1 || w->batch != (groups ? groups : 1) || w->cols != x->cols) return LP_ERR_SHAPE;
  const int64_t kmul = x->fmt == LP_MXFP4 ? 128 : x->fmt == LP_MXFP8 ? 64 : w->fmt == LP_NVFP4 ? 32 : 16;
  if (x->cols % kmul || w->rows % 16) return LP_ERR_SHAPE;
  if (x->rows >= kMaxProductRows || x->cols >= kMaxProductCols || w->rows >= kMaxProductCols) return LP_ERR_SHAPE;
  if (!tiles_ok(x->rows / 128 + (groups ? groups : 1) + 1, w->rows)) return LP_ERR_SHAPE;
  if (x->rows * w->rows > 0 && y == nullptr) return LP_ERR_NULL;
  if (!aligned(y, 16)) return LP_ERR_ALIGN;
  return LP_OK;
}

lp_status lp_linear_fwd(const lp_qtensor* x, const lp_qtensor* w, void* y, void* stream) {
  lp_status st = check_fwd(x, w, y, 0);
  if (st != LP_OK) return st;
  if (x->rows * w->rows == 0) return LP_OK;
  return hip_status(lp::launch_fwd(*x, *w, nullptr, 1, y, static_cast<hipStream_t>(stream)));
}

lp_status lp_grouped_fwd(const lp_qtensor* x, const lp_qtensor* w, const int32_t* offsets, int64_t groups, void* y,
                         void* stream) {
  if (groups < 1 || groups > 1024) return LP_ERR_SHAPE;
  lp_status st = check_fwd(x, w, y, groups);
  if (st != LP_OK) return st;
  if (offsets == nullptr) return LP_ERR_NULL;
  if (!aligned(offsets, 4)) return LP_ERR_ALIGN;
  if (x->rows * w->rows == 0) return LP_OK;
  return hip_status(lp::launch_fwd(*x, *w, offsets, (int32_t)groups, y, static_cast<hipStream_t>(stream)));
}

lp_status lp_grouped_bwd(const lp_qtensor* grad_out, const lp_qtensor* x, const lp_qtensor* w,
                         const int32_t* offsets, int64_t groups, void* grad_x, void* grad_w, void* stream) {
  if (grad_x == nullptr && grad_w == nullptr) return LP_OK;
  if (groups < 1 || groups > 1024) return LP_ERR_SHAPE;
  lp_status st = check_bwd(grad_out, x, w, grad_x, grad_w, groups);
  if (st != LP_OK) return st;
  if (offsets == nullptr) return LP_ERR_NULL;
  if (!aligned(offsets, 4)) return LP_ERR_ALIGN;
  return run_bwd(grad_out, x, w, offsets, groups, grad_x, grad_w, nullptr, 0, stream);
}

lp_status lp_grouped_dx_deferred(const lp_qtensor* grad_out, const void* w, int64_t K, const int32_t* offsets,
                                 int64_t groups, int64_t fuse_rows, void* grad_x, void* w_codes, void* w_scales,
                                 void* stream) {
  if (groups < 1 || groups > 1024 || fuse_rows < 0 || K < 0 || K > kMaxDim) return LP_ERR_SHAPE;
  lp_status st = check_tensor(grad_out);
  if (st != LP_OK) return st;
  if (grad_out->fmt != LP_MXFP8 || grad_out->scale_axis != -1) return LP_ERR_FORMAT;
  if (grad_out->batch != 1) return LP_ERR_SHAPE;
  const int64_t M = grad_out->rows, N = grad_out->cols;
  int64_t n = 0;
  if (K % 16 || !count_ok(groups, N, K, &n)) return LP_ERR_SHAPE;
  if (M >= kMaxProductRows || N >= kMaxProductCols || K >= kMaxProductCols) return LP_ERR_SHAPE;
  if (!tiles_ok(M / 128 + groups + 1, K)) return LP_ERR_SHAPE;
  if (offsets == nullptr) return LP_ERR_NULL;
  if (!aligned(offsets, 4)) return LP_ERR_ALIGN;
  if (M * K == 0) return LP_OK;
  if (grad_x == nullptr || (n > 0 && w == nullptr)) return LP_ERR_NULL;
  if ((fuse_rows < M || N % 512 || K % 32) && n > 0 && (w_codes == nullptr || w_scales == nullptr)) return LP_ERR_NULL;
  if (!aligned(grad_x, 16) || !aligned(w, 16) || !aligned(w_codes, 16) || !aligned(w_scales, 16)) return LP_ERR_ALIGN;
  return hip_status(lp::launch_grouped_dx_deferred(*grad_out, w, K, offsets, (int32_t)groups, fuse_rows, w_codes,
                                                   w_scales, grad_x, static_cast<hipStream_t>(stream)));
}

const char* lp_status_string(int32_t s) {
  switch (s) {
    case LP_OK: return "ok";
    case LP_ERR_NULL: return "a required pointer is NULL";
    case LP_ERR_SHAPE: return "operand sizes are invalid or disagree";
    case LP_ERR_FORMAT: return "unsupported format or scale axis for this call";
    case LP_ERR_ALIGN: return "a pointer breaks the alignment rule";
    case LP_ERR_HIP: return "the HIP runtime reported a launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
