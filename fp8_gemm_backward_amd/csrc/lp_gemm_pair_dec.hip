// grad_X and grad_W of a grouped layer through bf16 tiles in one launch.
//
// "Add Autograd Backward Support for FP4 GEMM Custom Ops": the grouped
// backward computes grad_X = grad_out @ W[g] per group and grad_W[g] =
// grad_out^T @ X over each group's rows from the same saved FP4 operands.
// The two products are independent.  In one launch, grad_X's 256 x 256
// tiles are dispatched first and grad_W's after them, so that grad_W's tiles
// (longest contraction first) start on the compute units that grad_X's last,
// partly filled round of tiles leaves idle, instead of after it.  Each tile
// is computed as in its own launch, so the results are the same bits.
#include "lp_gemm_kernel.hpp"

namespace lp {
namespace gk {
namespace {

constexpr int imax(int a, int b) { return a > b ? a : b; }

// bf16 gradient (P) with a QF operand scaled along its last axis: W in
// grad_X, X in grad_W.  dx_blocks: grad_X's tile count rounded up to a
// multiple of the 8 XCDs, so that grad_W's part keeps the dispatch-order
// dealing that its tile selection assumes.
template <int QF>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_pair_kernel(Params dx, Params dw,
                                                                                                    int dx_blocks) {
  using GX = GemmShape<Big, BF16, -1, QF, -1, false, false>;
  using GW = GemmShape<Big, BF16, -1, QF, -1, true, false>;
  constexpr int SP0 = imax(GX::SP0, GW::SP0), SP1 = imax(GX::SP1, GW::SP1), SP2 = imax(GX::SP2, GW::SP2);
  constexpr int SQ0 = imax(GX::SQ0, GW::SQ0), SQ1 = imax(GX::SQ1, GW::SQ1), SQ2 = imax(GX::SQ2, GW::SQ2);
  // sq1 and sq2 hold data only when Q is loaded straight into LDS (a bf16
  // Q); otherwise they are unused placeholders that take no LDS.
  static_assert(!GX::QD && !GW::QD, "a decoded Q in both products");
  static_assert(SP0 + SP1 + SP2 + SQ0 <= kMaxLds, "both products' buffers fit in LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t sp0[SP0];
  __shared__ __attribute__((aligned(1024))) uint8_t sp1[SP1];
  __shared__ __attribute__((aligned(1024))) uint8_t sp2[SP2];
  __shared__ __attribute__((aligned(1024))) uint8_t sq0[SQ0];
  __shared__ __attribute__((aligned(1024))) uint8_t sq1[SQ1];
  __shared__ __attribute__((aligned(1024))) uint8_t sq2[SQ2];
  const int b = blockIdx.x;
  if (b < dx_blocks) {
    if (b < dx.ntiles) gemm_tile<Big, BF16, -1, QF, -1, false>(dx, b, sp0, sp1, sp2, sq0, sq1, sq2);
  } else {
    gemm_tile<Big, BF16, -1, QF, -1, true>(dw, b - dx_blocks, sp0, sp1, sp2, sq0, sq1, sq2);
  }
}

}  // namespace

hipError_t dec_pair(const Params& dx, const Params& dw, int fmt_q, hipStream_t s) {
  if (dx.ntiles <= 0 || dw.ntiles <= 0) return hipErrorInvalidValue;
  const int dx_blocks = (dx.ntiles + 7) / 8 * 8;
  const dim3 grid(dx_blocks + dw.ntiles);
  if (fmt_q == LP_MXFP4)
    gemm_pair_kernel<MXFP4><<<grid, dim3(NT), 0, s>>>(dx, dw, dx_blocks);
  else if (fmt_q == LP_NVFP4)
    gemm_pair_kernel<NVFP4><<<grid, dim3(NT), 0, s>>>(dx, dw, dx_blocks);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gk
}  // namespace lp
