// Launcher of grad_X and grad_W of a per-tensor scaled FP8 gradient in one
// launch (one instantiation per pair of element formats).
#include "lp_gemm_mx_kernel.hpp"

namespace lp {
namespace gk {

hipError_t pt_pair(const Params& dx, const Params& dw, int fmt_p, int fmt_q, hipStream_t s) {
  const int dx_blocks = (dx.ntiles + 7) / 8 * 8;
  const int blocks = dx_blocks + dw.ntiles;
  if (blocks <= 0) return hipSuccess;
  const dim3 g(blocks), b(NT);
  const bool p5 = fmt_p == LP_FP8T_E5M2, q5 = fmt_q == LP_FP8T_E5M2;
  if (p5 && q5) pt_pair_kernel<1, 1><<<g, b, 0, s>>>(dx, dw, dx_blocks);
  else if (p5) pt_pair_kernel<1, 0><<<g, b, 0, s>>>(dx, dw, dx_blocks);
  else if (q5) pt_pair_kernel<0, 1><<<g, b, 0, s>>>(dx, dw, dx_blocks);
  else pt_pair_kernel<0, 0><<<g, b, 0, s>>>(dx, dw, dx_blocks);
  return hipGetLastError();
}

}  // namespace gk
}  // namespace lp
