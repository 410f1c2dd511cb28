// Launchers of the block-scaled MFMA kernel for per-tensor scaled FP8
// operands (grad_W: one instantiation per pair of element formats).
#include "lp_gemm_mx_kernel.hpp"

namespace lp {
namespace gk {

hipError_t dw_pt(const Params& prm, int fmt_p, int fmt_q, hipStream_t s) {
  if (prm.ntiles <= 0) return hipSuccess;
  const dim3 g(prm.ntiles), b(NT);
  const bool p5 = fmt_p == LP_FP8T_E5M2, q5 = fmt_q == LP_FP8T_E5M2;
  if (p5 && q5) fp8_mfma_kernel<true, kTensorMode, 1, 1><<<g, b, 0, s>>>(prm);
  else if (p5) fp8_mfma_kernel<true, kTensorMode, 1, 0><<<g, b, 0, s>>>(prm);
  else if (q5) fp8_mfma_kernel<true, kTensorMode, 0, 1><<<g, b, 0, s>>>(prm);
  else fp8_mfma_kernel<true, kTensorMode, 0, 0><<<g, b, 0, s>>>(prm);
  return hipGetLastError();
}

}  // namespace gk
}  // namespace lp
