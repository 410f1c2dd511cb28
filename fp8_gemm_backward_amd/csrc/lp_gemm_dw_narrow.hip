// grad_W kernels, 256 x 128 tiles, bf16 gradient, every saved-operand format.
#include "lp_gemm_kernel.hpp"

namespace lp {
namespace gk {

hipError_t dw_narrow(const lp_qtensor& q, const Params& prm, hipStream_t s) {
  return dispatch_q<Narrow, BF16, -1, true>(q, prm, s);
}

}  // namespace gk
}  // namespace lp
