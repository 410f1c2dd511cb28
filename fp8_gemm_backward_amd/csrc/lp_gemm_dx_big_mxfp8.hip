// grad_X kernels, 256 x 256 tiles, mxfp8 gradient, every saved-operand format.
#include "lp_gemm_kernel.hpp"

namespace lp {
namespace gk {

hipError_t dx_big_mxfp8(const lp_qtensor& q, const Params& prm, hipStream_t s) {
  return dispatch_q<Big, MXFP8, -1, false>(q, prm, s);
}

}  // namespace gk
}  // namespace lp
