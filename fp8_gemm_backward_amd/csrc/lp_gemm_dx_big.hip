// grad_X kernels, 256 x 256 tiles, bf16 gradient, every saved-operand format.
#include "lp_gemm_kernel.hpp"

namespace lp {
namespace gk {

hipError_t dx_big_bf16(const lp_qtensor& q, const Params& prm, hipStream_t s) {
  return dispatch_q<Big, BF16, -1, false>(q, prm, s);
}

}  // namespace gk
}  // namespace lp
