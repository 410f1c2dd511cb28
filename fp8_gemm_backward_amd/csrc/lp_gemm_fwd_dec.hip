// Forward y = x @ W^T of a layer whose operands go through bf16 tiles: the
// GEMM kernel with both operands k-major (the contraction runs along K, the
// columns of x and of every W[g]).
//
// "Train adapters on top of FP8 weights": FP8LinearFunction.forward and
// FP8GroupedMatmulFunction.forward multiply a bf16 input by an E4M3 weight
// with fp32 inverse scales per 128 x 128 block (dense, and grouped over
// int32 cumulative end offsets with rows past the last offset left
// unwritten).  "Add Autograd Backward Support for FP4 GEMM Custom Ops": the
// f4f4bf16 forward ops multiply FP4 inputs by FP4 weights into BF16.  Each
// quantized operand is decoded to bf16 inside the contraction, as the
// backward decodes it, and contracted on the bf16 MFMA with fp32 sums.  A
// bf16 x with an NVFP4 weight is the same product with x decoded
// beforehand (lp_dequant), once rather than in every tile that reads it.
#include "lp_gemm_kernel.hpp"

namespace lp {
namespace gk {

// narrow: the 256 x 128 tiles of a split grouped call's last round (the
// formats whose tiles are otherwise 256 x 256).
hipError_t fwd_dec(const Params& prm, int fmt_x, int fmt_w, bool narrow, hipStream_t s) {
  if (fmt_x == LP_BF16 && fmt_w == LP_BF16) return run<Narrow, BF16, -1, BF16, -1, false, true>(prm, s);
  if (fmt_x == LP_BF16 && fmt_w == LP_FP8_B128)
    return narrow ? run<Narrow, BF16, -1, FP8_B128, -1, false, true>(prm, s)
                  : run<Big, BF16, -1, FP8_B128, -1, false, true>(prm, s);
  if (fmt_x == LP_BF16 && fmt_w == LP_NVFP4)
    return narrow ? run<Narrow, BF16, -1, NVFP4, -1, false, true>(prm, s)
                  : run<Big, BF16, -1, NVFP4, -1, false, true>(prm, s);
  if (fmt_x == LP_NVFP4 && fmt_w == LP_NVFP4)
    return narrow ? run<Narrow, NVFP4, -1, NVFP4, -1, false, true>(prm, s)
                  : run<Big, NVFP4, -1, NVFP4, -1, false, true>(prm, s);
  return hipErrorInvalidValue;
}

}  // namespace gk
}  // namespace lp
