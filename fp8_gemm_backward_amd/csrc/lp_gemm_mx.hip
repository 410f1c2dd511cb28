// Launchers of the block-scaled MFMA kernel for MXFP8 operands.
#include "lp_gemm_mx_kernel.hpp"

namespace lp {
namespace gk {

hipError_t dx_mx(const Params& prm, hipStream_t s) {
  if (prm.ntiles <= 0) return hipSuccess;
  // Chunk mode needs 16-byte aligned gradient scale rows (N % 512 == 0).
  if (prm.P.scale_ld % 16 == 0)
    fp8_mfma_kernel<false, kChunkMode><<<dim3(prm.ntiles), dim3(NT), 0, s>>>(prm);
  else
    fp8_mfma_kernel<false, kGatherMode><<<dim3(prm.ntiles), dim3(NT), 0, s>>>(prm);
  return hipGetLastError();
}

hipError_t dw_mx(const Params& prm, hipStream_t s) {
  if (prm.ntiles <= 0) return hipSuccess;
  fp8_mfma_kernel<true, kChunkMode><<<dim3(prm.ntiles), dim3(NT), 0, s>>>(prm);
  return hipGetLastError();
}

}  // namespace gk
}  // namespace lp
