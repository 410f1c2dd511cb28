// Launchers of the block-scaled MFMA kernel for MXFP8 operands.
#include <atomic>

#include "lp_gemm_mx_kernel.hpp"

namespace lp {
namespace gk {

// Compute units of the current device (one persistent workgroup each).
int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t dx_mx(const Params& prm, hipStream_t s) {
  if (prm.ntiles <= 0) return hipSuccess;
  // Chunk mode needs 16-byte aligned gradient scale rows (N % 512 == 0).
  // With more tiles than compute units, one persistent workgroup per
  // compute unit (a multiple of the 8 XCDs) walks them.
  const int cus = compute_units() / 8 * 8;
  if (prm.P.scale_ld % 16 == 0 && prm.ntiles > cus && cus >= 8)
    fp8_mfma_paired<><<<dim3(cus), dim3(NT), 0, s>>>(prm);
  else if (prm.P.scale_ld % 16 == 0)
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
