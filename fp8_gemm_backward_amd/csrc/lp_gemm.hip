// Host side of the fused backward GEMMs: operand descriptors, tile-size
// choice and dispatch to the per-format kernel instantiations.
#include "lp_gemm_kernel.hpp"

namespace lp {
namespace gk {
namespace {

Op make_op(const lp_qtensor& t) {
  Op o{};
  o.codes = static_cast<const uint8_t*>(t.codes);
  o.scales = static_cast<const uint8_t*>(t.scales);
  o.tensor_scale = t.tensor_scale;
  o.rows = (int32_t)t.rows;
  const int64_t R = t.rows, Cc = t.cols;
  switch (t.fmt) {
    case LP_BF16:
      o.code_ld = (int32_t)(Cc * 2);
      break;
    case LP_MXFP4:
      o.code_ld = (int32_t)(Cc / 2);
      o.scale_ld = (int32_t)(Cc / 32);
      o.scale_bytes = R * (Cc / 32);
      break;
    case LP_NVFP4:
      o.code_ld = (int32_t)(Cc / 2);
      o.scale_ld = (int32_t)(Cc / 16);
      o.scale_bytes = R * (Cc / 16);
      break;
    case LP_FP8_B128:
      o.code_ld = (int32_t)Cc;
      o.scale_ld = (int32_t)(((Cc + 127) / 128) * 4);
      o.scale_bytes = ((R + 127) / 128) * ((Cc + 127) / 128) * 4;
      break;
    case LP_MXFP8:
      o.code_ld = (int32_t)Cc;
      if (t.scale_axis == -1) {
        o.scale_ld = (int32_t)(Cc / 32);
        o.scale_bytes = R * (Cc / 32);
      } else {
        o.scale_ld = (int32_t)Cc;
        o.scale_bytes = (R / 32) * Cc;
      }
      break;
  }
  o.code_batch = R * o.code_ld;
  o.scale_batch = o.scale_bytes;
  return o;
}


template <class C>
hipError_t launch_cfg(const GemmCall& call, Params prm, hipStream_t stream) {
  prm.nq = (int32_t)((prm.Qtot + C::BQ - 1) / C::BQ);
  if (!call.dw) {
    const int64_t ptiles = call.offsets ? (call.M / C::BP + call.groups) : (call.M + C::BP - 1) / C::BP;
    prm.ntiles = (int32_t)(ptiles * prm.nq);
    const bool mx = call.grad->fmt == LP_MXFP8;
    if constexpr (C::BQ == Big::BQ) return mx ? dx_big_mxfp8(*call.other, prm, stream) : dx_big_bf16(*call.other, prm, stream);
    else return mx ? dx_narrow_mxfp8(*call.other, prm, stream) : dx_narrow_bf16(*call.other, prm, stream);
  }
  const int64_t np = (prm.Ptot + C::BP - 1) / C::BP;
  prm.ntiles = (int32_t)(np * prm.nq * call.groups);
  if constexpr (C::BQ == Big::BQ) return dw_big(*call.other, prm, stream);
  else return dw_narrow(*call.other, prm, stream);
}

}  // namespace
}  // namespace gk

using namespace gk;

hipError_t launch_gemm(const GemmCall& call, hipStream_t stream) {
  Params prm{};
  prm.P = make_op(*call.grad);
  prm.Q = make_op(*call.other);
  prm.C = static_cast<uint16_t*>(call.out);
  prm.ldc = (int32_t)call.K;
  prm.Qtot = (int32_t)call.K;
  prm.offsets = call.offsets;
  prm.groups = call.groups;
  if (!call.dw) {
    prm.Ptot = (int32_t)call.M;
    prm.Ktot = (int32_t)call.N;
    prm.c_batch = 0;
  } else {
    prm.Ptot = (int32_t)call.N;
    prm.Ktot = (int32_t)call.M;
    prm.c_batch = call.N * call.K;
  }
  // Fewer than one full wave of 256-wide tiles across the 256 CUs: halve the
  // tile width so that every CU gets work.
  const int64_t big_tiles = (call.dw ? call.groups * ((call.N + 255) / 256) : (call.M + 255) / 256) *
                            ((call.K + 255) / 256);
  if (big_tiles < 256) return launch_cfg<Narrow>(call, prm, stream);
  return launch_cfg<Big>(call, prm, stream);
}

}  // namespace lp
