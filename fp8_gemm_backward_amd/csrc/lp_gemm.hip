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
    case LP_FP8T_E4M3:
    case LP_FP8T_E5M2:
      o.code_ld = (int32_t)Cc;
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


constexpr int kCUsPerXcd = 32;

// P-tile rows per group of the tile order (grouped_order): a group of g rows
// and kCUsPerXcd / g columns of tiles runs on one XCD at a time and fetches
// g * a + (kCUsPerXcd / g) * b bytes per slab into its L2 (a, b: bytes of one
// P-tile row and one Q-tile column of a slab), least at g = sqrt(32 b / a);
// the power of two nearest to it, ties to the smaller.
int32_t tile_group(int64_t a, int64_t b, int64_t np) {
  int32_t g = 1;
  while (g < kCUsPerXcd && (int64_t)(2 * g) * (2 * g) * a < (int64_t)kCUsPerXcd * b * 2) g *= 2;
  return (int32_t)(g < np ? g : (np > 0 ? np : 1));
}

// Bytes per element of an operand's codes, times 2.
int64_t code_bytes2(int fmt) {
  return fmt == LP_BF16 ? 4 : (fmt == LP_MXFP4 || fmt == LP_NVFP4) ? 1 : 2;
}

// Grouped grad_X and forward on 256 x 256 tiles (prm.ntiles: the host's
// bound on them) split by dispatch round: the whole rounds of kCUs tiles in
// this launch, a short last round as 256 x 128 tiles in a second launch
// (tail_params).  The group sizes live on the device, so the kernels count
// the tiles and both launches reach the same split, or none (the second
// launch then has no tile).  Returns whether to make the second launch.
// Only for contractions of at least kTailMinSlabs slabs: measured in steady
// state, the block-FP8 grouped forward (4096-long contraction, 544 tiles)
// went from 342.5 to 316.3 us, while the MXFP4 grouped grad_X (2048-long,
// 1088 tiles) went from 268.0 to 271.7 us; a short tile's fixed costs and
// the second launch outweigh what its narrower last round saves.
constexpr int kTailMinSlabs = 64;
bool tile_split(Params& prm) {
  if (prm.offsets == nullptr || prm.splits != 1 || prm.fuse_side != 0 || prm.ntiles < kCUs) return false;
  if (prm.Ktot < kTailMinSlabs * BK) return false;
  prm.tail = 1;
  return true;
}
Params tail_params(const Params& big) {
  Params t = big;
  t.tail = 2;
  t.nq = (int32_t)((t.Qtot + Narrow::BQ - 1) / Narrow::BQ);
  t.ntiles = kCUs;
  return t;
}

// The tile counts and order of a call on C tiles (prm from base_params, with
// any split plan already set).
template <class C>
Params cfg_params(const GemmCall& call, Params prm) {
  prm.nq = (int32_t)((prm.Qtot + C::BQ - 1) / C::BQ);
  if (call.offsets == nullptr && prm.splits == 1)
    prm.gm = tile_group(C::BP * code_bytes2(call.grad->fmt), C::BQ * code_bytes2(call.other->fmt),
                        (prm.Ptot + C::BP - 1) / C::BP);
  if (!call.dw) {
    const int64_t ptiles = call.offsets ? (call.M / C::BP + call.groups) : (call.M + C::BP - 1) / C::BP;
    prm.ntiles = (int32_t)(ptiles * prm.nq * prm.splits);
  } else {
    const int64_t np = (prm.Ptot + C::BP - 1) / C::BP;
    prm.ntiles = (int32_t)(np * prm.nq * call.groups * prm.splits);
  }
  return prm;
}

template <class C>
hipError_t launch_cfg(const GemmCall& call, Params prm, hipStream_t stream) {
  prm = cfg_params<C>(call, prm);
  if (!call.dw) {
    const bool mx = call.grad->fmt == LP_MXFP8;
    if constexpr (C::BQ == Big::BQ) {
      const bool split = tile_split(prm);
      const hipError_t e = mx ? dx_big_mxfp8(*call.other, prm, stream) : dx_big_bf16(*call.other, prm, stream);
      if (e != hipSuccess || !split) return e;
      const Params tail = tail_params(prm);
      return mx ? dx_narrow_mxfp8(*call.other, tail, stream) : dx_narrow_bf16(*call.other, tail, stream);
    } else {
      return mx ? dx_narrow_mxfp8(*call.other, prm, stream) : dx_narrow_bf16(*call.other, prm, stream);
    }
  }
  if constexpr (C::BQ == Big::BQ) return dw_big(*call.other, prm, stream);
  else return dw_narrow(*call.other, prm, stream);
}

constexpr int64_t kMinSplitSlabs = 16;     // contraction slabs per split, at least

// Output tiles of the 256 x 256 configuration.
int64_t big_tiles(const GemmCall& call) {
  const int64_t p = call.dw ? call.groups * ((call.N + 255) / 256) : (call.M + 255) / 256;
  return p * ((call.K + 255) / 256);
}

// Output tiles of the 256 x 128 configuration.
int64_t narrow_tiles(const GemmCall& call) {
  const int64_t p = call.dw ? call.groups * ((call.N + 255) / 256) : (call.M + 255) / 256;
  return p * ((call.K + 127) / 128);
}

// Split plan of a dense contraction whose output tiles would leave most CUs
// idle even at 256 x 128 (fewer than half as many tiles as CUs): as many
// splits of 256 x 256 tiles as keep one workgroup per CU, each split at
// least kMinSplitSlabs slabs long.  splits == 1: no split.  Measured on the
// 4096 x 2048 output of an 8192-long contraction (128 big tiles, two
// splits), the partials' write-back and re-read cost more than the narrower
// tiles lose, hence the threshold.
struct SplitPlan {
  int32_t splits, split_len;
  int64_t tiles;
  size_t bytes;
};

// dX of an MXFP8 gradient and an MXFP8 weight scaled along its rows: both
// scales run along the contraction, so the block-scaled MFMA applies them.
// Dense dW of an MXFP8 gradient and an MXFP8 input both scaled along their
// rows (the token axis, the contraction) likewise.
bool native_mx(const GemmCall& call) {
  if (call.grad->fmt != LP_MXFP8 || call.other->fmt != LP_MXFP8 || call.other->scale_axis != -2) return false;
  return !call.dw || (call.grad->scale_axis == -2 && call.offsets == nullptr);
}

bool is_fp8t(int f) { return f == LP_FP8T_E4M3 || f == LP_FP8T_E5M2; }

// Per-tensor scaled FP8 on both sides of the product.
bool native_pt(const GemmCall& call) { return is_fp8t(call.grad->fmt) && is_fp8t(call.other->fmt); }

SplitPlan split_plan(const GemmCall& call) {
  SplitPlan sp{1, 0, big_tiles(call), 0};
  if (call.offsets != nullptr || native_mx(call) || native_pt(call) || narrow_tiles(call) >= kCUs / 2 || sp.tiles == 0) return sp;
  const int64_t ktot = call.dw ? call.M : call.N;
  const int64_t nk = (ktot + BK - 1) / BK;
  int64_t s = kCUs / sp.tiles;
  if (s > nk / kMinSplitSlabs) s = nk / kMinSplitSlabs;
  if (s < 2) return sp;
  const int64_t per = (nk + s - 1) / s;                 // slabs per split
  s = (nk + per - 1) / per;                             // no empty split
  if (s < 2) return sp;
  sp.splits = (int32_t)s;
  sp.split_len = (int32_t)(per * BK);
  const size_t counters = ((size_t)sp.tiles * 4 + 255) / 256 * 256;
  sp.bytes = counters + (size_t)sp.tiles * s * Big::BP * Big::BQ * sizeof(float);
  return sp;
}

}  // namespace
}  // namespace gk

using namespace gk;

size_t gemm_workspace_bytes(const GemmCall& call) { return split_plan(call).bytes; }

namespace {

Params base_params(const GemmCall& call) {
  Params prm{};
  prm.P = make_op(*call.grad);
  prm.Q = make_op(*call.other);
  prm.C = static_cast<uint16_t*>(call.out);
  prm.ldc = (int32_t)call.K;
  prm.Qtot = (int32_t)call.K;
  prm.offsets = call.offsets;
  prm.groups = call.groups;
  prm.splits = 1;
  prm.fuse_rows = call.fuse_rows;
  prm.fuse_side = call.fuse_side;
  if (!call.dw) {
    prm.Ptot = (int32_t)call.M;
    prm.Ktot = (int32_t)call.N;
    prm.c_batch = 0;
  } else {
    prm.Ptot = (int32_t)call.N;
    prm.Ktot = (int32_t)call.M;
    prm.c_batch = call.N * call.K;
  }
  return prm;
}

// Tile counts of a contraction on the FP8 MFMA kernel (256 x 256 tiles).
Params native_params(const GemmCall& call) {
  Params prm = base_params(call);
  prm.nq = (int32_t)((prm.Qtot + Big::BQ - 1) / Big::BQ);
  // Dense calls order their tiles in blocks of gm row tiles; grouped grad_X
  // does the same inside each group (a group of fewer row tiles is one
  // block).
  if (call.offsets == nullptr || !call.dw)
    prm.gm = tile_group(Big::BP * code_bytes2(call.grad->fmt), Big::BQ * code_bytes2(call.other->fmt),
                        call.offsets == nullptr ? (prm.Ptot + Big::BP - 1) / Big::BP : kCUsPerXcd);
  if (call.dw) {
    prm.ntiles = (int32_t)(((call.N + Big::BP - 1) / Big::BP) * prm.nq * call.groups);
  } else {
    const int64_t ptiles = call.offsets ? (call.M / Big::BP + call.groups) : (call.M + Big::BP - 1) / Big::BP;
    prm.ntiles = (int32_t)(ptiles * prm.nq);
  }
  return prm;
}

}  // namespace

hipError_t launch_gemm(const GemmCall& call, hipStream_t stream) {
  if (native_mx(call) || native_pt(call)) {
    const Params prm = native_params(call);
    const int fp = call.grad->fmt, fq = call.other->fmt;
    if (native_pt(call)) return call.dw ? dw_pt(prm, fp, fq, stream) : dx_pt(prm, fp, fq, stream);
    return call.dw ? dw_mx(prm, stream) : dx_mx(prm, stream);
  }
  Params prm = base_params(call);
  if (big_tiles(call) >= kCUs) return launch_cfg<Big>(call, prm, stream);
  // Fewer than one full wave of 256 x 256 tiles across the CUs: split the
  // contraction when a large enough workspace is given, else halve the tile
  // width so that every CU gets work.
  const SplitPlan sp = split_plan(call);
  if (sp.splits > 1 && call.ws != nullptr && call.ws_bytes >= sp.bytes) {
    const size_t counters = ((size_t)sp.tiles * 4 + 255) / 256 * 256;
    prm.splits = sp.splits;
    prm.split_len = sp.split_len;
    prm.cnt = static_cast<uint32_t*>(call.ws);
    prm.ws = reinterpret_cast<float*>(static_cast<uint8_t*>(call.ws) + counters);
    return launch_cfg<Big>(call, prm, stream);
  }
  return launch_cfg<Narrow>(call, prm, stream);
}

hipError_t launch_fwd(const lp_qtensor& x, const lp_qtensor& w, const int32_t* offsets, int32_t groups, void* y,
                      hipStream_t stream) {
  Params prm{};
  prm.P = make_op(x);
  prm.Q = make_op(w);
  prm.C = static_cast<uint16_t*>(y);
  prm.Ptot = (int32_t)x.rows;
  prm.Qtot = (int32_t)w.rows;
  prm.Ktot = (int32_t)x.cols;
  prm.ldc = prm.Qtot;
  prm.offsets = offsets;
  prm.groups = groups;
  prm.splits = 1;
  // MX operands run on the block-scaled MFMA (256 x 256 tiles); the others
  // through bf16 tiles, 256 x 256 unless both are bf16 (256 x 128: three
  // stages of both tiles fit in LDS only at that width).
  const bool mx = x.fmt == LP_MXFP4 || x.fmt == LP_MXFP8;
  const int BP = 256, BQ = w.fmt == LP_BF16 ? 128 : 256;
  prm.nq = (int32_t)((prm.Qtot + BQ - 1) / BQ);
  if (offsets == nullptr)
    prm.gm = tile_group(BP * code_bytes2(x.fmt), BQ * code_bytes2(w.fmt), (prm.Ptot + BP - 1) / BP);
  const int64_t ptiles = offsets ? (x.rows / BP + groups) : (x.rows + BP - 1) / BP;
  prm.ntiles = (int32_t)(ptiles * prm.nq);
  if (mx) return fwd_mx(prm, x.fmt == LP_MXFP4, stream);
  const bool split = BQ == Big::BQ && tile_split(prm);
  const hipError_t e = fwd_dec(prm, x.fmt, w.fmt, false, stream);
  if (e != hipSuccess || !split) return e;
  return fwd_dec(tail_params(prm), x.fmt, w.fmt, true, stream);
}

hipError_t launch_grouped_dx_deferred(const lp_qtensor& grad, const void* w, int64_t K, const int32_t* offsets,
                                      int32_t groups, int64_t fuse_rows, void* w_codes, void* w_scales,
                                      void* grad_x, hipStream_t stream) {
  const int64_t M = grad.rows, N = grad.cols;
  // The fused kernel takes the gradient's scales in 16-byte chunks of its
  // scale rows (N % 512 == 0), and the quantizer that leaves out the fused
  // groups works on 32 x 32 tiles (K % 32 == 0); otherwise every weight is
  // quantized first.
  const bool can_fuse = N % 512 == 0 && K % 32 == 0;
  const int32_t fr = can_fuse ? (int32_t)(fuse_rows < M ? fuse_rows : M) : 0;
  // Groups of more than fr rows: weight quantized first, then the
  // block-scaled product on its codes.
  if (fr < M) {
    hipError_t e = fr > 0 ? launch_mx_quant_rows_groups(w, groups, N, K, offsets, M, fr, w_codes, w_scales, stream)
                          : launch_mx_quant(w, groups, N, K, -2, LP_MXFP8, w_codes, w_scales, stream);
    if (e != hipSuccess) return e;
    const lp_qtensor wq{LP_MXFP8, -2, groups, N, K, w_codes, w_scales, nullptr};
    GemmCall c{false, &grad, &wq, offsets, groups, M, N, K, grad_x, nullptr, 0};
    c.fuse_rows = fr;
    c.fuse_side = fr > 0 ? 1 : 0;
    if ((e = launch_gemm(c, stream)) != hipSuccess) return e;
  }
  // Groups of at most fr rows: the weight quantized inside the product.
  if (fr > 0) {
    const lp_qtensor wb{LP_BF16, -1, groups, N, K, w, nullptr, nullptr};
    GemmCall c{false, &grad, &wb, offsets, groups, M, N, K, grad_x, nullptr, 0};
    Params prm = base_params(c);
    prm.fuse_rows = fr;
    prm.fuse_side = 2;
    prm.nq = (int32_t)((K + 255) / 256);
    // Row tiles of the listed groups: at most M / 256 + G, and at most
    // G ceil(fr / 256).
    int64_t rt = M / 256 + groups;
    const int64_t rt2 = (int64_t)groups * ((fr + 255) / 256);
    rt = rt2 < rt ? rt2 : rt;
    prm.ntiles = (int32_t)(rt * prm.nq);
    return dx_wquant(prm, stream);
  }
  return hipSuccess;
}

hipError_t launch_gemm_pair(const GemmCall& dx, const GemmCall& dw, hipStream_t stream) {
  if (native_pt(dx) && native_pt(dw) && dx.other->fmt == dw.other->fmt)
    return pt_pair(native_params(dx), native_params(dw), dx.grad->fmt, dx.other->fmt, stream);
  // A grouped layer's grad_X and grad_W from a bf16 gradient and FP4 W and X
  // (scaled along their last axis), both on 256 x 256 tiles: one launch.
  const int fq = dx.other->fmt;
  if (dx.offsets != nullptr && dx.grad->fmt == LP_BF16 && (fq == LP_MXFP4 || fq == LP_NVFP4) &&
      dw.other->fmt == fq && dx.other->scale_axis == -1 && dw.other->scale_axis == -1 && dx.ws == nullptr &&
      dw.ws == nullptr && big_tiles(dx) >= kCUs && big_tiles(dw) >= kCUs)
    return dec_pair(cfg_params<Big>(dx, base_params(dx)), cfg_params<Big>(dw, base_params(dw)), fq, stream);
  const hipError_t e = launch_gemm(dx, stream);
  return e != hipSuccess ? e : launch_gemm(dw, stream);
}

}  // namespace lp
