// Forward of an MX-quantized linear or grouped (per-expert) matmul on gfx950's
// block-scaled MFMA: y[m][n] = sum_k x[m][k] * w[g][n][k], where x and w are
// both MXFP4 (E2M1) or both MXFP8 (E4M3) with one E8M0 scale per 32 along k,
// the contraction.
//
// "Add Autograd Backward Support for FP4 GEMM Custom Ops": the forward ops
// that the backward pairs with multiply FP4 inputs by FP4 weights, dense and
// grouped, into bf16.  "perf: defer mxfp8 backward quantization",
// MXFP8MatMul.forward: the MXFP8 forward contracts x quantized along its last
// axis with the weight quantized along the same (reduction) axis.
//
// Both scales run along the contraction, which is what
// v_mfma_scale_f32_32x32x64_f8f6f4 applies: every product code_x * code_w *
// 2^(sx + sw) is exact and the products are summed in fp32, so the result is
// the contraction of the decoded operands up to summation order.
//
// Operand layout of that instruction (measured with in-bounds probes): lane
// l feeds row (A) or column (B) l % 32 and supplies the scale byte of
// contraction block l / 32 of a 64-deep step.  E4M3: 32 bytes, bytes 0..15 =
// k 16 h + 0..15 and bytes 16..31 = k 32 + 16 h + 0..15 (h = l / 32).  E2M1:
// 16 bytes, the 32 values of block h in memory order (low nibble first); the
// upper 16 bytes of the operand are not read.
//
// Tiles: 256 x 256 outputs, four waves of 128 x 128, slabs of 64 bytes per
// row of each operand (64 E4M3 or 128 E2M1 values).  Both tiles are
// [row][64 B] with 16-byte chunk c of row r at c ^ ((r >> 2) & 3), so the
// fragment reads (16 consecutive rows, one chunk) hit distinct slots.  A
// lane's two chunks of a fragment, h and 2 + h, make one E4M3 operand or the
// operands of two E2M1 steps.  Each slab's scales (2 or 4 bytes per row and
// operand) come with the codes as one zero-extended dword per row.  Codes and
// scales go global -> LDS by direct loads, four stages deep, three slabs
// ahead; one barrier per slab.
#include "lp_gemm_kernel.hpp"

namespace lp {
namespace gk {
namespace {

constexpr int FBP = 256, FBQ = 256;             // output tile
constexpr int FWP = 128, FWQ = 128;             // wave tile
constexpr int FFP = 4, FFQ = 4;                 // 32 x 32 blocks per wave
constexpr int kRowBytes = 64;                   // code bytes per row and slab
constexpr int kOpBytes = FBP * kRowBytes;       // one operand's codes per slab
constexpr int kScaleBytes = FBP * 4;            // one operand's scales per slab (a dword per row)
constexpr int kStage = 2 * kOpBytes + 2 * kScaleBytes;
constexpr int T = 10;                           // direct loads per wave and slab
using FCfg = Cfg<FBP, FBQ>;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int f_swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ i32x8 low_half(i32x4 v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1); }

template <bool kFp4>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void mx_fwd_kernel(Params p) {
  constexpr int KS = kFp4 ? 128 : 64;            // contraction elements per slab
  constexpr int FMT = kFp4 ? 4 : 0;              // MFMA operand format
  __shared__ __attribute__((aligned(1024))) uint8_t st0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[kStage];
  static_assert(kMaxGroups * 4 <= kStage, "group ends alias stage 0");
  static_assert(FWP * FWQ * 2 <= kStage, "epilogue staging fits a stage");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave >> 1, wq = wave & 1;
  const Tile t = select_tile<FCfg, false>(p, reinterpret_cast<int32_t*>(st0));
  if (!t.valid) return;
  __syncthreads();                                               // group ends read; stage 0 reusable

  const int ldp = p.P.code_ld, ldq = p.Q.code_ld;                // code bytes per x / w row
  const int sldp = p.P.scale_ld, sldq = p.Q.scale_ld;            // scale bytes per row (K / 32)
  const int kend = t.kend;                                       // K, a multiple of KS
  const int64_t prows = (int64_t)(p.Ptot - t.p0), qrows = (int64_t)(p.Qtot - t.q0);
  const uint8_t* pc = p.P.codes + (int64_t)t.p0 * ldp;
  const uint8_t* qc = p.Q.codes + (int64_t)t.g * p.Q.code_batch + (int64_t)t.q0 * ldq;
  const Rsrc ps_r = make_rsrc(p.P.scales + (int64_t)t.p0 * sldp, prows * sldp);
  const Rsrc qs_r = make_rsrc(p.Q.scales + (int64_t)t.g * p.Q.scale_batch + (int64_t)t.q0 * sldq, qrows * sldq);

  // Code loads: wave w fills blocks 4 w + u (u = 0..3) of 16 rows x 64 B;
  // lane i takes row 16 (4 w + u) + i / 4 and physical chunk i % 4, whose
  // logical chunk (i % 4) ^ f_swz(row) = (i % 4) ^ ((i >> 4) & 3) does not
  // depend on u.  Rows past the operand's end read as zeros.
  const int chunk = (lane & 3) ^ ((lane >> 4) & 3);
  const int32_t p_off = (16 * 4 * wave + lane / 4) * ldp + 16 * chunk;   // + 16 u ldp
  const int32_t q_off = (16 * 4 * wave + lane / 4) * ldq + 16 * chunk;
  // Scale loads: wave w brings rows 64 w + i of each operand.
  const int32_t ps_off = (64 * wave + lane) * sldp, qs_off = (64 * wave + lane) * sldq;

  auto stage = [&](auto si) -> uint8_t* {
    constexpr int I = decltype(si)::value % 4;
    if constexpr (I == 0) return st0;
    else if constexpr (I == 1) return st1;
    else if constexpr (I == 2) return st2;
    else return st3;
  };

  // Item u of the slab at contraction k0: x codes (0..3), w codes (4..7),
  // x scales (8), w scales (9).
  auto issue = [&](auto ui, uint8_t* sb, int k0) {
    constexpr int u = decltype(ui)::value;
    const int kb = k0 * kRowBytes / KS;                          // byte offset of the slab in a row
    if constexpr (u < 4) {
      const Rsrc r = make_rsrc(pc + kb, prows * ldp - kb);
      dma<16>(r, (lds_void*)(sb + 1024 * (4 * wave + u)), p_off, 16 * u * ldp);
    } else if constexpr (u < 8) {
      constexpr int v = u - 4;
      const Rsrc r = make_rsrc(qc + kb, qrows * ldq - kb);
      dma<16>(r, (lds_void*)(sb + kOpBytes + 1024 * (4 * wave + v)), q_off, 16 * v * ldq);
    } else {
      const Rsrc r = u == 8 ? ps_r : qs_r;
      uint8_t* dst = sb + 2 * kOpBytes + (u == 8 ? 0 : kScaleBytes) + 256 * wave;
      if constexpr (kFp4)
        dma<4>(r, (lds_void*)dst, u == 8 ? ps_off : qs_off, k0 / 32);
      else
        dma<2>(r, (lds_void*)dst, u == 8 ? ps_off : qs_off, k0 / 32);
    }
  };

  // Fragment f (or j) of lane l: row 128 wp (128 wq) + 32 f + l % 32, chunks
  // h and 2 + h (h = l / 32); the swizzle of the row depends on l % 32 only.
  const int r32 = lane & 31, hh = lane >> 5;
  const int32_t a0 = r32 * kRowBytes + 16 * (hh ^ f_swz(r32));
  const int32_t a1 = r32 * kRowBytes + 16 * ((2 + hh) ^ f_swz(r32));
  const int32_t pa = wp * FWP * kRowBytes, qa = kOpBytes + wq * FWQ * kRowBytes;
  const int32_t psa = 2 * kOpBytes + (wp * FWP + r32) * 4, qsa = 2 * kOpBytes + kScaleBytes + (wq * FWQ + r32) * 4;

  i32x4 pf[2][FFP][2], qf[2][FFQ][2];
  uint32_t psc[2][FFP], qsc[2][FFQ];
  constexpr int NREAD = 2 * FFP + 2 * FFQ + FFP + FFQ;
  // Read r of the slab in stage sb into register set SET: x chunks, w
  // chunks, then the scale dwords.  Nothing here computes on a loaded value:
  // an operation on one would make the wave wait for every LDS read in
  // flight in the middle of the MFMA stream.
  auto read = [&](auto ri, auto seti, const uint8_t* sb) {
    constexpr int r = decltype(ri)::value, SET = decltype(seti)::value;
    if constexpr (r < 2 * FFP) {
      constexpr int f = r / 2, e = r % 2;
      pf[SET][f][e] = *reinterpret_cast<const i32x4*>(sb + pa + (e ? a1 : a0) + f * 32 * kRowBytes);
    } else if constexpr (r < 2 * FFP + 2 * FFQ) {
      constexpr int j = (r - 2 * FFP) / 2, e = (r - 2 * FFP) % 2;
      qf[SET][j][e] = *reinterpret_cast<const i32x4*>(sb + qa + (e ? a1 : a0) + j * 32 * kRowBytes);
    } else if constexpr (r < 2 * FFP + 2 * FFQ + FFP) {
      constexpr int f = r - 2 * FFP - 2 * FFQ;
      psc[SET][f] = *reinterpret_cast<const uint32_t*>(sb + psa + f * 32 * 4);
    } else {
      constexpr int j = r - 2 * FFP - 2 * FFQ - FFP;
      qsc[SET][j] = *reinterpret_cast<const uint32_t*>(sb + qsa + j * 32 * 4);
    }
  };
  // At the top of a slab (its reads complete): the scale dwords shifted so
  // that this lane's block h is the low byte (E2M1: block 2 + h is byte 2).
  int32_t ps[FFP], qs[FFQ];
  auto scales = [&](auto seti) {
    constexpr int SET = decltype(seti)::value;
#pragma unroll
    for (int i = 0; i < FFP; ++i) ps[i] = (int32_t)(psc[SET][i] >> (8 * hh));
#pragma unroll
    for (int j = 0; j < FFQ; ++j) qs[j] = (int32_t)(qsc[SET][j] >> (8 * hh));
  };

  f32x16 acc[FFP][FFQ];
#pragma unroll
  for (int i = 0; i < FFP; ++i)
#pragma unroll
    for (int j = 0; j < FFQ; ++j) acc[i][j] = f32x16{};

  // MFMA m of a slab: E4M3, one per block (i, j); E2M1, the first step of
  // every block, then the second.
  constexpr int NM = kFp4 ? 2 * FFP * FFQ : FFP * FFQ;
  auto mfma = [&](auto mi, auto seti) {
    constexpr int m = decltype(mi)::value, SET = decltype(seti)::value;
    constexpr int blk = m % (FFP * FFQ), i = blk / FFQ, j = blk % FFQ;
    if constexpr (kFp4) {
      constexpr int e = m / (FFP * FFQ);                         // k 0..63 or 64..127 of the slab
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(low_half(qf[SET][j][e]), low_half(pf[SET][i][e]),
                                                                   acc[i][j], FMT, FMT, 2 * e, qs[j], 2 * e, ps[i]);
    } else {
      const i32x8 qv = __builtin_shufflevector(qf[SET][j][0], qf[SET][j][1], 0, 1, 2, 3, 4, 5, 6, 7);
      const i32x8 pv = __builtin_shufflevector(pf[SET][i][0], pf[SET][i][1], 0, 1, 2, 3, 4, 5, 6, 7);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qv, pv, acc[i][j], FMT, FMT, 0, qs[j], 0, ps[i]);
    }
  };

  const int kbeg = t.kbeg;
  const int nk = (kend - kbeg) / KS;
  if (nk > 0) {
    static_for<3>([&](auto si) {
      constexpr int s = decltype(si)::value;
      static_for<T>([&](auto u) { issue(u, stage(si), kbeg + s * KS); });
    });
    barrier_vm<2 * T>();
    static_for<NREAD>([&](auto r) { read(r, IC<0>{}, stage(IC<0>{})); });
  }

  // Slab k = kt + J (stage J % 4): publish slab k+1, issue slab k+3 into the
  // stage of slab k-1 (all at once; spreading them over the MFMAs measured
  // the same in steady state), multiply slab k while reading slab k+1's
  // fragments.
  auto slab = [&](auto ji, int k) {
    constexpr int J = decltype(ji)::value;
    constexpr int CUR = J & 1, NXT = CUR ^ 1;
    barrier_vm<T>();
    uint8_t* const nxt = stage(IC<J + 1>{});
    uint8_t* const dst = stage(IC<J + 3>{});
    const int k3 = kbeg + (k + 3) * KS;
    scales(IC<CUR>{});
    static_for<T>([&](auto ui) { issue(ui, dst, k3); });         // all of slab k+3's loads first
    static_for<NM>([&](auto mi) {
      constexpr int m = decltype(mi)::value;
      mfma(mi, IC<CUR>{});
      static_for<NREAD>([&](auto ri) {
        if constexpr (decltype(ri)::value * NM / NREAD == m) read(ri, IC<NXT>{}, nxt);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int kt = 0; kt < nk; kt += 4) {
    static_for<4>([&](auto ji) {
      constexpr int J = decltype(ji)::value;
      if (kt + J < nk) slab(ji, kt + J);
    });
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  uint8_t* stg = wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3;
  store_acc<FCfg, false>(p, t, acc, wp, wq, lane, stg);
}

}  // namespace

hipError_t fwd_mx(const Params& prm, bool fp4, hipStream_t s) {
  if (prm.ntiles <= 0) return hipSuccess;
  if (fp4)
    mx_fwd_kernel<true><<<dim3(prm.ntiles), dim3(NT), 0, s>>>(prm);
  else
    mx_fwd_kernel<false><<<dim3(prm.ntiles), dim3(NT), 0, s>>>(prm);
  return hipGetLastError();
}

}  // namespace gk
}  // namespace lp
