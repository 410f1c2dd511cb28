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
// Tiles: 256 x 256 outputs, four waves of 128 x 128.  A slab is 64 bytes
// per row of each operand (64 E4M3 or 128 E2M1 values); a stage holds two
// slabs, so that every row's direct load is one whole 128-byte line.  Both
// code tiles are [row][128 B] with 16-byte chunk c of row r at
// c ^ ((r >> 1) & 7): the 16 rows of a fragment read hit 16 distinct slots
// mod 256 B.  A lane's two chunks of a fragment in slab s, 4 s + h and
// 4 s + 2 + h, make one E4M3 operand or the operands of two E2M1 steps.
// Each slab's scales (2 or 4 bytes per row and operand) come with the codes
// as one zero-extended dword per row.
//
// Two stages of 68 KiB.  Schedule, in slabs h (stage j = h / 2 in buffer
// j % 2): the fragments of slab h + 1 are read during the MFMAs of slab h;
// at the start of every odd slab 2j+1 one barrier (all loads landed)
// publishes stage j+1, issued at the start of slab 2j-1, and frees buffer
// j % 2, whose fragments every wave then holds; stage j+2's loads go into
// it at once.  The load lead is two slabs, as with single-slab stages four
// deep, and a tile issues no stage past its contraction.
#include "lp_gemm_kernel.hpp"

namespace lp {
namespace gk {
namespace {

constexpr int FBP = 256, FBQ = 256;             // output tile
constexpr int FWP = 128, FWQ = 128;             // wave tile
constexpr int FFP = 4, FFQ = 4;                 // 32 x 32 blocks per wave
constexpr int kRowBytes = 64;                   // code bytes per row and slab
constexpr int kLine = 2 * kRowBytes;            // code bytes per row and stage
constexpr int kOpBytes = FBP * kLine;           // one operand's codes per stage
constexpr int kScaleBytes = FBP * 4;            // one operand's scales per slab (a dword per row)
constexpr int kScaleBase = 2 * kOpBytes;        // scales of slab s, operand o at + (2 s + o) kScaleBytes
constexpr int kStage = kScaleBase + 4 * kScaleBytes;
constexpr int T = 20;                           // direct loads per wave and stage
using FCfg = Cfg<FBP, FBQ>;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int f_swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ i32x8 low_half(i32x4 v) { return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1); }

template <bool kFp4>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void mx_fwd_kernel(Params p) {
  constexpr int KS = kFp4 ? 128 : 64;            // contraction elements per slab
  constexpr int FMT = kFp4 ? 4 : 0;              // MFMA operand format
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kStage];
  static_assert(kMaxGroups * 4 <= kStage, "group ends alias stage 0");
  static_assert(2 * FWP * FWQ * 2 <= kStage, "two waves' epilogue staging fits a stage");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave >> 1, wq = wave & 1;
  const Tile t = select_tile<FCfg, false>(p, reinterpret_cast<int32_t*>(s0));
  if (!t.valid) return;
  __syncthreads();                                               // group ends read; stage 0 reusable

  const int ldp = p.P.code_ld, ldq = p.Q.code_ld;                // code bytes per x / w row
  const int sldp = p.P.scale_ld, sldq = p.Q.scale_ld;            // scale bytes per row (K / 32)
  const int kbeg = t.kbeg, kend = t.kend;                        // K, a multiple of KS
  const int64_t prows = (int64_t)(p.Ptot - t.p0), qrows = (int64_t)(p.Qtot - t.q0);
  const uint8_t* pc = p.P.codes + (int64_t)t.p0 * ldp;
  const uint8_t* qc = p.Q.codes + (int64_t)t.g * p.Q.code_batch + (int64_t)t.q0 * ldq;
  const Rsrc ps_r = make_rsrc(p.P.scales + (int64_t)t.p0 * sldp, prows * sldp);
  const Rsrc qs_r = make_rsrc(p.Q.scales + (int64_t)t.g * p.Q.scale_batch + (int64_t)t.q0 * sldq, qrows * sldq);

  // Code loads: wave w fills blocks 8 w + u (u = 0..7) of 8 rows x 128 B;
  // lane i takes row 64 w + 8 u + i / 8 and physical chunk i % 8, whose
  // logical chunk (i % 8) ^ f_swz(row) = (i % 8) ^ (4 (u & 1) + i / 16)
  // depends on u's parity only.  Rows past the operand's end read as zeros.
  const int c_even = (lane & 7) ^ (lane >> 4), c_odd = (lane & 7) ^ (4 + (lane >> 4));
  const int32_t p_row = (64 * wave + lane / 8) * ldp, q_row = (64 * wave + lane / 8) * ldq;   // + 8 u ld
  // Scale loads: wave w brings rows 64 w + i of each operand and slab.
  const int32_t ps_off = (64 * wave + lane) * sldp, qs_off = (64 * wave + lane) * sldq;

  auto stage = [&](auto si) -> uint8_t* {
    if constexpr (decltype(si)::value % 2 == 0) return s0;
    else return s1;
  };

  // Load u of the stage at contraction k0: x codes (0..7), w codes
  // (8..15), then the scales of slab s, operand o (16 + 2 s + o).
  auto issue = [&](auto ui, uint8_t* sb, int k0) {
    constexpr int u = decltype(ui)::value;
    const int kb = k0 * kRowBytes / KS;                          // byte offset of the stage in a row
    if constexpr (u < 8) {
      const Rsrc r = make_rsrc(pc + kb, prows * ldp - kb);
      dma<16>(r, (lds_void*)(sb + 1024 * (8 * wave + u)), p_row + 16 * ((u & 1) ? c_odd : c_even), 8 * u * ldp);
    } else if constexpr (u < 16) {
      constexpr int v = u - 8;
      const Rsrc r = make_rsrc(qc + kb, qrows * ldq - kb);
      dma<16>(r, (lds_void*)(sb + kOpBytes + 1024 * (8 * wave + v)), q_row + 16 * ((v & 1) ? c_odd : c_even),
              8 * v * ldq);
    } else {
      constexpr int s = (u - 16) / 2, o = (u - 16) % 2;
      const Rsrc r = o == 0 ? ps_r : qs_r;
      uint8_t* dst = sb + kScaleBase + (2 * s + o) * kScaleBytes + 256 * wave;
      if constexpr (kFp4)
        dma<4>(r, (lds_void*)dst, o == 0 ? ps_off : qs_off, (k0 + s * KS) / 32);
      else
        dma<2>(r, (lds_void*)dst, o == 0 ? ps_off : qs_off, (k0 + s * KS) / 32);
    }
  };

  // Fragment f (or j) of lane l in slab s of a stage: row 128 wp (128 wq)
  // + 32 f + l % 32, logical chunks 4 s + h and 4 s + 2 + h (h = l / 32);
  // the swizzle of the row depends on l % 32 only.
  const int r32 = lane & 31, hh = lane >> 5;
  int32_t fa[2][2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int e = 0; e < 2; ++e) fa[s2][e] = r32 * kLine + 16 * ((4 * s2 + 2 * e + hh) ^ f_swz(r32));
  const int32_t pa = wp * FWP * kLine, qa = kOpBytes + wq * FWQ * kLine;
  const int32_t psa = kScaleBase + (wp * FWP + r32) * 4, qsa = kScaleBase + kScaleBytes + (wq * FWQ + r32) * 4;

  i32x4 pf[2][FFP][2], qf[2][FFQ][2];
  uint32_t psc[2][FFP], qsc[2][FFQ];
  constexpr int NREAD = 2 * FFP + 2 * FFQ + FFP + FFQ;
  // Read r of slab SS of the stage in sb into register set SET: x chunks,
  // w chunks, then the scale dwords.  Nothing here computes on a loaded
  // value: an operation on one would make the wave wait for every LDS read
  // in flight in the middle of the MFMA stream.
  auto read = [&](auto ri, auto seti, auto ssi, const uint8_t* sb) {
    constexpr int r = decltype(ri)::value, SET = decltype(seti)::value, SS = decltype(ssi)::value;
    if constexpr (r < 2 * FFP) {
      constexpr int f = r / 2, e = r % 2;
      pf[SET][f][e] = *reinterpret_cast<const i32x4*>(sb + pa + fa[SS][e] + f * 32 * kLine);
    } else if constexpr (r < 2 * FFP + 2 * FFQ) {
      constexpr int j = (r - 2 * FFP) / 2, e = (r - 2 * FFP) % 2;
      qf[SET][j][e] = *reinterpret_cast<const i32x4*>(sb + qa + fa[SS][e] + j * 32 * kLine);
    } else if constexpr (r < 2 * FFP + 2 * FFQ + FFP) {
      constexpr int f = r - 2 * FFP - 2 * FFQ;
      psc[SET][f] = *reinterpret_cast<const uint32_t*>(sb + psa + 2 * SS * kScaleBytes + f * 32 * 4);
    } else {
      constexpr int j = r - 2 * FFP - 2 * FFQ - FFP;
      qsc[SET][j] = *reinterpret_cast<const uint32_t*>(sb + qsa + 2 * SS * kScaleBytes + j * 32 * 4);
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

  const int nh = (kend - kbeg) / KS;                             // slabs
  const int nst = (nh + 1) / 2;                                  // stages
  if (nh > 0) {
    static_for<T>([&](auto u) { issue(u, s0, kbeg); });
    if (nst > 1) {
      static_for<T>([&](auto u) { issue(u, s1, kbeg + 2 * KS); });
      barrier_vm<T>();
    } else {
      barrier_vm<0>();
    }
    static_for<NREAD>([&](auto r) { read(r, IC<0>{}, IC<0>{}, s0); });
  }

  // Slab h (H = h mod 4: stage buffer H / 2, slab SS = H % 2 of it).
  auto slab = [&](auto hi, int h) {
    constexpr int H = decltype(hi)::value;
    constexpr int SS = H % 2, CUR = H & 1, NXT = CUR ^ 1;
    uint8_t* const cur = stage(IC<H / 2>{});
    uint8_t* const nsb = stage(IC<(H + 1) / 2>{});
    if constexpr (SS == 1) {
      barrier_vm<0>();
      const int j2 = h / 2 + 2;
      if (j2 < nst) static_for<T>([&](auto ui) { issue(ui, cur, kbeg + 2 * KS * j2); });
    }
    scales(IC<CUR>{});
    static_for<NM>([&](auto mi) {
      constexpr int m = decltype(mi)::value;
      mfma(mi, IC<CUR>{});
      static_for<NREAD>([&](auto ri) {
        if constexpr (decltype(ri)::value * NM / NREAD == m) read(ri, IC<NXT>{}, IC<SS ^ 1>{}, nsb);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int ht = 0; ht < nh; ht += 4) {
    static_for<4>([&](auto hi) {
      constexpr int H = decltype(hi)::value;
      if (ht + H < nh) slab(hi, ht + H);
    });
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  uint8_t* stg = (wp == 0 ? s0 : s1) + wq * (FWP * FWQ * 2);
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
