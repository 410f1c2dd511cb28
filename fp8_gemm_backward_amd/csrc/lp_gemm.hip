// Fused dequantize + bf16 MFMA backward contractions (dense and grouped).
//
// "Add Autograd Backward Support for FP4 GEMM Custom Ops", Implementation
// Method: grad_X = grad_output @ W_bf16 and grad_W = grad_output.T @ X_bf16
// after dequantizing the saved operands; "Train adapters on top of FP8
// weights", FP8GroupedMatmulFunction.backward: the rows of each group
// (int32 cumulative end offsets) multiply that group's weight, rows past the
// last offset are skipped; "perf: defer mxfp8 backward quantization",
// MXFP8GMMFunction.op_dx: the same contraction with MX-quantized operands.
//
// Notation: the output tile is P x Q (P = rows of the output, Q = its
// columns, always the layer input dim K); the contraction runs over "k".
//   dx: out[m][q] = sum_n grad[m][n] * W[g][n][q]   P = m, k = n
//   dw: out[g][n][q] = sum_m grad[m][n] * X[m][q]   P = n, k = m (group rows)
//
// Each workgroup owns one BP x BQ output tile.  Per BK = 64 slab of the
// contraction it loads the packed codes and scales of both operands into
// registers (one 16-byte load per chunk), decodes them once for the whole
// workgroup into bf16 tiles in LDS, and runs v_mfma_f32_32x32x16_bf16 on
// them.  The next slab's global loads are issued before the current slab's
// MFMAs and LDS is double-buffered, so there is one barrier per slab.
//
// LDS layouts: an operand whose contraction index is contiguous in memory
// (grad in dx, "k-major") is stored [mn][k] and read with ds_read_b128; an
// operand whose contraction runs along its rows (W in dx, grad and X in dw,
// "mn-major") is stored [k][mn] exactly as loaded and read with
// ds_read_b64_tr_b16, which hands lane i of each 16-lane group column i of
// four consecutive rows, i.e. the MFMA operand layout.
//
// The MFMA is issued as D = Qfrag x Pfrag so that each lane's accumulator
// holds four consecutive output columns, stored as one 8-byte write.
#include "lp_device.hpp"
#include "lp_internal.hpp"

namespace lp {

namespace {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int BK = 64;
constexpr int kMaxGroups = 1024;

// One operand as the kernel sees it.
struct Op {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tensor_scale;
  int64_t code_batch;    // bytes between groups (grouped weight), else 0
  int64_t scale_batch;   // bytes between groups' scale grids
  int32_t code_ld;       // bytes per row of codes
  int32_t scale_ld;      // scale entries per row of the scale grid
  int32_t cols;          // logical columns (bounds of the mn index)
};

struct Params {
  Op P, Q;
  uint16_t* C;
  int64_t c_batch;       // elements between output groups (dw), else 0
  int32_t ldc;           // = Qtot
  int32_t Ptot;          // output rows: M (dx) or N (dw)
  int32_t Qtot;          // output columns: K
  int32_t Ktot;          // contraction length: N (dx) or M (dw)
  const int32_t* offsets;
  int32_t groups;
  int32_t np, nq;        // P- and Q-tiles (np per group for dw; dx computes per group)
  int32_t ntiles;        // grid size
};

template <int kBP, int kBQ, int kNWP, int kNWQ>
struct Cfg {
  static constexpr int BP = kBP, BQ = kBQ, NWP = kNWP, NWQ = kNWQ;
  static constexpr int NT = 64 * NWP * NWQ;
  static constexpr int WP = BP / NWP, WQ = BQ / NWQ;   // wave tile
  static constexpr int FP = WP / 32, FQ = WQ / 32;     // 32x32 MFMA blocks per wave
  static constexpr int PK = BK + 8;                    // k-major LDS pitch (bf16)
  static constexpr int PMP = BP + 32;                  // mn-major LDS pitch for P
  static constexpr int PMQ = BQ + 32;                  // mn-major LDS pitch for Q
};

// Codes per 16-byte chunk.
template <int F>
constexpr int elems_per_chunk() {
  return F == BF16 ? 8 : ((F == MXFP4 || F == NVFP4) ? 32 : 16);
}

// Raw (undecoded) contents of one chunk: 16 code bytes plus its scale
// information.  `s` holds up to 16 scale bytes (MXFP8 along rows) or one
// fp32 / E8M0 / pair of E4M3 scales in s[0].
struct Raw {
  u32x4 c;
  u32x4 s;
};

// Load the raw chunk at (row gk, column gm) of an operand; zero when out of
// range.  Zero codes with zero scales decode to +0.
template <int F, int A>
__device__ __forceinline__ Raw load_chunk(const Op& op, int64_t cbase, int64_t sbase, int gk, int gm, bool valid) {
  Raw r;
  r.c = u32x4{0, 0, 0, 0};
  r.s = u32x4{0, 0, 0, 0};
  if (!valid) return r;
  constexpr int bytes_num = (F == BF16) ? 2 : 1;   // bytes per element = num/den
  constexpr int bytes_den = (F == MXFP4 || F == NVFP4) ? 2 : 1;
  const uint8_t* cp = op.codes + cbase + (int64_t)gk * op.code_ld + (int64_t)gm * bytes_num / bytes_den;
  r.c = *reinterpret_cast<const u32x4*>(cp);
  const uint8_t* sp = op.scales + sbase;
  if constexpr (F == FP8_B128) {
    r.s[0] = reinterpret_cast<const uint32_t*>(sp)[(int64_t)(gk >> 7) * op.scale_ld + (gm >> 7)];
  } else if constexpr (F == MXFP4 || (F == MXFP8 && A == -1)) {
    r.s[0] = sp[(int64_t)gk * op.scale_ld + (gm >> 5)];
  } else if constexpr (F == NVFP4) {
    r.s[0] = *reinterpret_cast<const uint16_t*>(sp + (int64_t)gk * op.scale_ld + (gm >> 4));
  } else if constexpr (F == MXFP8 && A == -2) {
    r.s = *reinterpret_cast<const u32x4*>(sp + (int64_t)(gk >> 5) * op.scale_ld + gm);
  }
  return r;
}

// Decode a raw chunk to bf16 (EPC/2 dwords).  Values equal the standalone
// dequantization except that NaN payloads are left as the hardware makes them.
template <int F, int A>
__device__ __forceinline__ void decode_chunk(const Raw& r, float ts, uint32_t* o) {
  if constexpr (F == BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = r.c[j];
  } else if constexpr (F == MXFP4) {
    float cs = e8m0_to_cvt_scale(r.s[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) fp4x8_to_bf16_pow2(r.c[j], cs, o + 4 * j);
  } else if constexpr (F == NVFP4) {
    f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.s[0], 1.0f, false);
    float S0 = sv[0] * ts, S1 = sv[1] * ts;
    fp4x8_to_bf16_mul(r.c[0], S0, o + 0);
    fp4x8_to_bf16_mul(r.c[1], S0, o + 4);
    fp4x8_to_bf16_mul(r.c[2], S1, o + 8);
    fp4x8_to_bf16_mul(r.c[3], S1, o + 12);
  } else if constexpr (F == FP8_B128) {
    float S = __builtin_bit_cast(float, r.s[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) fp8x4_to_bf16_mul(r.c[j], S, o + 2 * j);
  } else if constexpr (F == MXFP8 && A == -1) {
    float cs = e8m0_to_cvt_scale(r.s[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) fp8x4_to_bf16_pow2(r.c[j], cs, o + 2 * j);
  } else {  // MXFP8 along rows: one scale byte per column
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t sw = r.s[j];
      float s0 = e8m0_to_cvt_scale(sw & 0xFFu);
      float s1 = e8m0_to_cvt_scale((sw >> 8) & 0xFFu);
      float s2 = e8m0_to_cvt_scale((sw >> 16) & 0xFFu);
      float s3 = e8m0_to_cvt_scale(sw >> 24);
      uint32_t a = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.c[j], s0, false));
      uint32_t b = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.c[j], s1, false));
      uint32_t c = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.c[j], s2, true));
      uint32_t d = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.c[j], s3, true));
      o[2 * j] = (a & 0xFFFFu) | (b & 0xFFFF0000u);
      o[2 * j + 1] = (c & 0xFFFFu) | (d & 0xFFFF0000u);
    }
  }
}

// Operand tile loader.  kKMajor: tile is R=BMN rows (mn) x BK columns (k) of
// the tensor; otherwise BK rows (k) x BMN columns (mn).
template <int F, int A, bool kKMajor, int BMN, int NT>
struct Loader {
  static constexpr int EPC = elems_per_chunk<F>();
  static constexpr int CPR = kKMajor ? BK / EPC : BMN / EPC;        // chunks per tile row
  static constexpr int CHUNKS = kKMajor ? BMN * CPR : BK * CPR;
  static constexpr int PER = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "tile not evenly divided among threads");
  static constexpr int PITCH = kKMajor ? BK + 8 : BMN + 32;        // LDS pitch in bf16
  static constexpr int LDS_ELEMS = kKMajor ? BMN * PITCH : BK * PITCH;

  Raw raw[PER];
  float ts;

  // k0: first contraction index of the slab; kend: end of the contraction
  // range; mn0 / mnend: the tile's mn range.
  __device__ __forceinline__ void load(const Op& op, int64_t cbase, int64_t sbase, int k0, int kend, int mn0,
                                       int mnend) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = threadIdx.x + i * NT;
      int row = c / CPR, col = (c % CPR) * EPC;
      if constexpr (kKMajor) {
        int gm = mn0 + row, gk = k0 + col;
        raw[i] = load_chunk<F, A>(op, cbase, sbase, gm, gk, gm < mnend && gk < kend);
      } else {
        int gk = k0 + row, gm = mn0 + col;
        raw[i] = load_chunk<F, A>(op, cbase, sbase, gk, gm, gk < kend && gm < mnend);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = threadIdx.x + i * NT;
      int row = c / CPR, col = (c % CPR) * EPC;
      uint32_t o[EPC / 2];
      decode_chunk<F, A>(raw[i], ts, o);
      u32x4* dst = reinterpret_cast<u32x4*>(lds + row * PITCH + col);
#pragma unroll
      for (int j = 0; j < EPC / 8; ++j) dst[j] = u32x4{o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
    }
  }
};

// k-major fragment: lane holds row (mn) `base + lane%32`, k = kk + (lane/32)*8 .. +7.
template <int PITCH>
__device__ __forceinline__ bf16x8 frag_kmajor(const uint16_t* lds, int base, int kk, int lane) {
  const uint16_t* p = lds + (base + (lane & 31)) * PITCH + kk + (lane >> 5) * 8;
  return *reinterpret_cast<const bf16x8*>(p);
}

// mn-major fragment (LDS [k][mn]): lane holds column `base + lane%32` at the
// same k's, assembled from two transposing reads of four rows each.
template <int PITCH>
__device__ __forceinline__ bf16x8 frag_mnmajor(const uint16_t* lds, int base, int kk, int lane) {
  int i16 = lane & 15, grp = lane >> 4;
  int row = kk + (grp >> 1) * 8 + (i16 >> 2);
  int col = base + (grp & 1) * 16 + (i16 & 3) * 4;
  const uint16_t* p = lds + row * PITCH + col;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * PITCH));
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
  i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Map the hardware workgroup id so that each XCD (workgroups are dealt to
// the 8 XCDs round-robin) receives a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int hw, int n) {
  constexpr int X = 8;
  int per = n / X, rem = n % X;
  int x = hw % X, j = hw / X;
  return x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

template <class C, int PF, int PA, int QF, int QA, bool kDW>
__global__ __launch_bounds__(C::NT) void gemm_kernel(Params p) {
  using LP = Loader<PF, PA, !kDW, C::BP, C::NT>;
  using LQ = Loader<QF, QA, false, C::BQ, C::NT>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (LP::LDS_ELEMS + LQ::LDS_ELEMS)];
  __shared__ int32_t s_ends[kMaxGroups];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave / C::NWQ, wq = wave % C::NWQ;
  const int tile = xcd_remap(blockIdx.x, p.ntiles);

  // ---- which output tile, group and contraction range
  int g = 0, p0, pend, q0, kbeg = 0, kend = p.Ktot;
  if constexpr (!kDW) {
    // Groups partition the output rows; tiles never straddle a group.
    int pidx = tile / p.nq;
    q0 = (tile % p.nq) * C::BQ;
    if (p.offsets == nullptr) {
      p0 = pidx * C::BP;
      pend = p.Ptot;
    } else {
      for (int i = tid; i < p.groups; i += C::NT) s_ends[i] = p.offsets[i];
      __syncthreads();
      int start = 0, seen = 0;
      p0 = -1;
      pend = 0;
      for (int gi = 0; gi < p.groups; ++gi) {
        int e = s_ends[gi];
        e = e < start ? start : (e > p.Ptot ? p.Ptot : e);        // clamp into [start, M]
        int t = (e - start + C::BP - 1) / C::BP;
        if (pidx < seen + t) {
          g = gi;
          p0 = start + (pidx - seen) * C::BP;
          pend = e;
          break;
        }
        seen += t;
        start = e;
      }
      if (p0 < 0) return;                                        // past the last tile
    }
    if (p0 >= pend) return;
  } else {
    // Groups partition the contraction; every group has np x nq tiles.
    const int per_group = p.np * p.nq;
    g = tile / per_group;
    int t = tile % per_group;
    p0 = (t / p.nq) * C::BP;
    q0 = (t % p.nq) * C::BQ;
    pend = p.Ptot;
    if (p.offsets != nullptr) {
      // The same clamped chain as for dx: end_g = clamp(offsets[g], end_{g-1}, M).
      for (int i = tid; i < p.groups; i += C::NT) s_ends[i] = p.offsets[i];
      __syncthreads();
      int start = 0, e = 0;
      for (int gi = 0; gi <= g; ++gi) {
        e = s_ends[gi];
        e = e < start ? start : (e > p.Ktot ? p.Ktot : e);
        if (gi < g) start = e;
      }
      kbeg = start;
      kend = e;
    }
  }

  // ---- operand bases
  const int64_t pcb = kDW ? 0 : 0, psb = 0;
  const int64_t qcb = kDW ? 0 : (int64_t)g * p.Q.code_batch;
  const int64_t qsb = kDW ? 0 : (int64_t)g * p.Q.scale_batch;

  LP lp;
  LQ lq;
  if constexpr (PF == NVFP4) lp.ts = *p.P.tensor_scale; else lp.ts = 0.0f;
  if constexpr (QF == NVFP4) lq.ts = *p.Q.tensor_scale; else lq.ts = 0.0f;

  // Stage s: P tile at smem + s*STAGE, Q tile right after it.
  constexpr int STAGE = LP::LDS_ELEMS + LQ::LDS_ELEMS;

  f32x16 acc[C::FP][C::FQ];
#pragma unroll
  for (int i = 0; i < C::FP; ++i)
#pragma unroll
    for (int j = 0; j < C::FQ; ++j) acc[i][j] = f32x16{};

  const int nk = (kend - kbeg + BK - 1) / BK;
  // P's mn range: output rows [p0, pend); Q's mn range: columns [q0, Qtot).
  if (nk > 0) {
    lp.load(p.P, pcb, psb, kbeg, kend, p0, pend);
    lq.load(p.Q, qcb, qsb, kbeg, kend, q0, p.Qtot);
    lp.store(smem);
    lq.store(smem + LP::LDS_ELEMS);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = kbeg + (kt + 1) * BK;
      lp.load(p.P, pcb, psb, k0, kend, p0, pend);
      lq.load(p.Q, qcb, qsb, k0, kend, q0, p.Qtot);
    }
    const uint16_t* sp = smem + cur * STAGE;
    const uint16_t* sq = sp + LP::LDS_ELEMS;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 pf[C::FP], qf[C::FQ];
#pragma unroll
      for (int i = 0; i < C::FP; ++i) {
        if constexpr (!kDW)
          pf[i] = frag_kmajor<LP::PITCH>(sp, wp * C::WP + i * 32, kk, lane);
        else
          pf[i] = frag_mnmajor<LP::PITCH>(sp, wp * C::WP + i * 32, kk, lane);
      }
#pragma unroll
      for (int j = 0; j < C::FQ; ++j) qf[j] = frag_mnmajor<LQ::PITCH>(sq, wq * C::WQ + j * 32, kk, lane);
#pragma unroll
      for (int i = 0; i < C::FP; ++i)
#pragma unroll
        for (int j = 0; j < C::FQ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[j], pf[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      lp.store(smem + (cur ^ 1) * STAGE);
      lq.store(smem + (cur ^ 1) * STAGE + LP::LDS_ELEMS);
    }
    __syncthreads();
  }

  // ---- epilogue: fp32 -> bf16 (nearest even), masked 8-byte stores
  uint16_t* out = p.C + (kDW ? (int64_t)g * p.c_batch : 0);
#pragma unroll
  for (int i = 0; i < C::FP; ++i) {
    const int row = p0 + wp * C::WP + i * 32 + (lane & 31);
    if (row >= pend) continue;
#pragma unroll
    for (int j = 0; j < C::FQ; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = q0 + wq * C::WQ + j * 32 + 8 * r4 + 4 * (lane >> 5);
        if (col < p.Qtot) {
          u32x2 v = {pack_bf16x2(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1]),
                     pack_bf16x2(acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3])};
          *reinterpret_cast<u32x2*>(out + (int64_t)row * p.ldc + col) = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- host side

Op make_op(const lp_qtensor& t) {
  Op o{};
  o.codes = static_cast<const uint8_t*>(t.codes);
  o.scales = static_cast<const uint8_t*>(t.scales);
  o.tensor_scale = t.tensor_scale;
  o.cols = (int32_t)t.cols;
  const int64_t R = t.rows, Cc = t.cols;
  switch (t.fmt) {
    case LP_BF16:
      o.code_ld = (int32_t)(Cc * 2);
      o.code_batch = R * Cc * 2;
      break;
    case LP_MXFP4:
      o.code_ld = (int32_t)(Cc / 2);
      o.code_batch = R * Cc / 2;
      o.scale_ld = (int32_t)(Cc / 32);
      o.scale_batch = R * (Cc / 32);
      break;
    case LP_NVFP4:
      o.code_ld = (int32_t)(Cc / 2);
      o.code_batch = R * Cc / 2;
      o.scale_ld = (int32_t)(Cc / 16);
      o.scale_batch = R * (Cc / 16);
      break;
    case LP_FP8_B128:
      o.code_ld = (int32_t)Cc;
      o.code_batch = R * Cc;
      o.scale_ld = (int32_t)((Cc + 127) / 128);
      o.scale_batch = ((R + 127) / 128) * ((Cc + 127) / 128) * 4;
      break;
    case LP_MXFP8:
      o.code_ld = (int32_t)Cc;
      o.code_batch = R * Cc;
      if (t.scale_axis == -1) {
        o.scale_ld = (int32_t)(Cc / 32);
        o.scale_batch = R * (Cc / 32);
      } else {
        o.scale_ld = (int32_t)Cc;
        o.scale_batch = (R / 32) * Cc;
      }
      break;
  }
  return o;
}

template <class C, int PF, int PA, int QF, int QA, bool kDW>
hipError_t run(const Params& prm, hipStream_t stream) {
  if (prm.ntiles <= 0) return hipSuccess;
  gemm_kernel<C, PF, PA, QF, QA, kDW><<<dim3(prm.ntiles), dim3(C::NT), 0, stream>>>(prm);
  return hipGetLastError();
}

// Q-operand format dispatch.
template <class C, int PF, int PA, bool kDW>
hipError_t dispatch_q(const lp_qtensor& q, const Params& prm, hipStream_t s) {
  switch (q.fmt) {
    case LP_BF16: return run<C, PF, PA, BF16, -1, kDW>(prm, s);
    case LP_MXFP4: return run<C, PF, PA, MXFP4, -1, kDW>(prm, s);
    case LP_NVFP4: return run<C, PF, PA, NVFP4, -1, kDW>(prm, s);
    case LP_FP8_B128: return run<C, PF, PA, FP8_B128, -1, kDW>(prm, s);
    case LP_MXFP8:
      return q.scale_axis == -1 ? run<C, PF, PA, MXFP8, -1, kDW>(prm, s) : run<C, PF, PA, MXFP8, -2, kDW>(prm, s);
  }
  return hipErrorInvalidValue;
}

template <class C>
hipError_t launch_cfg(const GemmCall& call, Params prm, hipStream_t stream) {
  prm.nq = (int32_t)((prm.Qtot + C::BQ - 1) / C::BQ);
  if (!call.dw) {
    const int64_t ptiles = call.offsets ? (call.M / C::BP + call.groups) : (call.M + C::BP - 1) / C::BP;
    prm.np = 0;
    prm.ntiles = (int32_t)(ptiles * prm.nq);
    if (call.grad->fmt == LP_MXFP8) return dispatch_q<C, MXFP8, -1, false>(*call.other, prm, stream);
    return dispatch_q<C, BF16, -1, false>(*call.other, prm, stream);
  }
  prm.np = (int32_t)((prm.Ptot + C::BP - 1) / C::BP);
  prm.ntiles = prm.np * prm.nq * call.groups;
  return dispatch_q<C, BF16, -1, true>(*call.other, prm, stream);
}

using Big = Cfg<256, 256, 2, 4>;     // 512 threads, wave tile 128 x 64
using Narrow = Cfg<256, 128, 2, 2>;  // 256 threads, wave tile 128 x 64

}  // namespace

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
