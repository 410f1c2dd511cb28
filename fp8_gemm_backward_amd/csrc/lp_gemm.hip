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
// "mn-major") is stored [k][mn] and read with ds_read_b64_tr_b16, which hands
// lane i of each 16-lane group column i of four consecutive rows, i.e. the
// MFMA operand layout.
//
// Bank rules of the gfx950 LDS (measured): a 16-byte write serves 8 lanes per
// cycle and is conflict-free when their 16-byte slots differ modulo 128 bytes;
// a 16-byte read serves 16 lanes per cycle (slots distinct modulo 256 bytes);
// the transposing 8-byte read serves 32 lanes, i.e. four rows of 64 bytes,
// which must fall in distinct quarters of 256 bytes.  The k-major tile uses a
// 144-byte row pitch (both directions conflict-free).  The mn-major tile uses
// a pitch of 64 mod 256 bytes (rows land in distinct quarters for the
// transposing read) and XORs the low two bits of the 16-byte chunk index
// with bits 1..2 of the row; eight consecutive lanes decode the same columns
// of eight consecutive rows, so their writes hit eight distinct slots.
//
// The MFMA is issued as D = Qfrag x Pfrag so that each lane's accumulator
// holds four consecutive output columns, stored as one 8-byte write.
#include <type_traits>

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
  int64_t code_batch;    // bytes between groups' codes (grouped weight)
  int64_t scale_batch;   // bytes between groups' scale grids
  int64_t scale_bytes;   // bytes of one group's scale grid
  int32_t code_ld;       // bytes per row of codes
  int32_t scale_ld;      // bytes per row of the scale grid
  int32_t rows;          // rows per group
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

template <int kBP, int kBQ, int kNWP, int kNWQ, bool kPP>
struct Cfg {
  static constexpr int BP = kBP, BQ = kBQ, NWP = kNWP, NWQ = kNWQ;
  static constexpr bool PINGPONG = kPP;                // two alternating wave groups
  static constexpr int NT = 64 * NWP * NWQ;
  static constexpr int WP = BP / NWP, WQ = BQ / NWQ;   // wave tile
  static constexpr int FP = WP / 32, FQ = WQ / 32;     // 32x32 MFMA blocks per wave
};

// ---------------------------------------------------------------- buffer loads
// Every global read goes through a buffer resource whose range ends where the
// valid data ends; reads past it return zero without touching memory.  This
// zero-fills contraction tails and out-of-range rows without branches.

typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int32_t kOOB = (int32_t)0x80000000;   // an offset beyond any range

__device__ __forceinline__ Rsrc make_rsrc(const void* base, int64_t bytes) {
  bytes = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(Rsrc r, int32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Codes per 16-byte chunk.
template <int F>
constexpr int elems_per_chunk() {
  return F == BF16 ? 8 : ((F == MXFP4 || F == NVFP4) ? 32 : 16);
}

// Undecoded contents of one chunk: 16 code bytes and its scale data (one
// E8M0 byte, a pair of E4M3 bytes, one fp32, or 16 E8M0 bytes for MXFP8 with
// scales along the rows).
template <int F, int A>
struct Raw {
  using S = std::conditional_t<(F == MXFP8 && A == -2), u32x4, uint32_t>;
  u32x4 c;
  S s;
};

// Decode a raw chunk to bf16 (EPC/2 dwords).  Values equal the standalone
// dequantization except that NaN payloads are left as the hardware makes them.
template <int F, int A>
__device__ __forceinline__ void decode_chunk(const Raw<F, A>& r, float ts, uint32_t* o) {
  if constexpr (F == BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = r.c[j];
  } else if constexpr (F == MXFP4) {
    float cs = e8m0_to_cvt_scale(r.s);   // the byte load zero-extends
#pragma unroll
    for (int j = 0; j < 4; ++j) fp4x8_to_bf16_pow2(r.c[j], cs, o + 4 * j);
  } else if constexpr (F == NVFP4) {
    f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.s, 1.0f, false);
    float S0 = sv[0] * ts, S1 = sv[1] * ts;
    fp4x8_to_bf16_mul(r.c[0], S0, o + 0);
    fp4x8_to_bf16_mul(r.c[1], S0, o + 4);
    fp4x8_to_bf16_mul(r.c[2], S1, o + 8);
    fp4x8_to_bf16_mul(r.c[3], S1, o + 12);
  } else if constexpr (F == FP8_B128) {
    float S = __builtin_bit_cast(float, r.s);
#pragma unroll
    for (int j = 0; j < 4; ++j) fp8x4_to_bf16_mul(r.c[j], S, o + 2 * j);
  } else if constexpr (F == MXFP8 && A == -1) {
    float cs = e8m0_to_cvt_scale(r.s);
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

// Operand tile loader.  kKMajor: the tile is BMN rows (mn) x BK columns (the
// contraction runs along the tensor's columns); otherwise BK rows (the
// contraction runs along its rows) x BMN columns.  Per-thread chunk
// positions are fixed for the whole k loop; only the window moves.
//
// NT threads share the work; with NSPLIT > 1 the tile's chunks are split into
// NSPLIT contiguous parts and this loader's threads own part `split`.
template <int F, int A, bool kKMajor, int BMN, int NT, int NSPLIT = 1>
struct Loader {
  static constexpr int EPC = elems_per_chunk<F>();
  static constexpr int CPR = kKMajor ? BK / EPC : BMN / EPC;        // chunks per tile row
  static constexpr int CHUNKS = kKMajor ? BMN * CPR : BK * CPR;
  static constexpr int PER = CHUNKS / (NT * NSPLIT);
  static_assert(CHUNKS % (NT * NSPLIT) == 0, "tile not evenly divided among threads");
  static constexpr int PITCH = kKMajor ? BK + 8 : BMN + 32;        // LDS pitch in bf16
  static constexpr int LDS_ELEMS = kKMajor ? BMN * PITCH : BK * PITCH;
  static constexpr int BPE2 = F == BF16 ? 4 : ((F == MXFP4 || F == NVFP4) ? 1 : 2);  // 2 x bytes per element

  using Stage = Raw<F, A>[PER];

  static constexpr int PIECES = EPC / 8;                            // 16-byte LDS writes per chunk

  int32_t voff[PER];     // code byte offset of each chunk inside the window
  int32_t row[PER];      // chunk's row in the tile
  int32_t lds[PER][PIECES];  // LDS offset (bf16 elements) of each 16-byte piece of the chunk
  int32_t mnc[PER];      // chunk's global mn index (mn-major) / column in the tile (k-major)
  const uint8_t* cbase;  // codes of this tile's group (and rows, k-major)
  const uint8_t* sbase;
  int64_t crows_bytes;   // k-major: bytes from cbase to the end of the tensor
  float ts;

  __device__ __forceinline__ void init(const Op& op, int g, int mn0, int mnend_rows, int t, int split) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = split * (CHUNKS / NSPLIT) + t + i * NT;
      // k-major: consecutive chunks run along a row.  mn-major: groups of
      // eight consecutive chunks run down eight rows at the same columns.
      const int r = kKMajor ? c / CPR : (c / (8 * CPR)) * 8 + (c & 7);
      const int col = kKMajor ? (c % CPR) * EPC : ((c >> 3) % CPR) * EPC;
      row[i] = r;
#pragma unroll
      for (int j = 0; j < PIECES; ++j) {
        if constexpr (kKMajor) {
          lds[i][j] = r * PITCH + col + 8 * j;
        } else {
          const int q = col / 8 + j;                                  // logical 16-byte chunk
          lds[i][j] = r * PITCH + 8 * ((q & ~3) | ((q & 3) ^ ((r >> 1) & 3)));
        }
      }
      if constexpr (kKMajor) {
        mnc[i] = col;
        voff[i] = r * op.code_ld + col * BPE2 / 2;
      } else {
        mnc[i] = mn0 + col;
        voff[i] = r * op.code_ld + (mn0 + col) * BPE2 / 2;
      }
    }
    if constexpr (kKMajor) {
      cbase = op.codes + (int64_t)mn0 * op.code_ld;
      sbase = op.scales + (int64_t)mn0 * op.scale_ld;
      crows_bytes = (int64_t)(mnend_rows - mn0) * op.code_ld;
    } else {
      cbase = op.codes + (int64_t)g * op.code_batch;
      sbase = op.scales + (int64_t)g * op.scale_batch;
      crows_bytes = 0;
    }
    if constexpr (F == NVFP4) ts = *op.tensor_scale; else ts = 0.0f;
  }

  // Issue the loads of the slab starting at contraction index k0 (reads
  // beyond kend come back as zero).  Never branches.
  __device__ __forceinline__ void load(Stage& st, const Op& op, int k0, int kend) const {
    if constexpr (kKMajor) {
      // window: this tile's rows, from column k0 on; columns >= kend masked.
      const Rsrc cr = make_rsrc(cbase + (int64_t)k0 * BPE2 / 2, crows_bytes - (int64_t)k0 * BPE2 / 2);
      const bool tail = k0 + BK > kend;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int off = (tail && k0 + mnc[i] >= kend) ? kOOB : voff[i];
        st[i].c = bload16(cr, off);
        if constexpr (F == MXFP8) {
          const Rsrc sr = make_rsrc(sbase + (k0 >> 5), crows_bytes / op.code_ld * op.scale_ld - (k0 >> 5));
          const int so = (tail && k0 + mnc[i] >= kend) ? kOOB : row[i] * op.scale_ld + (mnc[i] >> 5);
          st[i].s = __builtin_amdgcn_raw_buffer_load_b8(sr, so, 0, 0);
        }
      }
    } else {
      // window: rows [k0, kend) of this group's tensor.
      const int nrows = kend - k0;
      const Rsrc cr = make_rsrc(cbase + (int64_t)k0 * op.code_ld, (int64_t)nrows * op.code_ld);
#pragma unroll
      for (int i = 0; i < PER; ++i) st[i].c = bload16(cr, voff[i]);
      if constexpr (F == MXFP4 || (F == MXFP8 && A == -1) || F == NVFP4) {
        const Rsrc sr = make_rsrc(sbase + (int64_t)k0 * op.scale_ld, (int64_t)nrows * op.scale_ld);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int so = row[i] * op.scale_ld + (F == NVFP4 ? (mnc[i] >> 4) : (mnc[i] >> 5));
          if constexpr (F == NVFP4)
            st[i].s = __builtin_amdgcn_raw_buffer_load_b16(sr, so, 0, 0);
          else
            st[i].s = __builtin_amdgcn_raw_buffer_load_b8(sr, so, 0, 0);
        }
      } else if constexpr (F == FP8_B128 || F == MXFP8) {
        const Rsrc sr = make_rsrc(sbase, op.scale_bytes);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
          const int gk = k0 + row[i];
          if constexpr (F == FP8_B128) {
            const int so = gk < kend ? ((gk >> 7) * op.scale_ld + (mnc[i] >> 7) * 4) : kOOB;
            st[i].s = __builtin_amdgcn_raw_buffer_load_b32(sr, so, 0, 0);
          } else {
            const int so = gk < kend ? ((gk >> 5) * op.scale_ld + mnc[i]) : kOOB;
            st[i].s = bload16(sr, so);
          }
        }
      }
    }
  }

  // Decode and write the chunks i with i % NPARTS == PART (the store is
  // split so that its parts can be interleaved with a slab's MFMAs).
  template <int PART, int NPARTS>
  __device__ __forceinline__ void store_part(const Stage& st, uint16_t* buf) const {
#pragma unroll
    for (int i = PART; i < PER; i += NPARTS) {
      uint32_t o[EPC / 2];
      decode_chunk<F, A>(st[i], ts, o);
#pragma unroll
      for (int j = 0; j < PIECES; ++j)
        *reinterpret_cast<u32x4*>(buf + lds[i][j]) = u32x4{o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]};
    }
  }
  __device__ __forceinline__ void store(const Stage& st, uint16_t* buf) const { store_part<0, 1>(st, buf); }

  // LDS writes issued by store_part<PART, NPARTS>.
  static constexpr int writes(int part, int nparts) {
    int n = 0;
    for (int i = part; i < PER; i += nparts) n += EPC / 8;
    return n;
  }
  // Global loads issued by load().
  static constexpr int loads() {
    return PER * ((F == BF16) ? 1 : ((F == MXFP8 && A == -2) ? 2 : 2));
  }
};

// Scheduling pattern of one k-substep: N MFMAs, each followed by up to one
// LDS read, one global load, NV vector-ALU instructions and one LDS write,
// so that the fragment reads of the next substep and the decode of the next
// slab fill the issue slots while the matrix cores work.
template <int I, int N, int NDSR, int NVMEM, int NV, int NDSW>
__device__ __forceinline__ void interleave() {
  if constexpr (I < N) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
    if constexpr (I < NDSR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    if constexpr (I < NVMEM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0); // VMEM read
    if constexpr (I < NDSW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  // DS write
    interleave<I + 1, N, NDSR, NVMEM, NV, NDSW>();
  }
}

// k-major fragment: lane holds row (mn) `base + lane%32`, k = kk + (lane/32)*8 .. +7.
template <int PITCH>
__device__ __forceinline__ bf16x8 frag_kmajor(const uint16_t* lds, int base, int kk, int lane) {
  const uint16_t* p = lds + (base + (lane & 31)) * PITCH + kk + (lane >> 5) * 8;
  return *reinterpret_cast<const bf16x8*>(p);
}

// mn-major fragment (LDS [k][mn], swizzled as the loader stores it): lane
// holds column `base + lane%32` at the same k's, assembled from two
// transposing reads of four rows each.  base is a multiple of 32 and kk of
// 16, so the row's swizzle term depends on the lane only.
template <int PITCH>
__device__ __forceinline__ bf16x8 frag_mnmajor(const uint16_t* lds, int base, int kk, int lane) {
  const int i16 = lane & 15, grp = lane >> 4;
  const int row = kk + (grp >> 1) * 8 + (i16 >> 2);              // row % 8 == i16 / 4
  const int lc = (grp & 1) * 2 + ((i16 & 3) >> 1);                 // logical chunk in the fragment
  const int half = (i16 & 1) * 4;
  const int ha = (i16 >> 3) & 1, hb = 2 + ((i16 >> 3) & 1);        // ((row >> 1) & 3) for rows r, r + 4
  const uint16_t* pa = lds + row * PITCH + base + 8 * (lc ^ ha) + half;
  const uint16_t* pb = lds + (row + 4) * PITCH + base + 8 * (lc ^ hb) + half;
  i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pa));
  i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(pb));
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

// The output tile, group and contraction range of one workgroup.
struct Tile {
  int g, p0, pend, q0, kbeg, kend;
  bool valid;
};

// Map the workgroup to its tile.  s_ends: LDS for the group offsets.
template <class C, bool kDW>
__device__ __forceinline__ Tile select_tile(const Params& p, int32_t* s_ends) {
  const int tid = threadIdx.x;
  const int tile = xcd_remap(blockIdx.x, p.ntiles);
  Tile t{0, 0, 0, 0, 0, p.Ktot, true};
  if (p.offsets != nullptr) {
    for (int i = tid; i < p.groups; i += C::NT) s_ends[i] = p.offsets[i];
    __syncthreads();
  }
  if constexpr (!kDW) {
    // Groups partition the output rows; tiles never straddle a group.
    const int pidx = tile / p.nq;
    t.q0 = (tile % p.nq) * C::BQ;
    if (p.offsets == nullptr) {
      t.p0 = pidx * C::BP;
      t.pend = p.Ptot;
    } else {
      int start = 0, seen = 0;
      t.p0 = -1;
      for (int gi = 0; gi < p.groups; ++gi) {
        int e = s_ends[gi];
        e = e < start ? start : (e > p.Ptot ? p.Ptot : e);        // end_g = clamp(o_g, end_{g-1}, M)
        const int n = (e - start + C::BP - 1) / C::BP;
        if (pidx < seen + n) {
          t.g = gi;
          t.p0 = start + (pidx - seen) * C::BP;
          t.pend = e;
          break;
        }
        seen += n;
        start = e;
      }
    }
    t.valid = t.p0 >= 0 && t.p0 < t.pend;
  } else {
    // Groups partition the contraction; every group has np x nq tiles, whose
    // cost grows with the group's size.  Tiles are dealt round-robin over the
    // groups so that each XCD's contiguous range holds an equal share of
    // every group (dealing whole groups to XCDs would leave the XCD with the
    // largest group running long after the others).
    t.g = tile % p.groups;
    const int r = tile / p.groups;
    t.p0 = (r / p.nq) * C::BP;
    t.q0 = (r % p.nq) * C::BQ;
    t.pend = p.Ptot;
    if (p.offsets != nullptr) {
      int start = 0, e = 0;
      for (int gi = 0; gi <= t.g; ++gi) {
        e = s_ends[gi];
        e = e < start ? start : (e > p.Ktot ? p.Ktot : e);
        if (gi < t.g) start = e;
      }
      t.kbeg = start;
      t.kend = e;
    }
  }
  return t;
}

// fp32 -> bf16 (nearest even) and masked 8-byte stores of one wave's
// FP x FQ accumulator blocks (lane holds 4 consecutive output columns).
template <class C, bool kDW>
__device__ __forceinline__ void store_acc(const Params& p, const Tile& t, f32x16 (&acc)[C::FP][C::FQ], int wp,
                                          int wq, int lane) {
  uint16_t* out = p.C + (kDW ? (int64_t)t.g * p.c_batch : 0);
#pragma unroll
  for (int i = 0; i < C::FP; ++i) {
    const int row = t.p0 + wp * C::WP + i * 32 + (lane & 31);
    if (row >= t.pend) continue;
#pragma unroll
    for (int j = 0; j < C::FQ; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int col = t.q0 + wq * C::WQ + j * 32 + 8 * r4 + 4 * (lane >> 5);
        if (col < p.Qtot) {
          u32x2 v = {pack_bf16x2(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1]),
                     pack_bf16x2(acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3])};
          *reinterpret_cast<u32x2*>(out + (int64_t)row * p.ldc + col) = v;
        }
      }
    }
  }
}

// Fragments of one 16-deep k-substep and the MFMAs on them.
template <class C, bool kDW, int PPITCH, int QPITCH, int PELEMS>
struct Mma {
  bf16x8 p[C::FP];
  bf16x8 q[C::FQ];
  __device__ __forceinline__ void load(const uint16_t* sp, int kk, int wp, int wq, int lane) {
    const uint16_t* sq = sp + PELEMS;
#pragma unroll
    for (int i = 0; i < C::FP; ++i) {
      if constexpr (!kDW)
        p[i] = frag_kmajor<PPITCH>(sp, wp * C::WP + i * 32, kk, lane);
      else
        p[i] = frag_mnmajor<PPITCH>(sp, wp * C::WP + i * 32, kk, lane);
    }
#pragma unroll
    for (int j = 0; j < C::FQ; ++j) q[j] = frag_mnmajor<QPITCH>(sq, wq * C::WQ + j * 32, kk, lane);
  }
  __device__ __forceinline__ void run(f32x16 (&acc)[C::FP][C::FQ]) const {
#pragma unroll
    for (int i = 0; i < C::FP; ++i)
#pragma unroll
      for (int j = 0; j < C::FQ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q[j], p[i], acc[i][j], 0, 0, 0);
  }
};

// Single wave per SIMD: every wave multiplies, loads and decodes; slab k+2
// in flight and slab k+1 decoded into LDS (interleaved with the MFMAs by
// scheduling groups) while slab k is multiplied.
template <class C, int PF, int PA, int QF, int QA, bool kDW>
__global__ __launch_bounds__(C::NT) void gemm_kernel(Params p) {
  using LP = Loader<PF, PA, !kDW, C::BP, C::NT>;
  using LQ = Loader<QF, QA, false, C::BQ, C::NT>;
  using M = Mma<C, kDW, LP::PITCH, LQ::PITCH, LP::LDS_ELEMS>;
  constexpr int STAGE = LP::LDS_ELEMS + LQ::LDS_ELEMS;   // P tile, then Q tile
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  __shared__ int32_t s_ends[kMaxGroups];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave / C::NWQ, wq = wave % C::NWQ;
  const Tile t = select_tile<C, kDW>(p, s_ends);
  if (!t.valid) return;
  const int kend = t.kend, kbeg = t.kbeg;

  LP lp;
  LQ lq;
  // dx: P = grad rows [p0, pend) (k-major), Q = W[g] columns from q0.
  // dw: P = grad columns from p0, Q = X columns from q0, rows [kbeg, kend).
  lp.init(p.P, 0, t.p0, kDW ? 0 : p.P.rows, tid, 0);
  lq.init(p.Q, kDW ? 0 : t.g, t.q0, 0, tid, 0);

  f32x16 acc[C::FP][C::FQ];
#pragma unroll
  for (int i = 0; i < C::FP; ++i)
#pragma unroll
    for (int j = 0; j < C::FQ; ++j) acc[i][j] = f32x16{};

  constexpr int NM = C::FP * C::FQ;                                   // MFMAs per substep
  constexpr int NR = (kDW ? 2 * C::FP : C::FP) + 2 * C::FQ;          // fragment reads per substep
  constexpr int NL = LP::loads() + LQ::loads();                       // global loads per slab
  auto kstep = [&](typename LP::Stage& ldp, typename LQ::Stage& ldq, int kload, const typename LP::Stage& stp,
                   const typename LQ::Stage& stq, const uint16_t* cur, uint16_t* nxt) {
    M fa, fb;
    fa.load(cur, 0, wp, wq, lane);
    __builtin_amdgcn_sched_barrier(0);
    lp.load(ldp, p.P, kload, kend);
    lq.load(ldq, p.Q, kload, kend);
    fb.load(cur, 16, wp, wq, lane);
    lp.template store_part<0, 4>(stp, nxt);
    lq.template store_part<0, 4>(stq, nxt + LP::LDS_ELEMS);
    fa.run(acc);
    interleave<0, NM, NR, NL, 0, LP::writes(0, 4) + LQ::writes(0, 4)>();
    __builtin_amdgcn_sched_barrier(0);
    fa.load(cur, 32, wp, wq, lane);
    lp.template store_part<1, 4>(stp, nxt);
    lq.template store_part<1, 4>(stq, nxt + LP::LDS_ELEMS);
    fb.run(acc);
    interleave<0, NM, NR, 0, 0, LP::writes(1, 4) + LQ::writes(1, 4)>();
    __builtin_amdgcn_sched_barrier(0);
    fb.load(cur, 48, wp, wq, lane);
    lp.template store_part<2, 4>(stp, nxt);
    lq.template store_part<2, 4>(stq, nxt + LP::LDS_ELEMS);
    fa.run(acc);
    interleave<0, NM, NR, 0, 0, LP::writes(2, 4) + LQ::writes(2, 4)>();
    __builtin_amdgcn_sched_barrier(0);
    lp.template store_part<3, 4>(stp, nxt);
    lq.template store_part<3, 4>(stq, nxt + LP::LDS_ELEMS);
    fb.run(acc);
    interleave<0, NM, 0, 0, 0, LP::writes(3, 4) + LQ::writes(3, 4)>();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };

  // Two register stages (A, B) and two LDS buffers; the slab count is
  // rounded up to even so the body has no branch (slabs past the
  // contraction end load as zeros and add nothing).
  const int nk = (kend - kbeg + BK - 1) / BK;
  const int nk2 = (nk + 1) & ~1;
  typename LP::Stage pa, pb;
  typename LQ::Stage qa, qb;
  uint16_t* buf0 = smem;
  uint16_t* buf1 = smem + STAGE;
  if (nk > 0) {
    lp.load(pa, p.P, kbeg, kend);
    lq.load(qa, p.Q, kbeg, kend);
    lp.load(pb, p.P, kbeg + BK, kend);
    lq.load(qb, p.Q, kbeg + BK, kend);
    lp.store(pa, buf0);
    lq.store(qa, buf0 + LP::LDS_ELEMS);
    __syncthreads();
  }
  for (int kt = 0; kt < nk2; kt += 2) {
    kstep(pa, qa, kbeg + (kt + 2) * BK, pb, qb, buf0, buf1);
    kstep(pb, qb, kbeg + (kt + 3) * BK, pa, qa, buf1, buf0);
  }
  store_acc<C, kDW>(p, t, acc, wp, wq, lane);
}

// Two waves per SIMD in two groups that alternate ("ping-pong"): in each
// half of a slab one group multiplies while the other decodes its half of
// the next slab into LDS and issues the loads of the slab after, so every
// SIMD always has a wave feeding its matrix core.  Waves w and w + NT/128
// share a SIMD (waves are dealt to the four SIMDs round-robin).
template <class C, int PF, int PA, int QF, int QA, bool kDW>
__global__ __launch_bounds__(C::NT) void gemm_pingpong(Params p) {
  constexpr int GT = C::NT / 2;                                 // threads per group
  using LP = Loader<PF, PA, !kDW, C::BP, GT, 2>;
  using LQ = Loader<QF, QA, false, C::BQ, GT, 2>;
  using M = Mma<C, kDW, LP::PITCH, LQ::PITCH, LP::LDS_ELEMS>;
  constexpr int STAGE = LP::LDS_ELEMS + LQ::LDS_ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  __shared__ int32_t s_ends[kMaxGroups];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wp = wave / C::NWQ, wq = wave % C::NWQ;
  const int grp = tid / GT;                                     // 0: multiplies first
  const Tile t = select_tile<C, kDW>(p, s_ends);
  if (!t.valid) return;
  const int kend = t.kend, kbeg = t.kbeg;

  LP lp;
  LQ lq;
  lp.init(p.P, 0, t.p0, kDW ? 0 : p.P.rows, tid % GT, grp);
  lq.init(p.Q, kDW ? 0 : t.g, t.q0, 0, tid % GT, grp);

  f32x16 acc[C::FP][C::FQ];
#pragma unroll
  for (int i = 0; i < C::FP; ++i)
#pragma unroll
    for (int j = 0; j < C::FQ; ++j) acc[i][j] = f32x16{};

  auto multiply = [&](const uint16_t* cur) {
    M fa, fb;
    fa.load(cur, 0, wp, wq, lane);
    fb.load(cur, 16, wp, wq, lane);
    fa.run(acc);
    fa.load(cur, 32, wp, wq, lane);
    fb.run(acc);
    fb.load(cur, 48, wp, wq, lane);
    fa.run(acc);
    fb.run(acc);
  };

  const int nk = (kend - kbeg + BK - 1) / BK;
  typename LP::Stage ps;
  typename LQ::Stage qs;
  // prologue: slab 0 into LDS buffer 0, slab 1 into registers
  if (nk > 0) {
    lp.load(ps, p.P, kbeg, kend);
    lq.load(qs, p.Q, kbeg, kend);
    lp.store(ps, smem);
    lq.store(qs, smem + LP::LDS_ELEMS);
    lp.load(ps, p.P, kbeg + BK, kend);
    lq.load(qs, p.Q, kbeg + BK, kend);
    __syncthreads();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const uint16_t* cur = smem + (kt & 1) * STAGE;
    uint16_t* nxt = smem + ((kt + 1) & 1) * STAGE;
    const int kload = kbeg + (kt + 2) * BK;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half == grp) {
        multiply(cur);
      } else {
        lp.store(ps, nxt);
        lq.store(qs, nxt + LP::LDS_ELEMS);
        lp.load(ps, p.P, kload, kend);
        lq.load(qs, p.Q, kload, kend);
      }
      __syncthreads();
    }
  }
  store_acc<C, kDW>(p, t, acc, wp, wq, lane);
}

// ---------------------------------------------------------------- host side

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

template <class C, int PF, int PA, int QF, int QA, bool kDW>
hipError_t run(const Params& prm, hipStream_t stream) {
  if (prm.ntiles <= 0) return hipSuccess;
  if constexpr (C::PINGPONG)
    gemm_pingpong<C, PF, PA, QF, QA, kDW><<<dim3(prm.ntiles), dim3(C::NT), 0, stream>>>(prm);
  else
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

using Big = Cfg<256, 256, 2, 4, true>;      // 512 threads, two groups of 4 waves, wave tile 128 x 64
using Narrow = Cfg<256, 128, 2, 2, false>;  // 256 threads (one wave per SIMD), wave tile 128 x 64

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
