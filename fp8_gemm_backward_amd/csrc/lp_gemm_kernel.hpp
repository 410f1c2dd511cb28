// Fused dequantize + bf16 MFMA backward contractions (dense and grouped):
// kernel templates, shared by the per-format translation units.
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
// Each workgroup owns one BP x BQ output tile and runs four waves, one per
// SIMD, each owning a (BP/2) x (BQ/2) quarter held in accumulation registers.
// The contraction advances in BK = 64 slabs:
// * the bf16 gradient (P) goes from global memory straight into LDS
//   (buffer_load_dwordx4 ... lds), three LDS buffers deep, issued two slabs
//   ahead;
// * a quantized operand is loaded into registers three slabs ahead (two when
//   no operand is loaded straight into LDS) and decoded into a bf16 LDS tile
//   one slab ahead (two LDS buffers), once for the whole workgroup;
// * the MFMAs of slab k (v_mfma_f32_32x32x16_bf16, four 16-deep substeps)
//   run from register fragments read from LDS one substep ahead.
// Every MFMA is followed by a fixed share of the other work (fragment reads
// of the next substep, load issues, a quarter of a decoded piece), and
// scheduling fences keep that order, so the matrix core is fed while the
// rest proceeds: a wave issues in order, so work bunched behind one MFMA
// leaves the matrix core idle.  One barrier per slab, inside its last
// substep, publishes slab k+1.
//
// LDS layouts.  An operand whose contraction index is contiguous in memory
// (grad in dx, "k-major") is stored [mn][k] and read with ds_read_b128; an
// operand whose contraction runs along its rows (W in dx, grad and X in dw,
// "mn-major") is stored [k][mn] and read with ds_read_b64_tr_b16, which hands
// lane i of each 16-lane group column i of four consecutive rows, i.e. the
// MFMA operand layout.  Bank rules of the gfx950 LDS (measured): a 16-byte
// write serves 8 lanes per cycle, conflict-free when their 16-byte slots
// differ modulo 128 bytes; a 16-byte read serves 16 lanes per cycle (slots
// distinct modulo 256 bytes); the transposing 8-byte read serves 32 lanes,
// i.e. four rows of 64 bytes, which must fall in distinct quarters of 256
// bytes.  Rows are unpadded and 16-byte chunks are XOR-swizzled by row:
// * mn-major: chunk q of row r at q ^ (4 (r & 3) | ((r >> 1) & 3)); eight
//   consecutive lanes decode the same columns of eight consecutive rows;
// * k-major (direct): chunk c of row r at c ^ ((r >> 1) & 7);
// * k-major decoded (MXFP8 grad): 144-byte pitch, no swizzle.
//
// The MFMA is issued as D = Qfrag x Pfrag so that each lane's accumulator
// holds four consecutive output columns, stored as one 8-byte write.
#pragma once

#include <type_traits>
#include <utility>

#include "lp_device.hpp"
#include "lp_internal.hpp"

namespace lp {
namespace gk {

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef short i16x8v __attribute__((ext_vector_type(8)));

constexpr int BK = 64;
constexpr int NT = 256;                 // four waves, one per SIMD
constexpr int kMaxGroups = 1024;
constexpr int kLptGroups = 256;         // grouped dW ranks groups by size up to this many
constexpr int kMaxLds = 160 * 1024;

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N-1>) in order.
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int V>
using IC = std::integral_constant<int, V>;

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
  int32_t nq;            // Q-tiles
  int32_t ntiles;        // grid size (output tiles x splits)
  int32_t gm;            // dense calls: P-tile rows per group of the tile order (1: row-major order)
  // Split contraction (dense calls only): `splits` workgroups share each
  // output tile, split s covering contraction [s * split_len, (s+1) * split_len).
  int32_t splits;        // 1: no split
  int32_t split_len;     // multiple of BK
  float* ws;             // fp32 partial tiles [tile][split][BP * BQ]
  uint32_t* cnt;         // per-tile arrival counters, zero between calls
  // Grouped grad_X split by group size (small groups quantize their weight
  // inside the product, in a launch of their own): fuse_side 1 lists no
  // tiles for groups of at most fuse_rows rows, 2 lists tiles for those
  // only, 0 lists every group.
  int32_t fuse_rows;
  int32_t fuse_side;
  // Grouped grad_X and forward through bf16 tiles, split by dispatch round
  // (tile_split): 1 takes the whole rounds of kCUs 256-wide tiles (all the
  // tiles when there is no split), 2 the last partial round as 256 x 128
  // tiles, in a second launch.  0: no split.
  int32_t tail;
};

// Compute units of the GPU: one 256 x 256 (or 256 x 128) tile workgroup
// each, since its LDS takes a whole CU.
constexpr int kCUs = 256;

template <int kBP, int kBQ>
struct Cfg {
  static constexpr int BP = kBP, BQ = kBQ;
  static constexpr int WP = BP / 2, WQ = BQ / 2;       // 2 x 2 waves
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
// Direct global -> LDS load of kSize bytes per lane (written at M0 = dst,
// lane i at dst + kSize * i; 1- and 2-byte loads write a zero-extended dword
// at dst + 4 i), issued as inline assembly.  The compiler's waitcnt pass
// cannot tell apart the LDS stages that such loads fill across loop
// iterations, and would make every LDS read wait for all of them; the
// kernels that use this wait for their loads themselves (barrier_vm) before
// reading what they wrote.  Default cache policy: the streaming policies
// (sc0 sc1, nt) measured no faster on the MXFP4 forward and the MXFP8 dX in
// steady state (nt slower).
template <int kSize>
__device__ __forceinline__ void dma(Rsrc r, lds_void* dst, int32_t voff, int32_t soff) {
  const uint32_t m0 = (uint32_t)(size_t)dst;
  if constexpr (kSize == 16)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
  else if constexpr (kSize == 4)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
  else if constexpr (kSize == 2)
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ushort %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_ubyte %1, %2, %3 offen lds" ::"s"(m0), "v"(voff), "s"(r), "s"(soff)
                 : "memory", "m0");
}

__device__ __forceinline__ u32x4 bload16(Rsrc r, int32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// 16 bytes per lane from a buffer straight into LDS: lane i writes bytes
// [16i, 16i+16) after `lds` (wave-uniform).
__device__ __forceinline__ void lds_load16(Rsrc r, uint8_t* lds, int32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, off, 0, 0, 0);
}

// 16-byte chunk swizzles (see the header).
__device__ __forceinline__ constexpr int swz_mn(int r) { return ((r & 3) << 2) | ((r >> 1) & 3); }
__device__ __forceinline__ constexpr int swz_k(int r) { return (r >> 1) & 7; }

// Codes per 16-byte chunk.
template <int F>
constexpr int elems_per_chunk() {
  return F == BF16 ? 8 : ((F == MXFP4 || F == NVFP4) ? 32 : 16);
}

// Undecoded contents of one chunk: 16 code bytes and its scale data (one
// E8M0 byte, a pair of E4M3 bytes, one fp32, or 16 E8M0 bytes for MXFP8 with
// scales along the rows).  Scales keep the exact type their load returns: a
// widening at the load would be a separate instruction that the compiler
// may hoist to the loop back edge, where it waits for the load to land.
template <int F, int A>
struct Raw {
  using S = std::conditional_t<
      (F == MXFP8 && A == -2), u32x4,
      std::conditional_t<F == NVFP4, uint16_t, std::conditional_t<F == FP8_B128, uint32_t, uint8_t>>>;
  u32x4 c;
  S s;
};

// Decode quarter Q (two elements, one output dword) of 16-byte piece J
// (eight elements) of a raw chunk to bf16.  The quarters of a piece are
// decoded in order; quarter 0 leaves the piece's scale factor in `sc` for the
// others, so that the work of a piece can be spread over several MFMAs.
// Values equal the standalone dequantization except that NaN payloads are
// left as the hardware makes them.
template <int F, int A, int J, int Q>
__device__ __forceinline__ uint32_t decode_quarter(const Raw<F, A>& r, float ts, float& sc) {
  if constexpr (F == BF16) {
    return r.c[Q];
  } else if constexpr (F == MXFP4) {
    if constexpr (Q == 0) sc = e8m0_to_cvt_scale(r.s);
    return bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.c[J], sc, Q));
  } else if constexpr (F == NVFP4) {
    if constexpr (Q == 0) {
      const f32x2 sv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((uint32_t)r.s, 1.0f, false);
      sc = sv[J / 2] * ts;                                   // scale of elements 16 (J/2) .. +15
    }
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.c[J], 1.0f, Q);
    return pack_bf16x2(v[0] * sc, v[1] * sc);
  } else if constexpr (F == FP8_B128) {
    const float S = __builtin_bit_cast(float, r.s);
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(r.c[2 * J + Q / 2], 1.0f, Q % 2 == 1);
    return pack_bf16x2(v[0] * S, v[1] * S);
  } else if constexpr (F == MXFP8 && A == -1) {
    if constexpr (Q == 0) sc = e8m0_to_cvt_scale(r.s);
    return bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r.c[2 * J + Q / 2], sc, Q % 2 == 1));
  } else {  // MXFP8 along rows: one scale byte per column (elements 2h, 2h+1 of the word)
    constexpr bool hi = Q % 2 == 1;
    const uint32_t w = r.c[2 * J + Q / 2], sw = r.s[2 * J + Q / 2];
    const uint32_t s0 = hi ? (sw >> 16) & 0xFFu : sw & 0xFFu;
    const uint32_t s1 = hi ? sw >> 24 : (sw >> 8) & 0xFFu;
    const uint32_t x = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, e8m0_to_cvt_scale(s0), hi));
    const uint32_t y = bf16x2_bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, e8m0_to_cvt_scale(s1), hi));
    return (x & 0xFFFFu) | (y & 0xFFFF0000u);
  }
}

// Decoding state of the piece in progress.
struct DecState {
  float sc;
  uint32_t o[4];
};

// ---------------------------------------------------------------- operand tiles
// Quantized operand: loaded into registers, decoded into an LDS tile.
// kKMajor: the tile is BMN rows (mn) x BK columns (the contraction runs
// along the tensor's columns); otherwise BK rows x BMN columns.  Per-thread
// chunk positions are fixed for the whole k loop; only the window moves.
// kSwz (k-major only): unpadded rows with the chunk swizzle of direct
// k-major tiles, read like them; otherwise rows padded by 16 bytes.
template <int F, int A, bool kKMajor, int BMN, bool kSwz = false>
struct Decoded {
  static constexpr bool kDirect = false;
  static constexpr int EPC = elems_per_chunk<F>();
  static constexpr int CPR = kKMajor ? BK / EPC : BMN / EPC;        // chunks per tile row
  static constexpr int CHUNKS = kKMajor ? BMN * CPR : BK * CPR;
  static constexpr int PER = CHUNKS / NT;                            // chunks per thread
  static_assert(CHUNKS % NT == 0, "tile not evenly divided among threads");
  static constexpr int PIECES = EPC / 8;                             // 16-byte LDS writes per chunk
  static_assert(!kSwz || kKMajor, "the swizzle is for k-major tiles");
  static constexpr int PITCH = kKMajor ? (kSwz ? BK : BK + 8) : BMN;  // LDS row pitch, bf16 elements
  static constexpr int BUF_BYTES = (kKMajor ? BMN : BK) * PITCH * 2;
  static constexpr int BPE2 = F == BF16 ? 4 : ((F == MXFP4 || F == NVFP4) ? 1 : 2);  // 2 x bytes per element
  static constexpr bool kScale = F != BF16;
  static constexpr int ITEMS = PER;                                  // load items per slab
  static constexpr int VMEM = PER * (kScale ? 2 : 1);                // vector-memory loads per slab
  static constexpr int QUARTERS = F == BF16 ? 1 : 4;                 // decode items per piece
  static constexpr int DECODES = PER * PIECES * QUARTERS;            // decode items per slab
  static_assert(kKMajor ? ((F == MXFP8 && A == -1) || F == NVFP4 || F == FP8_B128) : true,
                "k-major decode needs scales along the contraction");

  using Stage = Raw<F, A>[PER];

  int32_t voff[PER];         // code byte offset of each chunk inside the window
  int32_t row[PER];          // chunk's row in the tile
  int32_t mnc[PER];          // chunk's global mn index (mn-major) / column in the tile (k-major)
  int32_t lds[PER][PIECES];  // byte offset of each 16-byte piece inside an LDS buffer
  const uint8_t* cbase;
  const uint8_t* sbase;
  int64_t crows_bytes;       // k-major: bytes from cbase to the end of the tensor
  float ts;

  struct Win {
    Rsrc cr, sr;
    int k0, kend;
    bool tail;
  };

  __device__ __forceinline__ void init(const Op& op, int g, int mn0, int mnend_rows, int t) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = t + i * NT;
      // k-major: consecutive chunks run along a row.  mn-major: groups of
      // eight consecutive chunks run down eight rows at the same columns.
      const int r = kKMajor ? c / CPR : (c / (8 * CPR)) * 8 + (c & 7);
      const int col = kKMajor ? (c % CPR) * EPC : ((c >> 3) % CPR) * EPC;
      row[i] = r;
#pragma unroll
      for (int j = 0; j < PIECES; ++j) {
        const int q = col / 8 + j;                                   // logical 16-byte chunk
        lds[i][j] = 2 * r * PITCH + 16 * (kKMajor ? (kSwz ? q ^ swz_k(r) : q) : (q ^ swz_mn(r)));
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
      // Rows [mn0, mnend_rows) of group g (FP8 blocks: mn0 % 128 == 0).
      cbase = op.codes + (int64_t)g * op.code_batch + (int64_t)mn0 * op.code_ld;
      sbase = op.scales + (int64_t)g * op.scale_batch + (int64_t)(F == FP8_B128 ? mn0 >> 7 : mn0) * op.scale_ld;
      crows_bytes = (int64_t)(mnend_rows - mn0) * op.code_ld;
    } else {
      cbase = op.codes + (int64_t)g * op.code_batch;
      sbase = op.scales + (int64_t)g * op.scale_batch;
      crows_bytes = 0;
    }
    if constexpr (F == NVFP4) ts = *op.tensor_scale; else ts = 0.0f;
  }

  // Buffer windows of the slab starting at contraction index k0 (reads at or
  // beyond kend come back as zero).
  __device__ __forceinline__ Win window(const Op& op, int k0, int kend) const {
    Win w;
    w.k0 = k0;
    w.kend = kend;
    w.tail = k0 + BK > kend;
    if constexpr (kKMajor) {
      // A slab (BK = 64 columns, k0 % 64 == 0) lies inside one 128-column
      // FP8 block, so one scale column serves it.
      constexpr int KS = F == NVFP4 ? 4 : (F == FP8_B128 ? 7 : 5);    // log2 columns per scale
      const int64_t nrows = crows_bytes / op.code_ld;
      const int64_t srows = F == FP8_B128 ? (nrows + 127) >> 7 : nrows;
      const int soff = F == FP8_B128 ? (k0 >> 7) * 4 : (k0 >> KS);
      w.cr = make_rsrc(cbase + (int64_t)k0 * BPE2 / 2, crows_bytes - (int64_t)k0 * BPE2 / 2);
      w.sr = make_rsrc(sbase + soff, srows * op.scale_ld - soff);
    } else {
      const int64_t nrows = kend - k0;
      w.cr = make_rsrc(cbase + (int64_t)k0 * op.code_ld, nrows * op.code_ld);
      if constexpr (F == MXFP4 || (F == MXFP8 && A == -1) || F == NVFP4)
        w.sr = make_rsrc(sbase + (int64_t)k0 * op.scale_ld, nrows * op.scale_ld);
      else
        w.sr = make_rsrc(sbase, op.scale_bytes);
    }
    return w;
  }

  // Loads of chunk I (codes, then its scale data).
  template <int I>
  __device__ __forceinline__ void load(Stage& st, const Win& w, const Op& op) const {
    if constexpr (kKMajor) {
      const bool out = w.tail && w.k0 + mnc[I] >= w.kend;
      st[I].c = bload16(w.cr, out ? kOOB : voff[I]);
      if constexpr (F == NVFP4)
        st[I].s = __builtin_amdgcn_raw_buffer_load_b16(w.sr, out ? kOOB : row[I] * op.scale_ld + (mnc[I] >> 4), 0, 0);
      else if constexpr (F == FP8_B128)
        st[I].s = __builtin_amdgcn_raw_buffer_load_b32(w.sr, out ? kOOB : (row[I] >> 7) * op.scale_ld, 0, 0);
      else
        st[I].s = __builtin_amdgcn_raw_buffer_load_b8(w.sr, out ? kOOB : row[I] * op.scale_ld + (mnc[I] >> 5), 0, 0);
    } else {
      st[I].c = bload16(w.cr, voff[I]);
      if constexpr (F == MXFP4 || (F == MXFP8 && A == -1)) {
        st[I].s = __builtin_amdgcn_raw_buffer_load_b8(w.sr, row[I] * op.scale_ld + (mnc[I] >> 5), 0, 0);
      } else if constexpr (F == NVFP4) {
        st[I].s = __builtin_amdgcn_raw_buffer_load_b16(w.sr, row[I] * op.scale_ld + (mnc[I] >> 4), 0, 0);
      } else if constexpr (F == FP8_B128) {
        const int gk = w.k0 + row[I];
        const int so = gk < w.kend ? ((gk >> 7) * op.scale_ld + (mnc[I] >> 7) * 4) : kOOB;
        st[I].s = __builtin_amdgcn_raw_buffer_load_b32(w.sr, so, 0, 0);
      } else if constexpr (F == MXFP8) {
        const int gk = w.k0 + row[I];
        st[I].s = bload16(w.sr, gk < w.kend ? ((gk >> 5) * op.scale_ld + mnc[I]) : kOOB);
      }
    }
  }

  // Decode item Q (a quarter, or the whole piece for bf16) of piece J of
  // chunk I; the last one writes the piece to the LDS buffer.
  template <int I, int J, int Q>
  __device__ __forceinline__ void decode(const Stage& st, uint8_t* buf, DecState& d) const {
    if constexpr (F == BF16) {
      *reinterpret_cast<u32x4*>(buf + lds[I][J]) = st[I].c;
    } else {
      d.o[Q] = decode_quarter<F, A, J, Q>(st[I], ts, d.sc);
      if constexpr (Q == 3) *reinterpret_cast<u32x4*>(buf + lds[I][J]) = u32x4{d.o[0], d.o[1], d.o[2], d.o[3]};
    }
  }
};

// bf16 operand: global memory straight into LDS.  One buffer_load_dwordx4
// ... lds moves 1 KiB, lane i filling bytes [16i, 16i+16) of the block, so
// the (swizzled) layout is set by which global chunk each lane fetches.  The
// four waves issue PER blocks each.
template <bool kKMajor, int BMN>
struct Direct {
  static constexpr bool kDirect = true;
  static constexpr int BUF_BYTES = BMN * BK * 2;
  static constexpr int BLOCKS = BUF_BYTES / 1024;
  static constexpr int PER = BLOCKS / 4;                             // blocks per wave
  static constexpr int RPB = kKMajor ? 8 : 1024 / (2 * BMN);         // tile rows per block
  static constexpr int LPR = 64 / RPB;                               // lanes per tile row
  static constexpr int ITEMS = PER;
  static constexpr int VMEM = PER;
  static constexpr int DECODES = 0;
  static constexpr int PIECES = 1;
  struct Stage {};
  struct Win {
    Rsrc r;
    int k0, kend;
    bool tail;
  };

  int32_t voff[PER];   // lane's byte offset inside the window
  int32_t colk[PER];   // k-major: lane's first column inside the slab (tail mask)
  int32_t lds0;        // byte offset of the wave's first block inside a buffer
  const uint8_t* base;
  int64_t rows_bytes;  // k-major: bytes from base to the end of the tensor
  int32_t ld;

  __device__ __forceinline__ void init(const Op& op, int g, int mn0, int mnend_rows, int wave, int lane) {
    ld = op.code_ld;
    lds0 = wave * PER * 1024;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int row = RPB * (wave * PER + i) + lane / LPR;
      const int pc = lane % LPR;                                     // physical chunk in the row
      if constexpr (kKMajor) {
        const int q = pc ^ swz_k(row);
        voff[i] = row * ld + 16 * q;
        colk[i] = 8 * q;
      } else {
        const int q = pc ^ swz_mn(row);
        voff[i] = row * ld + 2 * mn0 + 16 * q;
        colk[i] = 0;
      }
    }
    if constexpr (kKMajor) {
      base = op.codes + (int64_t)g * op.code_batch + (int64_t)mn0 * ld;
      rows_bytes = (int64_t)(mnend_rows - mn0) * ld;
    } else {
      base = op.codes + (int64_t)g * op.code_batch;
      rows_bytes = 0;
    }
  }

  __device__ __forceinline__ Win window(const Op&, int k0, int kend) const {
    Win w;
    w.k0 = k0;
    w.kend = kend;
    w.tail = k0 + BK > kend;
    if constexpr (kKMajor)
      w.r = make_rsrc(base + 2 * (int64_t)k0, rows_bytes - 2 * (int64_t)k0);
    else
      w.r = make_rsrc(base + (int64_t)k0 * ld, (int64_t)(kend - k0) * ld);
    return w;
  }

  template <int I>
  __device__ __forceinline__ void load(uint8_t* buf, const Win& w) const {
    int32_t off = voff[I];
    if constexpr (kKMajor) off = (w.tail && w.k0 + colk[I] >= w.kend) ? kOOB : off;
    lds_load16(w.r, buf + lds0 + 1024 * I, off);
  }
};

// ---------------------------------------------------------------- fragments
// Per-lane LDS byte addresses of one wave's MFMA fragments; substep s adds a
// constant (or, for direct k-major tiles, has its own address).
//
// k-major tile: lane holds row (mn) `base + lane%32`, k = 16 s + (lane/32)*8 .. +7.
// mn-major tile: lane holds column `base + lane%32` at the same k's, from two
// transposing reads (rows r and r + 4 of each 8-row half).
template <bool kKMajor, bool kDirect, int BMN, int NF>
struct FragAddr {
  static constexpr int PITCH = kKMajor ? (kDirect ? BK : BK + 8) : BMN;   // bf16 elements
  static constexpr int NREAD = kKMajor ? 1 : 2;                           // reads per fragment
  static constexpr int SUB = kKMajor ? 32 : 16 * 2 * BMN;                 // bytes between substeps
  static constexpr int NA = kKMajor ? (kDirect ? 4 : 1) : NF;
  static constexpr int NB = kKMajor ? 1 : NF;
  int32_t a[NA];
  int32_t b[NB];

  __device__ __forceinline__ void init(int mn_base, int lane) {
    if constexpr (kKMajor) {
      const int r = lane & 31;                                        // (mn_base is a multiple of 32)
      if constexpr (kDirect) {
#pragma unroll
        for (int s = 0; s < 4; ++s) a[s] = 2 * (mn_base + r) * PITCH + 16 * ((2 * s + (lane >> 5)) ^ swz_k(r));
      } else {
        a[0] = 2 * (mn_base + r) * PITCH + 16 * (lane >> 5);
      }
      b[0] = 0;
    } else {
      const int i16 = lane & 15, grp = lane >> 4;
      const int row = (grp >> 1) * 8 + (i16 >> 2);                   // plus 16 s; row % 8 == i16 / 4
      const int lc = (grp & 1) * 2 + ((i16 & 3) >> 1);               // logical chunk in the 4-chunk group
      const int half = (i16 & 1) * 8;                                 // bytes
      const int s4 = row & 3, ha = (row >> 1) & 3, hb = ((row + 4) >> 1) & 3;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int m = mn_base / 32 + f;                                // 4-chunk group of the fragment
        a[f] = 2 * row * PITCH + 16 * (4 * (m ^ s4) + (lc ^ ha)) + half;
        b[f] = 2 * (row + 4) * PITCH + 16 * (4 * (m ^ s4) + (lc ^ hb)) + half;
      }
    }
  }

  // Read R (0 .. NREAD-1) of fragment f at substep S into dst.
  template <int S, int R, int f>
  __device__ __forceinline__ void read(const uint8_t* buf, i16x8v& dst) const {
    if constexpr (kKMajor) {
      const int off = (kDirect ? a[S] : a[0] + S * SUB) + f * 32 * 2 * PITCH;
      dst = __builtin_bit_cast(i16x8v, *reinterpret_cast<const u32x4*>(buf + off));
    } else {
      const uint8_t* p = buf + (R == 0 ? a[f] : b[f]) + S * SUB;
      const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
      typedef short i16x4v __attribute__((ext_vector_type(4)));
      if constexpr (R == 0)
        dst.lo = __builtin_bit_cast(i16x4v, v);
      else
        dst.hi = __builtin_bit_cast(i16x4v, v);
    }
  }
};

// Map the hardware workgroup id so that each XCD (workgroups are dealt to
// the 8 XCDs round-robin) receives a contiguous range of logical tiles.
__device__ __forceinline__ int xcd_remap(int hw, int n) {
  constexpr int X = 8;
  int per = n / X, rem = n % X;
  int x = hw % X, j = hw / X;
  return x < rem ? x * (per + 1) + j : rem * (per + 1) + (x - rem) * per + j;
}

// Tile order of a dense contraction: groups of gm P-tile rows, each group's
// tiles column by column, so that the tiles one XCD runs at a time (a
// contiguous range of tile indices) form a gm x (32 / gm) block that shares
// operand rows and columns in that XCD's L2.  Returns (P-tile, Q-tile);
// a bijection of [0, np * nq).
__device__ __forceinline__ int2 grouped_order(int tile, int np, int nq, int gm) {
  const int per = gm * nq;
  const int gid = tile / per, first = gid * gm;
  const int gsz = np - first < gm ? np - first : gm;
  const int r = tile - gid * per;
  return make_int2(first + r % gsz, r / gsz);
}

// The output tile, group and contraction range of one workgroup.
struct Tile {
  int g, p0, pend, q0, kbeg, kend;
  int tile, split;       // output tile and contraction split (split calls)
  bool valid;
};

// The group holding listed row tile pidx (row tiles of BP rows, groups in
// order, a group listed or not by its row count), with the clamped group
// ends end_g = clamp(o_g, end_{g-1}, M); pidx past every listed tile:
// found = false and seen = the listed row tiles in all.  Each wave reads 64
// group ends with one LDS read and walks them from registers (readlane), so
// that no LDS round trip sits in the per-group chain: walking one group per
// LDS read cost up to 20k cycles per tile with 64 groups.
// A walk may resume from an earlier hit (hint) whose first row tile is at
// or before pidx: a persistent workgroup's tiles come in increasing order,
// and restarting from group 0 for each cost it more as its tiles moved to
// later groups.
struct GroupHit {
  int g, start, end, seen;
  bool found;
};
template <int BP, class Listed>
__device__ __forceinline__ GroupHit find_row_tile(const int32_t* s_ends, int groups, int M, int pidx, Listed listed,
                                                  const GroupHit* hint = nullptr) {
  const int lane = threadIdx.x & 63;
  int g0 = 0, start = 0, seen = 0;
  if (hint != nullptr && hint->found && hint->seen <= pidx) {
    g0 = hint->g;
    start = hint->start;
    seen = hint->seen;
  }
  for (int base = g0; base < groups; base += 64) {
    const int v = base + lane < groups ? s_ends[base + lane] : 0;
    const int cnt = groups - base < 64 ? groups - base : 64;
    for (int j = 0; j < cnt; ++j) {
      int e = __builtin_amdgcn_readlane(v, j);
      e = e < start ? start : (e > M ? M : e);
      const int n = listed(e - start) ? (e - start + BP - 1) / BP : 0;
      if (pidx < seen + n) return GroupHit{base + j, start, e, seen, true};
      seen += n;
      start = e;
    }
  }
  return GroupHit{0, 0, 0, seen, false};
}

// Map the workgroup to its tile.  s_ends: LDS for the group offsets.  hw:
// the workgroup's index among the p.ntiles of this contraction, in dispatch
// order (blockIdx.x unless several contractions share a launch).
// persistent = true: hw is already the logical tile index (a persistent
// workgroup's own tile order), and s_ends already holds the group ends.
template <class C, bool kDW>
__device__ __forceinline__ Tile select_tile(const Params& p, int32_t* s_ends, int hw = blockIdx.x,
                                            bool persistent = false, GroupHit* hint = nullptr) {
  const int tid = threadIdx.x;
  int tile = persistent ? hw : xcd_remap(hw, p.ntiles);
  int split = 0;
  if (p.splits > 1) {                                          // the splits of a tile are neighbours
    split = tile % p.splits;
    tile /= p.splits;
  }
  Tile t{0, 0, 0, 0, 0, p.Ktot, tile, split, true};
  if (p.offsets != nullptr && !persistent) {
    for (int i = tid; i < p.groups; i += NT) s_ends[i] = p.offsets[i];
    __syncthreads();
  }
  if (!kDW) {
    // Groups partition the output rows; tiles never straddle a group.
    int pidx = tile / p.nq;
    t.q0 = (tile % p.nq) * C::BQ;
    if (p.offsets == nullptr) {
      if (p.gm > 1) {
        const int2 pq = grouped_order(tile, (p.Ptot + C::BP - 1) / C::BP, p.nq, p.gm);
        pidx = pq.x;
        t.q0 = pq.y * C::BQ;
      }
      t.p0 = pidx * C::BP;
      t.pend = p.Ptot;
    } else {
      t.p0 = -1;
      // fuse_side 0 lists every group; 1 the groups of more than fuse_rows
      // rows; 2 those of at most fuse_rows.
      auto listed = [&](int n) { return p.fuse_side == 0 || ((n <= p.fuse_rows) == (p.fuse_side == 2)); };
      if (p.fuse_side != 0 && !persistent && p.splits == 1) {
        // A filtered listing, whose tile count the host only bounds: deal
        // the listed tiles themselves over the XCDs, or the bound's empty
        // tail would leave whole XCDs idle.
        const int nt = find_row_tile<C::BP>(s_ends, p.groups, p.Ptot, INT32_MAX, listed).seen * p.nq;
        tile = hw < nt ? xcd_remap(hw, nt) : nt;                 // nt: past every listed tile
        pidx = tile / p.nq;
        t.q0 = (tile % p.nq) * C::BQ;
        t.tile = tile;
      } else if (p.tail != 0) {
        // Split by dispatch round.  The ntb 256 x 256 tiles, one per CU at
        // a time, run in rounds of kCUs; a last round of r <= kCUs / 2
        // tiles would leave most CUs idle for a whole tile's time, so those
        // tiles go to a second launch as 2r (at most) 256 x 128 tiles, each
        // about half as long.  The row tiles (BP = 256) are the same in both
        // launches and every tile sums its products in the same order, so
        // the split changes no result bit.
        const int nqb = (p.Qtot + 255) / 256;
        const int rows = find_row_tile<C::BP>(s_ends, p.groups, p.Ptot, INT32_MAX, listed).seen;
        const int ntb = rows * nqb, full = ntb / kCUs * kCUs, rest = ntb - full;
        const bool split = full > 0 && rest > 0 && 2 * rest <= kCUs;
        int nt = split ? full : ntb, base = 0;
        if (p.tail == 2) {
          // big tile `full` is row tile full / nqb, 256-column tile full % nqb
          base = (full / nqb) * p.nq + 2 * (full % nqb);
          nt = split ? rows * p.nq - base : 0;
        }
        tile = hw < nt ? base + xcd_remap(hw, nt) : rows * p.nq; // rows nq: past every tile
        pidx = tile / p.nq;
        t.q0 = (tile % p.nq) * C::BQ;
        t.tile = tile;
      }
      const GroupHit h = find_row_tile<C::BP>(s_ends, p.groups, p.Ptot, pidx, listed, hint);
      if (hint != nullptr && h.found) *hint = h;
      if (h.found) {
        t.g = h.g;
        t.p0 = h.start + (pidx - h.seen) * C::BP;
        t.pend = h.end;
        if (p.gm > 1) {
          // Inside the group, the dense order in blocks of gm row tiles
          // (grouped_order): the tiles an XCD runs together share both
          // gradient rows and weight columns in its L2.
          const int n = (h.end - h.start + C::BP - 1) / C::BP;
          const int2 pq = grouped_order(tile - h.seen * p.nq, n, p.nq, p.gm);
          t.p0 = h.start + pq.x * C::BP;
          t.q0 = pq.y * C::BQ;
        }
      }
    }
    t.valid = t.p0 >= 0 && t.p0 < t.pend;
  } else if (p.offsets != nullptr && p.groups <= kLptGroups) {
    // Groups partition the contraction; every group has np x nq tiles, whose
    // cost grows with the group's size.  Longest first: the tiles are listed
    // by group in decreasing size (ties by group index) and taken in
    // hardware dispatch order, which deals consecutive tiles to the XCDs in
    // turn, so every XCD starts on its share of the largest group and the
    // short tiles fill in behind (longest-processing-time-first list
    // scheduling).
    int32_t* ends = s_ends + kMaxGroups / 2;                   // clamped ends (groups <= kLptGroups)
    int32_t* pick = s_ends + kMaxGroups - 1;
    for (int i = tid; i < p.groups; i += NT) {
      int e = 0;                                               // end_i = min(max(0, o_0..o_i), M)
      for (int j = 0; j <= i; ++j) e = s_ends[j] > e ? s_ends[j] : e;
      ends[i] = e < p.Ktot ? e : p.Ktot;
    }
    __syncthreads();
    const int per = p.ntiles / p.groups;                       // tiles per group
    const int pos = hw;
    const int rank = pos / per;
    for (int i = tid; i < p.groups; i += NT) {
      const int si = ends[i] - (i ? ends[i - 1] : 0);
      int r = 0;
      for (int j = 0; j < p.groups; ++j) {
        const int sj = ends[j] - (j ? ends[j - 1] : 0);
        r += (sj > si || (sj == si && j < i)) ? 1 : 0;
      }
      if (r == rank) *pick = i;
    }
    __syncthreads();
    t.g = *pick;
    // Inside a group the P-tile index runs fastest, so that the tiles one
    // XCD receives (every eighth) share their gradient columns (P tiles
    // p, p + 8, ...) rather than each XCD reading every gradient block of
    // the group; per is np nq.
    const int r = pos - rank * per;
    const int np = per / p.nq;
    t.p0 = (r % np) * C::BP;
    t.q0 = (r / np) * C::BQ;
    t.pend = p.Ptot;
    t.kbeg = t.g ? ends[t.g - 1] : 0;
    t.kend = ends[t.g];
  } else {
    // Dense dW, or too many groups to rank per workgroup: tiles are dealt
    // round-robin over the groups so that each XCD's contiguous range holds
    // an equal share of every group.
    t.g = tile % p.groups;
    const int r = tile / p.groups;
    t.p0 = (r / p.nq) * C::BP;
    t.q0 = (r % p.nq) * C::BQ;
    if (p.offsets == nullptr && p.gm > 1) {
      const int2 pq = grouped_order(r, (p.Ptot + C::BP - 1) / C::BP, p.nq, p.gm);
      t.p0 = pq.x * C::BP;
      t.q0 = pq.y * C::BQ;
    }
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
  if (p.splits > 1) {
    t.kbeg = split * p.split_len;
    t.kend = t.kbeg + p.split_len < p.Ktot ? t.kbeg + p.split_len : p.Ktot;
  }
  return t;
}

// Epilogue: fp32 -> bf16 (nearest even) through an LDS staging area of the
// wave's own (`stage`, 128 x WQ bf16), so that the global stores are 16
// bytes per lane and whole 256-byte row segments per 16 lanes.  A lane's
// accumulator holds four consecutive columns of one row (8-byte pieces);
// 8-byte slot s of row r is staged at s ^ (r & 15), which keeps both the
// staging writes (rows 0..15 of one column) and the row-wise reads free of
// bank conflicts.
// alpha multiplies every result before rounding when kAlpha is set.
template <class C, bool kDW, bool kAlpha = false>
__device__ __forceinline__ void store_acc(const Params& p, const Tile& t, f32x16 (&acc)[C::FP][C::FQ], int wp,
                                          int wq, int lane, uint8_t* stage, float alpha = 1.0f) {
  constexpr int ROWB = C::WQ * 2;                                  // staged row bytes
  constexpr int SLOTS = ROWB / 8;                                  // 8-byte slots per row
  static_assert(SLOTS >= 16, "swizzle needs 16 slots per row");
#pragma unroll
  for (int i = 0; i < C::FP; ++i) {
    const int r = i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < C::FQ; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int slot = (j * 32 + 8 * r4 + 4 * (lane >> 5)) / 4;
        float e[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) e[d] = kAlpha ? acc[i][j][4 * r4 + d] * alpha : acc[i][j][4 * r4 + d];
        const u32x2 v = {pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3])};
        *reinterpret_cast<u32x2*>(stage + r * ROWB + 8 * (slot ^ (r & 15))) = v;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);                              // lgkmcnt(0): own staging writes done
  uint16_t* out = p.C + (kDW ? (int64_t)t.g * p.c_batch : 0);
  constexpr int LPR = ROWB / 16;                                   // lanes per staged row
  constexpr int RPI = 64 / LPR;                                    // rows per instruction
  const int c16 = lane % LPR;
  const int col = t.q0 + wq * C::WQ + 8 * c16;
#pragma unroll 4
  for (int it = 0; it < C::WP / RPI; ++it) {
    const int r = it * RPI + lane / LPR;
    const uint8_t* src = stage + r * ROWB;
    const u32x2 lo = *reinterpret_cast<const u32x2*>(src + 8 * ((2 * c16) ^ (r & 15)));
    const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 8 * ((2 * c16 + 1) ^ (r & 15)));
    const int row = t.p0 + wp * C::WP + r;
    if (row < t.pend && col < p.Qtot)
      *reinterpret_cast<u32x4*>(out + (int64_t)row * p.ldc + col) = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
}

// Split contraction: every split writes its fp32 partial tile to the
// workspace, then counts itself in at the tile's counter; the workgroup that
// arrives last adds the partials of all splits in split order (its own from
// registers) and goes on to the bf16 epilogue, the others end.  Nothing
// waits on another workgroup.  The sum is the same whichever split arrives
// last.  The last one clears the counter for the next call.  Partials are
// laid out [wave][16-byte piece][lane] so that every access of a wave is one
// contiguous KiB.  `flag` is LDS for broadcasting the arrival count.
// Ordering: each wave waits for its own partial stores, the workgroup
// barrier orders them before thread 0's device-scope acquire-release
// increment (whose release writes the L2 back, whose acquire invalidates the
// L2 and this CU's L1), and a second barrier orders that increment before
// any wave of the last arriver reads the other partials.  One release and
// one acquire per workgroup: issuing them from every wave costs a whole-L2
// write-back each.
template <class C>
__device__ __forceinline__ bool reduce_split(const Params& p, const Tile& t, f32x16 (&acc)[C::FP][C::FQ], int wave,
                                             int lane, uint32_t* flag) {
  constexpr int NV = C::FP * C::FQ * 4;                          // 16-byte pieces per lane
  constexpr size_t kTileFloats = (size_t)C::BP * C::BQ;
  f32x4* const base = reinterpret_cast<f32x4*>(p.ws + (size_t)t.tile * p.splits * kTileFloats) +
                      (size_t)wave * NV * 64 + lane;
  constexpr size_t kSplitStride = kTileFloats / 4;               // f32x4 pieces per split
  f32x4* const mine = base + (size_t)t.split * kSplitStride;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const f32x16& a = acc[v / (4 * C::FQ)][(v / 4) % C::FQ];
    const int r = v % 4;
    __builtin_nontemporal_store(f32x4{a[4 * r], a[4 * r + 1], a[4 * r + 2], a[4 * r + 3]}, mine + v * 64);
  }
  __builtin_amdgcn_s_waitcnt(0);                                 // this wave's partial stores done
  __syncthreads();
  if (threadIdx.x == 0) *flag = __hip_atomic_fetch_add(p.cnt + t.tile, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const bool last = *flag == (uint32_t)(p.splits - 1);
  __syncthreads();                                               // flag read before LDS is reused
  if (!last) return false;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    f32x16& a = acc[v / (4 * C::FQ)][(v / 4) % C::FQ];
    const int r = v % 4;
    const f32x4 own = {a[4 * r], a[4 * r + 1], a[4 * r + 2], a[4 * r + 3]};
    f32x4 sum = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < p.splits; ++s) {
      const f32x4 x = s == t.split ? own : __builtin_nontemporal_load(base + (size_t)s * kSplitStride + v * 64);
      sum[0] += x[0];
      sum[1] += x[1];
      sum[2] += x[2];
      sum[3] += x[3];
    }
    a[4 * r] = sum[0];
    a[4 * r + 1] = sum[1];
    a[4 * r + 2] = sum[2];
    a[4 * r + 3] = sum[3];
  }
  if (threadIdx.x == 0) __hip_atomic_store(p.cnt + t.tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// s_waitcnt vmcnt(N) lgkmcnt(0), then s_barrier.  Written out because the
// compiler's workgroup barrier waits for every outstanding load (direct LDS
// loads count as LDS writes), which would drain the prefetch each slab.
template <int N>
__device__ __forceinline__ void barrier_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt out of range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The bf16 P operand lands in three LDS buffers that are separate variables,
// so that the compiler can tell the buffer being read from the two being
// filled by direct loads and waits only for the load that filled it.  This
// needs the buffer of each slab fixed at compile time: the main loop covers
// three slabs, and decoded operands use three register stages to match.
//
// kFwd: the forward y = x @ W^T (P = x rows, Q = W[g] rows, both k-major,
// the contraction running along K, the columns of both).
// Operand paths and LDS buffers of one instantiation.
template <class C, int PF, int PA, int QF, int QA, bool kDW, bool kFwd>
struct GemmShape {
  static_assert(!(kFwd && kDW), "the forward lists its tiles as grad_X does");
  static constexpr bool PK = !kDW;                               // P k-major in dx and the forward, mn-major in dw
  static constexpr bool QK = kFwd;                               // Q k-major in the forward only
  static constexpr bool PD = PF == BF16;                         // P loaded straight into LDS
  // Q straight into LDS too when both operands are bf16 and three Q stages fit.
  static constexpr bool QD =
      PD && QF == BF16 && 3 * Direct<PK, C::BP>::BUF_BYTES + 3 * Direct<QK, C::BQ>::BUF_BYTES <= kMaxLds;
  using LP = std::conditional_t<PD, Direct<PK, C::BP>, Decoded<PF, PA, PK, C::BP>>;
  // A decoded k-major Q tile drops its row padding when two padded buffers
  // would not fit beside P's.
  static constexpr bool QSWZ = QK && !QD && (PD ? 3 : 2) * LP::BUF_BYTES + 2 * C::BQ * (BK + 8) * 2 > kMaxLds;
  using LQ = std::conditional_t<QD, Direct<QK, C::BQ>, Decoded<QF, QA, QK, C::BQ, QSWZ>>;
  static constexpr int PBUF = LP::BUF_BYTES, QBUF = LQ::BUF_BYTES;
  static constexpr int SB = C::WP * C::WQ * 2;                   // epilogue staging bytes per wave
  static constexpr int QBUF0 = QD ? (QBUF > SB ? QBUF : SB) : 2 * QBUF;   // Q buffer 0 (also wave 3's staging)
  // Bytes of the six LDS buffers sp0, sp1, sp2, sq0, sq1, sq2.
  static constexpr int SP0 = PD ? PBUF : 2 * PBUF, SP1 = PD ? PBUF : 16, SP2 = PD ? PBUF : 16;
  static constexpr int SQ0 = QBUF0, SQ1 = QD ? QBUF : 16, SQ2 = QD ? QBUF : 16;
  static_assert((PD ? 3 * PBUF : 2 * PBUF) + QBUF0 + (QD ? 2 * QBUF : 0) <= kMaxLds, "LDS budget");
  static_assert(kMaxGroups * 4 <= PBUF, "group ends alias P buffer 0");
};

// One output tile: hw is the workgroup's index among p.ntiles (see
// select_tile); sp0 .. sq2 are the six LDS buffers of GemmShape, separate
// variables of the calling kernel.
template <class C, int PF, int PA, int QF, int QA, bool kDW, bool kFwd = false>
__device__ __forceinline__ void gemm_tile(const Params& p, int hw, uint8_t* sp0, uint8_t* sp1, uint8_t* sp2,
                                          uint8_t* sq0, uint8_t* sq1, uint8_t* sq2) {
  using G = GemmShape<C, PF, PA, QF, QA, kDW, kFwd>;
#include "lp_gemm_tile_body.inc"
}

template <class C, int PF, int PA, int QF, int QA, bool kDW, bool kFwd = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(Params p) {
  using G = GemmShape<C, PF, PA, QF, QA, kDW, kFwd>;
  __shared__ __attribute__((aligned(1024))) uint8_t sp0[G::SP0];
  __shared__ __attribute__((aligned(1024))) uint8_t sp1[G::SP1];
  __shared__ __attribute__((aligned(1024))) uint8_t sp2[G::SP2];
  __shared__ __attribute__((aligned(1024))) uint8_t sq0[G::SQ0];
  __shared__ __attribute__((aligned(1024))) uint8_t sq1[G::SQ1];
  __shared__ __attribute__((aligned(1024))) uint8_t sq2[G::SQ2];
  const int hw = blockIdx.x;
#include "lp_gemm_tile_body.inc"
}

template <class C, int PF, int PA, int QF, int QA, bool kDW, bool kFwd = false>
inline hipError_t run(const Params& prm, hipStream_t stream) {
  if (prm.ntiles <= 0) return hipSuccess;
  gemm_kernel<C, PF, PA, QF, QA, kDW, kFwd><<<dim3(prm.ntiles), dim3(NT), 0, stream>>>(prm);
  return hipGetLastError();
}

// Q-operand format dispatch.
template <class C, int PF, int PA, bool kDW>
inline hipError_t dispatch_q(const lp_qtensor& q, const Params& prm, hipStream_t s) {
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

// Launch of one operand-format combination; each is instantiated in its own
// translation unit (lp_gemm_<dx|dw>_<tile>[_<grad format>].hip).
using Big = Cfg<256, 256>;      // wave tile 128 x 128
using Narrow = Cfg<256, 128>;   // wave tile 128 x 64
hipError_t dx_big_bf16(const lp_qtensor& q, const Params& prm, hipStream_t s);
hipError_t dx_big_mxfp8(const lp_qtensor& q, const Params& prm, hipStream_t s);
hipError_t dx_narrow_bf16(const lp_qtensor& q, const Params& prm, hipStream_t s);
hipError_t dx_narrow_mxfp8(const lp_qtensor& q, const Params& prm, hipStream_t s);
hipError_t dw_big(const lp_qtensor& q, const Params& prm, hipStream_t s);
hipError_t dw_narrow(const lp_qtensor& q, const Params& prm, hipStream_t s);
// MXFP8 gradient x MXFP8 weight scaled along its rows, on the block-scaled MFMA
// (256 x 256 tiles, no split).
hipError_t dx_mx(const Params& prm, hipStream_t s);
// Dense grad_W of an MXFP8 gradient and an MXFP8 input, both scaled along
// their rows (the contraction), on the block-scaled MFMA.
hipError_t dw_mx(const Params& prm, hipStream_t s);
// Grouped grad_X of an MXFP8 gradient and a bf16 weight that the kernel
// quantizes to MXFP8 along its rows (256 x 128 tiles; the groups that
// prm.fuse_side / fuse_rows list).
hipError_t dx_wquant(const Params& prm, hipStream_t s);
// Compute units of the current device, looked up once per device.
int compute_units();
// grad_X / grad_W of a per-tensor scaled FP8 gradient and a per-tensor
// scaled FP8 operand (formats LP_FP8T_*), on the same MFMA with unit block
// scales; grouped calls included.
hipError_t dx_pt(const Params& prm, int fmt_p, int fmt_q, hipStream_t s);
hipError_t dw_pt(const Params& prm, int fmt_p, int fmt_q, hipStream_t s);
// Forward y = x @ w^T of MX operands scaled along k, both MXFP4 (fp4) or
// both MXFP8.
hipError_t fwd_mx(const Params& prm, bool fp4, hipStream_t s);
// Forward y = x @ w^T through bf16 tiles (fused decode): bf16 x with a bf16
// weight (256 x 128 tiles) or a block-FP8 or NVFP4 weight, NVFP4 x with an
// NVFP4 weight (256 x 256 tiles; 256 x 128 when narrow, the last round of a
// split grouped call).
hipError_t fwd_dec(const Params& prm, int fmt_x, int fmt_w, bool narrow, hipStream_t s);
// Both of them in one launch (X and W in the same format fmt_q).
hipError_t pt_pair(const Params& dx, const Params& dw, int fmt_p, int fmt_q, hipStream_t s);
// Grouped grad_X and grad_W of a bf16 gradient through 256 x 256 bf16 tiles
// in one launch, grad_X's tiles first; W and X both LP_MXFP4 or both
// LP_NVFP4 (fmt_q), scaled along their last axis.
hipError_t dec_pair(const Params& dx, const Params& dw, int fmt_q, hipStream_t s);

}  // namespace gk
}  // namespace lp
