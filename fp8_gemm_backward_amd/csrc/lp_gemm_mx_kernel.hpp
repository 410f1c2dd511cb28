// Backward contractions on gfx950's block-scaled FP8 MFMA: an MXFP8 gradient
// times an MXFP8 operand whose E8M0 scales both run along the contraction,
// or a per-tensor scaled FP8 gradient times a per-tensor scaled FP8 operand.
//
// "perf: defer mxfp8 backward quantization", MXFP8GMMFunction.op_dx: the
// backward re-quantizes the gradient along its last axis and the weight along
// its reduction axis (one E8M0 scale per 32) and contracts the two quantized
// operands with their per-32 scales (group sizes [1, 1, 32]).  Both scales
// therefore run along the contraction, which is exactly what
// v_mfma_scale_f32_32x32x64_f8f6f4 applies: each lane brings 32 E4M3 codes and
// the E8M0 scale of their block, and the products code_a * code_b *
// 2^(sa + sb) are accumulated in fp32.  Every product is exact, so the result
// is the contraction of the decoded operands up to fp32 summation order, as
// in the decode-to-bf16 path, with no decode work and at the FP8 MFMA rate.
//
//   dX: out[m][q] = sum_n grad[m][n] * W[g][n][q]    (rows m of group g)
//   dW: out[n][q] = sum_m grad[m][n] * X[m][q]       (dense; grad and X both
//       MX-quantized along their rows, the Deferred-MXFP8 page's
//       MXFP8MatMul.backward with dual-axis gradient quantization)
//
// Layout facts of the two gfx950 instructions used (checked on the hardware
// with in-bounds probes):
// * v_mfma_scale_f32_32x32x64_f8f6f4: lane l feeds row (A) or column (B)
//   l % 32; with h = l / 32 its bytes 0..15 hold k = 16 h + 0..15 and bytes
//   16..31 hold k = 32 + 16 h + 0..15; the scale byte (selected by opsel) of
//   lane r covers k 0..31 of row r, that of lane r + 32 covers k 32..63.  The
//   result layout is that of the bf16 32x32 MFMA.
// * ds_read_b64_tr_b8: in each 16-lane group, lane i receives byte i % 8 of
//   the eight 8-byte rows addressed by lanes 2 s + i / 8 (s = 0..7).  With
//   lane q addressing row n0 + q / 2 at byte 8 (q & 1) of a 16-column chunk,
//   lane i receives column i of rows n0 .. n0 + 7: the weight's transpose.
//
// Tiles: 256 (output rows) x 256 (output columns) per workgroup, four waves of
// 128 x 128, 64-deep slabs.  Everything a slab needs - 16 KiB of gradient
// codes, 16 KiB of weight codes and the scale bytes gathered into the
// order the lanes read them - goes from global memory straight into LDS
// (buffer_load ... lds), four stages deep in separate LDS variables, issued
// three slabs ahead.  A slab's fragments are read during the previous slab's
// MFMAs.  One barrier per slab.  In dX the gradient tile is [m][64 B] (its
// contraction contiguous, read with ds_read_b128); in dW both tiles are
// [contraction][256 B] and both are read through the transposing read.
#pragma once

#include "lp_gemm_kernel.hpp"

namespace lp {
namespace gk {

constexpr int XBP = 256, XBQ = 256;             // output tile
constexpr int XWP = 128, XWQ = 128;             // wave tile
constexpr int XFP = 4, XFQ = 4;                 // 32 x 32 blocks per wave
constexpr int XBK = 64;                         // contraction per slab
constexpr int kPBytes = XBP * XBK;              // gradient codes per slab
constexpr int kQBytes = XBK * XBQ;              // weight codes per slab
constexpr int kTileBytes = kPBytes + kQBytes;
constexpr int kGatherBytes = 4096;              // gathered scales of one slab (byte-gather mode)
constexpr int kChunkSlabs = 8;                  // slabs per scale chunk (chunk mode)
constexpr int kChunkBytes = XBP * 16 + 16 * XBQ;  // grad [256 rows][16 blocks] + weight [16 blocks][256 cols]
using XCfg = Cfg<XBP, XBQ>;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// Gradient tile [m][64 B], 16-byte chunk c of row m at c ^ ((m >> 2) & 3):
// the fragment reads (16 consecutive rows, one chunk) hit 16 distinct slots.
__device__ __forceinline__ int p_swz(int m) { return (m >> 2) & 3; }
// Weight tile [n][256 B], chunk c of row n at c ^ (2 (n & 7)): a transposing
// read of 32 lanes (rows n0..n0+7, chunks c and c+1, c even) hits 16
// distinct slots.
__device__ __forceinline__ int q_swz(int n) { return 2 * (n & 7); }

// How the E8M0 scale operands of the MFMA are fed (kMode):
// * kTensorMode: per-tensor scaled codes.  Every scale operand is 127 (2^0),
//   no scale is loaded, and the fp32 results are multiplied by the product
//   of the two tensor scales before rounding to bf16.
// Otherwise the MX scale bytes reach LDS in one of two ways.
// * Chunk mode (the gradient's scale rows are 16-byte aligned: N % 512 ==
//   0): every eight slabs, one 16-byte load per gradient row (its next 16
//   scale blocks) and 16 weight scale rows of 256 bytes, double-buffered;
//   each slab a lane reads its eight scale bytes (four fragments of each
//   operand) with byte reads.  Scale blocks at or past the end of the
//   contraction are zeroed in registers (their codes are zero, and a NaN
//   scale would turn the zero products into NaN).
// * Byte-gather mode (any N % 32 == 0): every slab, 1-byte direct loads
//   gather exactly the bytes each lane needs.  A 1- or 2-byte direct load
//   writes each lane's value as a zero-extended dword at 4 i (measured),
//   which is the form the MFMA's scale operand takes (opsel 0).  The 4 KiB
//   block holds grad scales [wp][256] then weight scales [wq][256]; position
//   x = 64 u + i of a region holds the scale of block x / 128 of row
//   (column) 32 (i % 4) + 16 (u & 1) + i / 4 of that wave tile, so that one
//   16-byte read gives a lane its four fragments' scales.  This issues one
//   memory request per byte, which costs a quarter of the dense throughput.
enum : int { kGatherMode = 0, kChunkMode = 1, kTensorMode = 2 };

template <int kMode>
constexpr int stage_bytes() { return kMode == kGatherMode ? kTileBytes + kGatherBytes : kTileBytes; }
template <int kMode>
constexpr int chunk_bytes() { return kMode == kChunkMode ? kChunkBytes : 16; }

// The LDS of one workgroup: four slab stages and two scale-chunk buffers.
#define LP_MX_LDS(kMode)                                                                   \
  __shared__ __attribute__((aligned(1024))) uint8_t st0[stage_bytes<kMode>()];             \
  __shared__ __attribute__((aligned(1024))) uint8_t st1[stage_bytes<kMode>()];             \
  __shared__ __attribute__((aligned(1024))) uint8_t st2[stage_bytes<kMode>()];             \
  __shared__ __attribute__((aligned(1024))) uint8_t st3[stage_bytes<kMode>()];             \
  __shared__ __attribute__((aligned(1024))) uint8_t sc0[chunk_bytes<kMode>()];             \
  __shared__ __attribute__((aligned(1024))) uint8_t sc1[chunk_bytes<kMode>()]

// Persistent grad_X (mx_tile_pair): the epilogue writes with buffer stores
// whose masked elements take an out-of-range offset, so that every wave
// issues exactly kEpiStores store instructions per tile and the next tile's
// first barrier, which waits for loads issued before those stores (vector
// memory operations complete in issue order), can count them.
constexpr int kEpiStores = XWP * XWQ * 2 / (64 * 16);     // 16-byte stores per wave and tile
constexpr int kEpiRows = 32;                              // rows per epilogue pass

// What a persistent workgroup carries from one tile to the next.
struct Persist {
  int32_t* ends;     // LDS holding the group ends (a stage may hold the next prologue)
  int next;          // the workgroup's next tile (>= ntiles: none)
  bool issued;       // this tile's prologue was issued by the previous tile
  GroupHit hint;     // the group walk's last hit (the workgroup's tiles only move forward)
};

// One output tile.  hw: the workgroup's index among p.ntiles (see
// select_tile); indices at or past p.ntiles have no tile.  kFP, kFQ: MFMA
// format codes of the gradient and the other operand (0 E4M3, 1 E5M2); the
// MX modes take E4M3 only.  Returns kNoTile when hw names no tile, else
// kDone (mx_tile_pair: kDoneNextIssued when the next tile's prologue has
// been issued).
enum : int { kNoTile = 0, kDone = 1, kDoneNextIssued = 2 };
template <bool kDW, int kMode, int kFP = 0, int kFQ = 0>
__device__ __forceinline__ int mx_tile(const Params& p, int hw, uint8_t* st0, uint8_t* st1, uint8_t* st2,
                                        uint8_t* st3, uint8_t* sc0, uint8_t* sc1) {
  constexpr bool kChunk = kMode == kChunkMode, kGather = kMode == kGatherMode;
  static_assert(!kDW || !kGather, "dW scale rows (N or K bytes, multiples of 16) always load in chunks");
  static_assert(kMode == kTensorMode || (kFP == 0 && kFQ == 0), "MX operands are E4M3");
  constexpr int kStage = stage_bytes<kMode>();
  constexpr int T = kGather ? 12 : 8;                            // direct loads per wave and slab
  constexpr int S = 2;                                           // chunk loads per wave
  constexpr int UNROLL = kChunk ? 2 * kChunkSlabs : 4;           // stage, register set and chunk buffer fixed
  static_assert(kMaxGroups * 4 <= kStage, "group ends alias stage 0");
  static_assert(XWP * XWQ * 2 <= kStage, "epilogue staging fits a stage");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave >> 1, wq = wave & 1;
  if (hw >= p.ntiles) return kNoTile;
  const Tile t = select_tile<XCfg, kDW>(p, reinterpret_cast<int32_t*>(st0), hw);
  if (!t.valid) return kNoTile;
  __syncthreads();                                               // group ends read; stage 0 reusable

  const int ldp = p.P.code_ld;                                   // N bytes per gradient row
  const int sldp = p.P.scale_ld;                                 // dX: N / 32; dW: N (scales per 32 rows)
  const int ldq = p.Q.code_ld;                                   // K bytes per weight row
  const int sldq = p.Q.scale_ld;                                 // K scale bytes per 32 weight rows
  const int M = p.Ptot;
  const int kbeg = t.kbeg, kend = t.kend;
  const uint8_t* pc = p.P.codes + (int64_t)t.p0 * ldp;
  const uint8_t* ps = p.P.scales + (int64_t)t.p0 * sldp;
  // dX reads only the rows of the tile's group (rows past them read as
  // zeros: their results are never stored); dW reads to the end.
  const int pend = kDW ? M : t.pend;
  const int64_t prow_bytes = (int64_t)(pend - t.p0) * ldp;
  const int64_t psrow_bytes = (int64_t)(pend - t.p0) * sldp;
  // dX: the weight of the tile's group; dW: the input X, one tensor for all
  // groups (its rows are the contraction).
  const int64_t qg = kDW ? 0 : t.g;
  const uint8_t* qc = p.Q.codes + qg * p.Q.code_batch;
  const Rsrc qs_r = make_rsrc(p.Q.scales + qg * p.Q.scale_batch, p.Q.scale_bytes);
  const Rsrc ps_r = kDW ? make_rsrc(p.P.scales, p.P.scale_bytes) : make_rsrc(ps, psrow_bytes);

  // Per-lane parts of the direct loads, fixed for the whole loop; the parts
  // that differ between a wave's loads are uniform (scalar offsets).
  // Gradient codes: wave w fills blocks 4 w + u (u = 0..3) of 16 rows x 64 B;
  // lane i takes row 16 (4 w + u) + i / 4, physical chunk i % 4, whose
  // logical chunk (i % 4) ^ p_swz(row) = (i % 4) ^ ((i >> 4) & 3) is the same
  // for every u.
  const int pchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const int32_t p_off = (16 * 4 * wave + lane / 4) * ldp + 16 * pchunk;     // + 16 u ldp
  const int p_col = 16 * pchunk;                                 // first slab column of the lane's chunk
  // Weight codes: blocks 4 w + u of 4 rows x 256 B; lane i takes row
  // n = 4 (4 w + u) + i / 16, logical chunk (i % 16) ^ q_swz(n), which is
  // c0 ^ 8 (u & 1) with c0 = (i % 16) ^ 2 (i / 16).
  const int qc0 = (lane & 15) ^ (2 * (lane >> 4));
  const int32_t q_base = (16 * wave + lane / 16) * ldq + t.q0;   // + 4 u ldq
  const int32_t q_off_even = q_base + 16 * qc0, q_off_odd = q_base + 16 * (qc0 ^ 8);
  // dW: the gradient tile is loaded like the weight tile, at columns p0.
  const int32_t pq_base = (16 * wave + lane / 16) * ldp + t.p0;
  const int32_t pq_off_even = pq_base + 16 * qc0, pq_off_odd = pq_base + 16 * (qc0 ^ 8);
  // Byte-gather mode: waves 0, 1 gather the grad regions, waves 2, 3 the
  // weight regions, 64 positions per load u.
  const bool s_grad = wave < 2;
  const int s_rc = (wave & 1) * 128 + 32 * (lane & 3) + lane / 4;   // + 16 (u & 1)
  const int32_t s_lane = s_grad ? s_rc * sldp : t.q0 + s_rc;
  const int32_t s_rstep = s_grad ? sldp : 1;                     // per row (column)
  const int32_t s_bstep = s_grad ? 1 : sldq;                     // per scale block
  const Rsrc s_rsrc = s_grad ? ps_r : qs_r;
  const int s_dst = kTileBytes + 1024 * wave;

  auto stage = [&](auto si) -> uint8_t* {
    constexpr int I = decltype(si)::value % 4;
    if constexpr (I == 0) return st0;
    else if constexpr (I == 1) return st1;
    else if constexpr (I == 2) return st2;
    else return st3;
  };
  auto chunkbuf = [&](auto ci) -> uint8_t* {
    if constexpr (decltype(ci)::value % 2 == 0) return sc0;
    else return sc1;
  };

  // Direct loads of the slab at contraction k0 into stage buffer `sb`,
  // item u: gradient codes (0..3), weight codes (4..7), gathered scale bytes
  // (8..11, byte-gather mode).  In dX a gradient row runs on into the next
  // row, so a 16-byte chunk at or past the end of the contraction (N % 16
  // == 0) is read as zeros.
  auto issue = [&](auto ui, uint8_t* sb, int k0) {
    constexpr int u = decltype(ui)::value;
    if constexpr (u < 4 && kDW) {
      const Rsrc r = make_rsrc(p.P.codes + (int64_t)k0 * ldp, (int64_t)(kend - k0) * ldp);
      dma<16>(r, (lds_void*)(sb + 1024 * (4 * wave + u)), (u & 1) ? pq_off_odd : pq_off_even, 4 * u * ldp);
    } else if constexpr (u < 4) {
      const Rsrc r = make_rsrc(pc + k0, prow_bytes - k0);
      const bool out = k0 + p_col >= kend;
      dma<16>(r, (lds_void*)(sb + 1024 * (4 * wave + u)), out ? kOOB : p_off, 16 * u * ldp);
    } else if constexpr (u < 8) {
      constexpr int v = u - 4;
      const Rsrc r = make_rsrc(qc + (int64_t)k0 * ldq, (int64_t)(kend - k0) * ldq);
      dma<16>(r, (lds_void*)(sb + kPBytes + 1024 * (4 * wave + v)), (v & 1) ? q_off_odd : q_off_even, 4 * v * ldq);
    } else {
      constexpr int v = u - 8;
      const bool out = k0 + 32 * (v / 2) >= kend;
      const int32_t so = 16 * (v & 1) * s_rstep + ((k0 >> 5) + v / 2) * s_bstep;
      dma<1>(s_rsrc, (lds_void*)(sb + s_dst + 256 * v), out ? kOOB : s_lane, so);
    }
  };
  // Chunk mode: scale blocks [kb, kb + 16) of the tile, kb = k0 / 32 of the
  // chunk's first slab.  Gradient: row 64 w + i, 16 bytes; weight: block row
  // 4 w + i / 16, 16 bytes at column 16 (i % 16).
  auto issue_chunk = [&](uint8_t* cb, int k0) {
    const int kb = k0 >> 5;
    if constexpr (kDW)   // gradient scales [M / 32][N]: block row 4 w + i / 16, columns p0 + 16 (i % 16)
      dma<16>(ps_r, (lds_void*)(cb + 1024 * wave), (4 * wave + lane / 16) * sldp + t.p0 + 16 * (lane & 15), kb * sldp);
    else
      dma<16>(ps_r, (lds_void*)(cb + 1024 * wave), (64 * wave + lane) * sldp, kb);
    dma<16>(qs_r, (lds_void*)(cb + XBP * 16 + 1024 * wave), (4 * wave + lane / 16) * sldq + t.q0 + 16 * (lane & 15),
            kb * sldq);
  };

  // Fragment addresses inside a stage.  Gradient fragment f of lane l: row
  // m = wp 128 + 32 f + l % 32, chunks h and 2 + h (h = l / 32); the swizzle
  // of m does not depend on f, so f is an immediate offset.  Weight fragment
  // j, read tt: rows n = 32 (tt / 2) + 16 h + 8 (tt % 2) + i / 2 (i = l % 16)
  // at chunk (wq 8 + 2 j + (l / 16) % 2) ^ q_swz(n); q_swz(n) depends on i
  // only, and 2 j occupies chunk bits no other term sets, so fragment j is
  // fragment 0's address XOR 32 j and tt an immediate offset.
  const int r32 = lane & 31, hh = lane >> 5;
  const int32_t pa0 = (wp * XWP + r32) * XBK + 16 * (hh ^ p_swz(r32));
  const int32_t pa1 = (wp * XWP + r32) * XBK + 16 * ((2 + hh) ^ p_swz(r32));
  int32_t qa[XFQ];
  {
    const int i16 = lane & 15, c16 = (lane >> 4) & 1;
    const int n0 = 16 * hh + i16 / 2;
    const int32_t a0 = kPBytes + n0 * XBQ + 16 * ((wq * (XWQ / 16) + c16) ^ q_swz(n0)) + 8 * (i16 & 1);
#pragma unroll
    for (int j = 0; j < XFQ; ++j) qa[j] = a0 ^ (32 * j);
  }
  // Scale addresses: byte-gather mode, one 16-byte read per operand;
  // chunk mode, fragment f's byte is at + 16 * 32 f (gradient) or + 32 f
  // (weight), slab position s8 in the chunk adds 2 s8 (gradient) or
  // 2 s8 * 256 (weight).
  int32_t pqa[XFP];                                              // dW: gradient fragments like the weight's
  {
    const int i16 = lane & 15, c16 = (lane >> 4) & 1;
    const int n0 = 16 * hh + i16 / 2;
    const int32_t a0 = n0 * XBQ + 16 * ((wp * (XWP / 16) + c16) ^ q_swz(n0)) + 8 * (i16 & 1);
#pragma unroll
    for (int f = 0; f < XFP; ++f) pqa[f] = a0 ^ (32 * f);
  }
  const int32_t psa = kDW ? hh * XBP + wp * XWP + r32
                          : (kChunk ? 16 * (wp * XWP + r32) + hh : kTileBytes + wp * 1024 + (hh * 32 + r32) * 16);
  const int32_t qsa = kChunk ? XBP * 16 + hh * XBQ + wq * XWQ + r32
                             : kTileBytes + 2048 + wq * 1024 + (hh * 32 + r32) * 16;

  i32x8 pf[2][XFP], qf[2][XFQ];
  int32_t psc[2][XFP], qsc[2][XFQ];
  bool sval[2];                                                  // chunk mode: this lane's scale block exists
  // Read r of the fragments of the slab at contraction k0 (stage sb, slab
  // position S8 in its scale chunk cb) into register set SET: gradient
  // fragments (two 16-byte reads each), weight fragments (four transposing
  // reads each), then the scales.
  constexpr int NFRAG = 2 * XFP + 4 * XFQ;
  constexpr int NREAD = NFRAG + (kChunk ? XFP + XFQ : kGather ? 2 : 0);
  auto read = [&](auto ri, auto seti, auto s8i, const uint8_t* sb, const uint8_t* cb, int k0) {
    constexpr int r = decltype(ri)::value, SET = decltype(seti)::value, S8 = decltype(s8i)::value;
    if constexpr (r < 2 * XFP && kDW) {
      constexpr int f = r / 2, e = r % 2;                        // two transposing reads per r
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int tt = 2 * e + h2;
        const int toff = (32 * (tt / 2) + 8 * (tt % 2)) * XBQ;
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(sb + pqa[f] + toff));
        pf[SET][f][2 * tt] = v[0];
        pf[SET][f][2 * tt + 1] = v[1];
      }
    } else if constexpr (r < 2 * XFP) {
      constexpr int f = r / 2, e = r % 2;
      const u32x4 v = *reinterpret_cast<const u32x4*>(sb + (e ? pa1 : pa0) + f * 32 * XBK);
#pragma unroll
      for (int d = 0; d < 4; ++d) pf[SET][f][4 * e + d] = (int)v[d];
    } else if constexpr (r < NFRAG) {
      constexpr int j = (r - 2 * XFP) / 4, tt = (r - 2 * XFP) % 4;
      constexpr int toff = (32 * (tt / 2) + 8 * (tt % 2)) * XBQ;
      const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(sb + qa[j] + toff));
      qf[SET][j][2 * tt] = v[0];
      qf[SET][j][2 * tt + 1] = v[1];
    } else if constexpr (kGather) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(sb + (r == NFRAG ? psa : qsa));
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if constexpr (r == NFRAG) psc[SET][f] = (int)v[f];
        else qsc[SET][f] = (int)v[f];
      }
    } else {
      // Raw bytes: masking them here would make the wave wait for every LDS
      // read in flight in the middle of the MFMA stream; `scales` masks them
      // at the top of the slab that uses them.
      if constexpr (r == NFRAG) sval[SET] = k0 + 32 * hh < kend;
      if constexpr (r < NFRAG + XFP) {
        constexpr int f = r - NFRAG;
        psc[SET][f] = kDW ? cb[psa + 32 * f + 2 * S8 * XBP] : cb[psa + 16 * 32 * f + 2 * S8];
      } else {
        constexpr int j = r - NFRAG - XFP;
        qsc[SET][j] = cb[qsa + 32 * j + 2 * S8 * XBQ];
      }
    }
  };
  // Chunk mode, at the top of a slab: scale blocks at or past the end of the
  // contraction are zeroed (their codes are zero, and a NaN scale would turn
  // the zero products into NaN).
  auto scales = [&](auto seti) {
    constexpr int SET = decltype(seti)::value;
    if constexpr (kChunk) {
#pragma unroll
      for (int i = 0; i < XFP; ++i) psc[SET][i] = sval[SET] ? psc[SET][i] : 0;
#pragma unroll
      for (int j = 0; j < XFQ; ++j) qsc[SET][j] = sval[SET] ? qsc[SET][j] : 0;
    }
  };

  f32x16 acc[XFP][XFQ];
#pragma unroll
  for (int i = 0; i < XFP; ++i)
#pragma unroll
    for (int j = 0; j < XFQ; ++j) acc[i][j] = f32x16{};

  auto mfma = [&](auto mi, auto seti) {
    constexpr int m = decltype(mi)::value, SET = decltype(seti)::value;
    constexpr int i = m / XFQ, j = m % XFQ;
    if constexpr (kMode == kTensorMode)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[SET][j], pf[SET][i], acc[i][j], kFQ, kFP, 0,
                                                                   127, 0, 127);
    else
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[SET][j], pf[SET][i], acc[i][j], 0, 0, 0,
                                                                   qsc[SET][j], 0, psc[SET][i]);
  };
  constexpr int NM = XFP * XFQ;

  const int nk = (kend - kbeg + XBK - 1) / XBK;
  if (nk > 0) {
    // Prologue: (chunk 0,) slabs 0, 1, 2 in flight; slab 0 landed and
    // published; its fragments read.
    if constexpr (kChunk) issue_chunk(chunkbuf(IC<0>{}), kbeg);
    static_for<3>([&](auto si) {
      constexpr int s = decltype(si)::value;
      static_for<T>([&](auto u) { issue(u, stage(si), kbeg + s * XBK); });
    });
    barrier_vm<2 * T>();
    static_for<NREAD>([&](auto r) { read(r, IC<0>{}, IC<0>{}, stage(IC<0>{}), chunkbuf(IC<0>{}), kbeg); });
  }

  // Slab k = kt + J (stage J % 4): publish slab k+1, issue slab k+3 into the
  // stage of slab k-1 (in chunk mode, first the next scale chunk at chunk
  // position 4), multiply slab k while reading slab k+1's fragments.
  auto slab = [&](auto ji, int k) {
    constexpr int J = decltype(ji)::value;
    constexpr int CUR = J & 1, NXT = CUR ^ 1;
    constexpr int S8 = J % kChunkSlabs, S8N = (J + 1) % kChunkSlabs;
    // Loads issued after slab k+1's tiles: slab k+2's, plus a scale chunk
    // issued at chunk position 4 of slab k-1.
    barrier_vm<T + ((kChunk && S8 == 5) ? S : 0)>();
    uint8_t* const nxt = stage(IC<J + 1>{});
    uint8_t* const dst = stage(IC<J + 3>{});
    const uint8_t* const cnxt = chunkbuf(IC<(J + 1) / kChunkSlabs>{});
    const int k3 = kbeg + (k + 3) * XBK;
    const int k1 = kbeg + (k + 1) * XBK;
    if constexpr (kChunk && S8 == 4) issue_chunk(chunkbuf(IC<J / kChunkSlabs + 1>{}), kbeg + (k + 4) * XBK);
    scales(IC<CUR>{});
    static_for<NM>([&](auto mi) {
      constexpr int m = decltype(mi)::value;
      mfma(mi, IC<CUR>{});
      static_for<T>([&](auto ui) {                                   // loads over the first MFMAs
        if constexpr (decltype(ui)::value == m) issue(ui, dst, k3);
      });
      static_for<NREAD>([&](auto ri) {                               // reads over all of them
        if constexpr (decltype(ri)::value * NM / NREAD == m) read(ri, IC<NXT>{}, IC<S8N>{}, nxt, cnxt, k1);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int kt = 0; kt < nk; kt += UNROLL) {
    static_for<UNROLL>([&](auto ji) {
      constexpr int J = decltype(ji)::value;
      if (kt + J < nk) slab(ji, kt + J);
    });
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  {
    uint8_t* stg = wave == 0 ? st0 : wave == 1 ? st1 : wave == 2 ? st2 : st3;
    if constexpr (kMode == kTensorMode)
      store_acc<XCfg, kDW, true>(p, t, acc, wp, wq, lane, stg, *p.P.tensor_scale * *p.Q.tensor_scale);
    else
      store_acc<XCfg, kDW>(p, t, acc, wp, wq, lane, stg);
    return kDone;
  }
}

template <bool kDW, int kMode, int kFP = 0, int kFQ = 0>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void fp8_mfma_kernel(Params p) {
  LP_MX_LDS(kMode);
  mx_tile<kDW, kMode, kFP, kFQ>(p, blockIdx.x, st0, st1, st2, st3, sc0, sc1);
}

// ---------------------------------------------------------------- paired stages
// Persistent grad_X (MXFP8, chunk mode) with 128-deep stages.  A stage holds
// two 64-deep halves: the gradient tile [256 m][128 B] and the weight tile
// [128 n][256 B], 64 KiB together, in two LDS buffers.  Against the four
// 64-deep stages of mx_tile this halves the barriers (one per stage) and
// makes each gradient row's load one whole 128-byte line instead of two
// halves of one in consecutive slabs.
//
// Schedule, in 64-deep halves h (stage j = h / 2 in buffer j % 2):
// * the fragments of half h + 1 are read during the MFMAs of half h;
// * at the start of every odd half 2j+1 one barrier (vmcnt(0)) publishes
//   stage j+1, whose loads were issued at the start of half 2j-1; every wave
//   then has its half-2j+1 fragments in registers, so buffer j % 2 is free
//   and stage j+2's loads go into it, spread over the half's MFMAs;
// * a scale chunk (8 halves) is issued at chunk position 3 and lands by the
//   barrier of position 7, before position 8 reads it.
// The load lead is thus two halves, as with mx_tile's three slabs ahead of
// four stages.  A persistent workgroup issues the next tile's first scale
// chunk and stage 0 before storing the current tile's results, which it
// stages through buffer 1; stage 1 follows at the next tile's start.
constexpr int YBK = 2 * XBK;                    // contraction per stage
constexpr int kYPBytes = XBP * YBK;             // gradient codes per stage
constexpr int kYStage = kYPBytes + YBK * XBQ;   // plus weight codes
constexpr int TY = 16;                          // direct loads per wave and stage
static_assert(XWQ * 2 * kEpiRows * 4 <= kYStage, "four waves' epilogue passes fit one stage");

// Gradient tile [m][128 B]: chunk c of row m at c ^ ((m >> 1) & 7); the 16
// rows a fragment read serves together hit 16 distinct slots mod 256 B.
__device__ __forceinline__ int y_swz(int m) { return (m >> 1) & 7; }

template <int kFP, int kFQ>
__device__ __forceinline__ int mx_tile_pair(const Params& p, int hw, uint8_t* s0, uint8_t* s1, uint8_t* sc0,
                                             uint8_t* sc1, Persist* pst) {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wp = wave >> 1, wq = wave & 1;
  if (hw >= p.ntiles) return kNoTile;
  const Tile t = select_tile<XCfg, false>(p, pst->ends, hw, true, &pst->hint);
  if (!t.valid) return kNoTile;
  __syncthreads();                                               // the previous epilogue's staging read

  const int ldp = p.P.code_ld, sldp = p.P.scale_ld;
  const int ldq = p.Q.code_ld, sldq = p.Q.scale_ld;
  const int M = p.Ptot;
  const int kbeg = t.kbeg, kend = t.kend;
  const uint8_t* pc = p.P.codes + (int64_t)t.p0 * ldp;
  const int64_t prow_bytes = (int64_t)(t.pend - t.p0) * ldp;
  const Rsrc ps_r = make_rsrc(p.P.scales + (int64_t)t.p0 * sldp, (int64_t)(t.pend - t.p0) * sldp);
  const uint8_t* qc = p.Q.codes + (int64_t)t.g * p.Q.code_batch;
  const Rsrc qs_r = make_rsrc(p.Q.scales + (int64_t)t.g * p.Q.scale_batch, p.Q.scale_bytes);

  // Gradient codes: wave w fills blocks 8 w + u (u = 0..7) of 8 rows x
  // 128 B; lane i takes row 64 w + 8 u + i / 8, physical chunk i % 8, whose
  // logical chunk (i % 8) ^ y_swz(row) = (i % 8) ^ (4 (u & 1) + i / 16)
  // depends on u's parity only.
  const int pl_even = (lane & 7) ^ (lane >> 4), pl_odd = (lane & 7) ^ (4 + (lane >> 4));
  const int32_t p_row = (64 * wave + lane / 8) * ldp;            // + 8 u ldp
  const int32_t p_off_even = p_row + 16 * pl_even, p_off_odd = p_row + 16 * pl_odd;
  // Weight codes: blocks 8 w + v of 4 rows x 256 B; lane i takes row
  // 32 w + 4 v + i / 16, logical chunk (i % 16) ^ q_swz(row) = c0 ^ 8 (v & 1).
  const int qc0 = (lane & 15) ^ (2 * (lane >> 4));
  const int32_t q_base = (32 * wave + lane / 16) * ldq + t.q0;  // + 4 v ldq
  const int32_t q_off_even = q_base + 16 * qc0, q_off_odd = q_base + 16 * (qc0 ^ 8);

  auto stagebuf = [&](auto bi) -> uint8_t* {
    if constexpr (decltype(bi)::value % 2 == 0) return s0;
    else return s1;
  };
  auto chunkbuf = [&](auto ci) -> uint8_t* {
    if constexpr (decltype(ci)::value % 2 == 0) return sc0;
    else return sc1;
  };
  // Direct load u of the stage starting at contraction k0 into buffer sb:
  // gradient codes (0..7), weight codes (8..15).  A gradient row runs on
  // into the next row, so a 16-byte chunk at or past the end of the
  // contraction (N % 16 == 0) is read as zeros.
  auto issue = [&](auto ui, uint8_t* sb, int k0) {
    constexpr int u = decltype(ui)::value;
    if constexpr (u < 8) {
      const Rsrc r = make_rsrc(pc + k0, prow_bytes - k0);
      const bool out = k0 + 16 * ((u & 1) ? pl_odd : pl_even) >= kend;
      dma<16>(r, (lds_void*)(sb + 1024 * (8 * wave + u)), out ? kOOB : ((u & 1) ? p_off_odd : p_off_even),
              8 * u * ldp);
    } else {
      constexpr int v = u - 8;
      const Rsrc r = make_rsrc(qc + (int64_t)k0 * ldq, (int64_t)(kend - k0) * ldq);
      dma<16>(r, (lds_void*)(sb + kYPBytes + 1024 * (8 * wave + v)), (v & 1) ? q_off_odd : q_off_even,
              4 * v * ldq);
    }
  };
  // Scale blocks [kb, kb + 16) of the tile (kb = k0 / 32): gradient row
  // 64 w + i, 16 bytes; weight block row 4 w + i / 16, 16 bytes at column
  // 16 (i % 16).
  auto issue_chunk = [&](uint8_t* cb, int k0) {
    const int kb = k0 >> 5;
    dma<16>(ps_r, (lds_void*)(cb + 1024 * wave), (64 * wave + lane) * sldp, kb);
    dma<16>(qs_r, (lds_void*)(cb + XBP * 16 + 1024 * wave), (4 * wave + lane / 16) * sldq + t.q0 + 16 * (lane & 15),
            kb * sldq);
  };

  // Fragment addresses inside a stage.  Gradient fragment f of lane l: row
  // m = wp 128 + 32 f + l % 32 (y_swz(m) = y_swz(l % 32)), read e of half s:
  // logical chunk 4 s + 2 e + l / 32.  Weight fragment j, read tt, half s:
  // rows n = 64 s + 32 (tt / 2) + 16 h + 8 (tt % 2) + i / 2, as in mx_tile.
  const int r32 = lane & 31, hh = lane >> 5;
  int32_t pa[2][2];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int e = 0; e < 2; ++e) pa[s2][e] = (wp * XWP + r32) * YBK + 16 * ((4 * s2 + 2 * e + hh) ^ y_swz(r32));
  int32_t qa[XFQ];
  {
    const int i16 = lane & 15, c16 = (lane >> 4) & 1;
    const int n0 = 16 * hh + i16 / 2;
    const int32_t a0 = kYPBytes + n0 * XBQ + 16 * ((wq * (XWQ / 16) + c16) ^ q_swz(n0)) + 8 * (i16 & 1);
#pragma unroll
    for (int j = 0; j < XFQ; ++j) qa[j] = a0 ^ (32 * j);
  }
  const int32_t psa = 16 * (wp * XWP + r32) + hh;
  const int32_t qsa = XBP * 16 + hh * XBQ + wq * XWQ + r32;

  i32x8 pf[2][XFP], qf[2][XFQ];
  int32_t psc[2][XFP], qsc[2][XFQ];
  bool sval[2];
  constexpr int NFRAG = 2 * XFP + 4 * XFQ;
  constexpr int NREAD = NFRAG + XFP + XFQ;
  // Read r of half SS of the stage in sb (scale-chunk position S8 in cb,
  // the half starting at contraction k0) into register set SET.
  auto read = [&](auto ri, auto seti, auto ssi, auto s8i, const uint8_t* sb, const uint8_t* cb, int k0) {
    constexpr int r = decltype(ri)::value, SET = decltype(seti)::value;
    constexpr int SS = decltype(ssi)::value, S8 = decltype(s8i)::value;
    if constexpr (r < 2 * XFP) {
      constexpr int f = r / 2, e = r % 2;
      const u32x4 v = *reinterpret_cast<const u32x4*>(sb + pa[SS][e] + f * 32 * YBK);
#pragma unroll
      for (int d = 0; d < 4; ++d) pf[SET][f][4 * e + d] = (int)v[d];
    } else if constexpr (r < NFRAG) {
      constexpr int j = (r - 2 * XFP) / 4, tt = (r - 2 * XFP) % 4;
      constexpr int toff = (64 * SS + 32 * (tt / 2) + 8 * (tt % 2)) * XBQ;
      const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(sb + qa[j] + toff));
      qf[SET][j][2 * tt] = v[0];
      qf[SET][j][2 * tt + 1] = v[1];
    } else {
      if constexpr (r == NFRAG) sval[SET] = k0 + 32 * hh < kend;
      if constexpr (r < NFRAG + XFP) {
        constexpr int f = r - NFRAG;
        psc[SET][f] = cb[psa + 16 * 32 * f + 2 * S8];
      } else {
        constexpr int j = r - NFRAG - XFP;
        qsc[SET][j] = cb[qsa + 32 * j + 2 * S8 * XBQ];
      }
    }
  };
  auto scales = [&](auto seti) {
    constexpr int SET = decltype(seti)::value;
#pragma unroll
    for (int i = 0; i < XFP; ++i) psc[SET][i] = sval[SET] ? psc[SET][i] : 0;
#pragma unroll
    for (int j = 0; j < XFQ; ++j) qsc[SET][j] = sval[SET] ? qsc[SET][j] : 0;
  };

  f32x16 acc[XFP][XFQ];
#pragma unroll
  for (int i = 0; i < XFP; ++i)
#pragma unroll
    for (int j = 0; j < XFQ; ++j) acc[i][j] = f32x16{};
  auto mfma = [&](auto mi, auto seti) {
    constexpr int m = decltype(mi)::value, SET = decltype(seti)::value;
    constexpr int i = m / XFQ, j = m % XFQ;
    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[SET][j], pf[SET][i], acc[i][j], kFQ, kFP, 0,
                                                                 qsc[SET][j], 0, psc[SET][i]);
  };
  constexpr int NM = XFP * XFQ;
  static_assert(TY == NM, "one stage load per MFMA of an odd half");

  const int nh = (kend - kbeg + XBK - 1) / XBK;                 // 64-deep halves
  const int npair = (nh + 1) / 2;
  if (nh > 0) {
    // Prologue: chunk 0 and stages 0 and 1 in flight, chunk 0 and stage 0
    // landed and published, half 0's fragments read.
    if (!pst->issued) {
      issue_chunk(sc0, kbeg);
      static_for<TY>([&](auto u) { issue(u, s0, kbeg); });
      static_for<TY>([&](auto u) { issue(u, s1, kbeg + YBK); });
      barrier_vm<TY>();
    } else {
      // Chunk 0 and stage 0 came before the previous tile's result stores.
      static_for<TY>([&](auto u) { issue(u, s1, kbeg + YBK); });
      barrier_vm<TY + kEpiStores>();
    }
    static_for<NREAD>([&](auto r) { read(r, IC<0>{}, IC<0>{}, IC<0>{}, s0, sc0, kbeg); });
  }

  // Half h = 2 jj + SS (H = h mod 16: stage buffer (H / 2) % 2, scale chunk
  // (H / 8) % 2, chunk position H % 8).
  auto half = [&](auto hi, int h) {
    constexpr int H = decltype(hi)::value;
    constexpr int SS = H % 2, CUR = H & 1, NXT = CUR ^ 1;
    constexpr int S8 = H % 8, S8N = (H + 1) % 8;
    uint8_t* const cur = stagebuf(IC<H / 2>{});
    uint8_t* const nsb = stagebuf(IC<(H + 1) / 2>{});
    const uint8_t* const cnxt = chunkbuf(IC<(H + 1) / 8>{});
    const int k1 = kbeg + (h + 1) * XBK;
    const int k2 = kbeg + (h + 3) * XBK;                         // stage jj + 2
    if constexpr (SS == 1) {
      barrier_vm<0>();
      if constexpr (S8 == 3) issue_chunk(chunkbuf(IC<H / 8 + 1>{}), kbeg + (h + 5) * XBK);
    }
    scales(IC<CUR>{});
    static_for<NM>([&](auto mi) {
      constexpr int m = decltype(mi)::value;
      mfma(mi, IC<CUR>{});
      if constexpr (SS == 1) issue(mi, cur, k2);
      static_for<NREAD>([&](auto ri) {
        if constexpr (decltype(ri)::value * NM / NREAD == m) read(ri, IC<NXT>{}, IC<SS ^ 1>{}, IC<S8N>{}, nsb, cnxt, k1);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int jt = 0; jt < npair; jt += 8) {
    static_for<16>([&](auto hi) {
      constexpr int H = decltype(hi)::value;
      if (jt + H / 2 < npair) half(hi, 2 * jt + H);
    });
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();

  // The next tile's first scale chunk and stage 0, then this tile's results.
  bool issued = false;
  if (pst->next < p.ntiles) {
    const Tile tn = select_tile<XCfg, false>(p, pst->ends, pst->next, true, &pst->hint);
    if (tn.valid && tn.kend > tn.kbeg) {
      const uint8_t* const npc = p.P.codes + (int64_t)tn.p0 * ldp;
      const int64_t nprow = (int64_t)(tn.pend - tn.p0) * ldp;
      const uint8_t* const nqc = p.Q.codes + (int64_t)tn.g * p.Q.code_batch;
      const Rsrc nps_r = make_rsrc(p.P.scales + (int64_t)tn.p0 * sldp, (int64_t)(tn.pend - tn.p0) * sldp);
      const Rsrc nqs_r = make_rsrc(p.Q.scales + (int64_t)tn.g * p.Q.scale_batch, p.Q.scale_bytes);
      const int32_t nq_base = (32 * wave + lane / 16) * ldq + tn.q0;
      const int k0 = tn.kbeg;
      dma<16>(nps_r, (lds_void*)(sc0 + 1024 * wave), (64 * wave + lane) * sldp, k0 >> 5);
      dma<16>(nqs_r, (lds_void*)(sc0 + XBP * 16 + 1024 * wave), (4 * wave + lane / 16) * sldq + tn.q0 + 16 * (lane & 15),
              (k0 >> 5) * sldq);
      static_for<8>([&](auto ui) {
        constexpr int u = decltype(ui)::value;
        const Rsrc r = make_rsrc(npc + k0, nprow - k0);
        const bool out = k0 + 16 * ((u & 1) ? pl_odd : pl_even) >= tn.kend;
        dma<16>(r, (lds_void*)(s0 + 1024 * (8 * wave + u)), out ? kOOB : ((u & 1) ? p_off_odd : p_off_even),
                8 * u * ldp);
      });
      static_for<8>([&](auto vi) {
        constexpr int v = decltype(vi)::value;
        const Rsrc r = make_rsrc(nqc + (int64_t)k0 * ldq, (int64_t)(tn.kend - k0) * ldq);
        dma<16>(r, (lds_void*)(s0 + kYPBytes + 1024 * (8 * wave + v)), nq_base + 16 * ((v & 1) ? (qc0 ^ 8) : qc0),
                4 * v * ldq);
      });
      issued = true;
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // Results through buffer 1: four passes of 32 rows per wave, 8 KiB each,
  // every wave issuing exactly kEpiStores stores (masked ones out of range).
  // (Two passes of 64 rows measured the same.)
  constexpr int ROWB = XWQ * 2;
  int el = lane;
  asm volatile("" : "+v"(el));
  uint8_t* const stg = s1 + wave * (ROWB * kEpiRows);
  const int row0 = t.p0 + wp * XWP, col0 = t.q0 + wq * XWQ;
  const Rsrc orsrc = make_rsrc(p.C + (int64_t)row0 * p.ldc + col0, ((int64_t)(M - row0) * p.ldc - col0) * 2);
  const int c16 = el & 15;
  const bool col_ok = col0 + 8 * c16 < p.Qtot;
#pragma unroll
  for (int i = 0; i < XFP; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    const int r = el & 31;
#pragma unroll
    for (int j = 0; j < XFQ; ++j) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int sl = (j * 32 + 8 * r4 + 4 * (el >> 5)) / 4;
        const u32x2 v = {pack_bf16x2(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1]),
                         pack_bf16x2(acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3])};
        *reinterpret_cast<u32x2*>(stg + r * ROWB + 8 * (sl ^ (r & 15))) = v;
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                          // lgkmcnt(0): the pass is staged
#pragma unroll
    for (int it = 0; it < kEpiRows / 4; ++it) {
      const int rr = it * 4 + el / 16;
      const uint8_t* src = stg + rr * ROWB;
      const u32x2 lo = *reinterpret_cast<const u32x2*>(src + 8 * ((2 * c16) ^ (rr & 15)));
      const u32x2 hi = *reinterpret_cast<const u32x2*>(src + 8 * ((2 * c16 + 1) ^ (rr & 15)));
      const int32_t off = (row0 + i * kEpiRows + rr < t.pend && col_ok) ? ((i * kEpiRows + rr) * p.ldc + 8 * c16) * 2
                                                                        : kOOB;
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{lo[0], lo[1], hi[0], hi[1]}, orsrc, off, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                          // read back before the next pass overwrites
    __builtin_amdgcn_sched_barrier(0);
  }
  return issued ? kDoneNextIssued : kDone;
}

// Persistent grad_X (MXFP8, chunk mode): one workgroup per compute unit
// walks the tile list.  Workgroup b runs on XCD b % 8 (the hardware deals
// workgroups to the XCDs in turn); at each step the 32 workgroups of an XCD
// take 32 consecutive tiles (the column tiles of about one gradient row
// tile, which that XCD's L2 then holds once), and the eight XCDs take
// neighbouring row tiles, so that row tiles of one large expert share that
// expert's weight slices in the Infinity Cache.  The grouped tile list ends
// with its unused entries, so the first missing tile ends the walk.  Tiles
// with an empty contraction issue no loads; the next tile then issues its
// own prologue.
template <int kFP = 0, int kFQ = 0>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void fp8_mfma_paired(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t s0[kYStage];
  __shared__ __attribute__((aligned(1024))) uint8_t s1[kYStage];
  __shared__ __attribute__((aligned(1024))) uint8_t sc0[kChunkBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t sc1[kChunkBytes];
  __shared__ int32_t s_ends[kMaxGroups];
  const int nwg = gridDim.x, xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  Persist ps{s_ends, 0, false, GroupHit{0, 0, 0, 0, false}};
  if (p.offsets != nullptr) {
    for (int i = threadIdx.x; i < p.groups; i += NT) s_ends[i] = p.offsets[i];
    __syncthreads();
  }
  for (int l = xcd * (nwg / 8) + slot; l < p.ntiles; l += nwg) {
    ps.next = l + nwg;
    const int r = mx_tile_pair<kFP, kFQ>(p, l, s0, s1, sc0, sc1, &ps);
    if (r == kNoTile) break;
    ps.issued = r == kDoneNextIssued;
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// grad_X and grad_W of one per-tensor scaled gradient in one launch: the
// first dx_blocks workgroups (dx.ntiles rounded up to a multiple of the 8
// XCDs, so that both parts keep the dispatch-order dealing that
// select_tile assumes) take grad_X's tiles, the rest grad_W's.  When
// neither contraction has tiles enough for every compute unit, the two
// together fill more of the GPU than either one after the other; the
// longer grad_X tiles are dispatched first.  kFQ: format of X and W.
template <int kFP, int kFQ>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void pt_pair_kernel(Params dx, Params dw,
                                                                                                  int dx_blocks) {
  LP_MX_LDS(kTensorMode);
  const int b = blockIdx.x;
  if (b < dx_blocks)
    mx_tile<false, kTensorMode, kFP, kFQ>(dx, b, st0, st1, st2, st3, sc0, sc1);
  else
    mx_tile<true, kTensorMode, kFP, kFQ>(dw, b - dx_blocks, st0, st1, st2, st3, sc0, sc1);
}

}  // namespace gk
}  // namespace lp
