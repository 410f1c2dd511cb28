// grad_X of the deferred MXFP8 recipe with the weight quantized inside the
// product.
//
// "perf: defer mxfp8 backward quantization", MXFP8GMMFunction.op_dx: the
// backward quantizes the bf16 weight along its reduction axis (one E8M0
// scale per 32 rows of W[g], E4M3 codes) and contracts the MXFP8 gradient
// with it; the page trades that backward compute for saved memory.  An
// expert with at most 256 rows is one row tile: its weight is read once
// whichever way it is done, so quantizing it here (rather than in a pass of
// its own that writes the codes and scales, which this product then reads
// back) removes a write and a read of the weight's quantized copy, three
// bytes per element of the four the standalone pass and the read cost.
//
// Tiles: 256 (rows) x 256 (output columns), eight waves (two per SIMD),
// wave w owning output columns 32 w .. 32 w + 31 over all 256 rows, so that
// every weight element is quantized by exactly one lane, in registers, into
// the very MFMA operand that consumes it.  Per 64-deep slab the gradient
// codes (16 KiB) and the bf16 weight slab (64 rows x 256 columns, 32 KiB)
// go from global memory straight into LDS (three buffers each; gradient
// slabs two ahead, weight slabs three); the gradient's scales arrive in
// chunks of eight slabs.  During slab k each wave reads its 32 columns of
// weight slab k + 1 with transposing LDS reads (a lane gets one column's
// rows in pairs, which is the MFMA operand's layout), takes the column
// amax over each 32 rows (its 16 rows and those of the lane 32 away), the
// E8M0 scale byte max(E - 8, 0) (E: exponent field of the bf16 amax), and
// converts with the scaled bf16 -> E4M3 conversion after clamping each
// magnitude to 448 times the scale on the bit patterns: the arithmetic of
// the standalone quantizer (lp_mxq.hpp), bit for bit.  That work is spread
// between slab k's eight MFMAs.  The products are the same block-scaled
// MFMAs, over the same 64-deep steps, as with a weight quantized
// beforehand, so the results are the same bits.
#include "lp_gemm_mx_kernel.hpp"
#include "lp_mxq.hpp"

namespace lp {
namespace gk {

namespace {

constexpr int WBP = 256, WBQ = 256;             // output tile
constexpr int NF = WBP / 32;                    // 32 x 32 blocks per wave: a column strip of 32
constexpr int NT8 = 512;                        // eight waves, two per SIMD
using WCfg = Cfg<WBP, WBQ>;
constexpr int kWTile = XBK * WBQ * 2;           // bf16 weight slab: 64 rows x 512 B
constexpr int kGTile = WBP * XBK;               // gradient codes slab: 256 rows x 64 B
constexpr int kGChunk = WBP * 16;               // gradient scales of one chunk: 256 rows x 16 blocks
constexpr int kWBase = 0, kGBase = 3 * kWTile, kCBase = kGBase + 3 * kGTile;
constexpr int kLds = kCBase + 2 * kGChunk;      // 152 KiB
constexpr int kStageRow = 32 * 2;               // staged result row of a wave (bytes)
static_assert(kMaxGroups * 4 <= kWTile, "group ends alias the first weight buffer");
static_assert(8 * WBP * kStageRow <= kGBase + 3 * kGTile, "epilogue staging fits the slab buffers");

typedef __bf16 bf16x2e __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ uint32_t pk_min_s16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(s16x2, a), __builtin_bit_cast(s16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_subsat_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, a), __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_add_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) + __builtin_bit_cast(u16x2, b));
}

// The workgroup barrier for waves that issue no direct loads: their LDS
// operations done, no wait on the memory counter (their stores).
__device__ __forceinline__ void barrier_lgkm() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// bf16 weight slab [64 rows][512 B]: 16-byte chunk c of row n at physical
// chunk c ^ 4 (n & 3).  A transposing read covers rows n0 .. n0 + 3 and
// n0 + 16 .. n0 + 19 (n0 % 4 == 0) of one 64-byte segment: the swizzle puts
// the four rows of each half on distinct banks.
__device__ __forceinline__ int wb_swz(int n) { return 4 * (n & 3); }

// One listed tile: its group, rows [p0, pend) and first output column; a
// null tile (past a workgroup's list) has valid == false and empty ranges.
struct WTile {
  int g, p0, pend, q0;
  bool valid;
};

template <int kDummy = 0>
__global__ __launch_bounds__(NT8) __attribute__((amdgpu_waves_per_eu(2, 2))) void fp8_mfma_wquant_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kLds];
  __shared__ int32_t s_ends[kMaxGroups];
  // Waves 0 .. 3 issue every direct load, waves 4 .. 7 every store of
  // results: a wave's memory counter covers loads and stores together, in
  // issue order, so a loading wave that stored a tile's results would wait
  // for those stores before it could count the next tile's loads as landed.
  constexpr int TG = 4, TW = 8;                  // direct loads per loading wave and slab: gradient, weight
  constexpr int S = 4;                           // scale chunk loads per loading wave

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int M = p.Ptot, K = p.Qtot, N = p.Ktot;
  for (int i = tid; i < p.groups; i += NT8) s_ends[i] = p.offsets[i];
  __syncthreads();

  // The listed tiles (groups of 1 .. fuse_rows rows, ceil(rows / 256) row
  // tiles each, nq column tiles per row tile), in order of group, then
  // column tile, then row tile.  XCD x (workgroups b with b % 8 == x) takes
  // the x-th eighth of the list and its workgroups deal it out in turn, so
  // that the tiles one XCD runs together are neighbours: column tiles of the
  // same rows, whose gradient rows its L2 then serves, and the row tiles of
  // one weight slice, which its L2 then streams once.
  auto listed = [&](int n) { return n <= p.fuse_rows; };
  const int nlist = find_row_tile<WBP>(s_ends, p.groups, M, INT32_MAX, listed).seen * p.nq;
  const int nslot = gridDim.x / 8, xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int per = (nlist + 7) / 8;
  const int lo = xcd * per, hi = lo + per < nlist ? lo + per : nlist;
  const int first = lo + slot;
  const int mine = first < hi ? (hi - first + nslot - 1) / nslot : 0;
  if (mine == 0) return;
  GroupHit hint{0, 0, 0, 0, false};              // the walk's last hit: tiles come in increasing order
  auto tile_at = [&](int i) __attribute__((always_inline)) {
    WTile t{0, 0, 0, 0, false};
    if (i >= mine) return t;
    const int l = first + i * nslot;
    // A group's n row tiles hold entries [seen nq, (seen + n) nq) of the
    // list, so l / nq names a row tile of l's group.
    const GroupHit h = find_row_tile<WBP>(s_ends, p.groups, M, l / p.nq, listed, &hint);
    if (h.found) {
      hint = h;
      const int n = (h.end - h.start + WBP - 1) / WBP;
      const int local = l - h.seen * p.nq;
      const int col = local / n;
      t.q0 = col * WBQ;
      t.g = h.g;
      t.p0 = h.start + (local - col * n) * WBP;
      t.pend = h.end;
      t.valid = true;
    }
    return t;
  };

  const int ldp = p.P.code_ld;                   // N bytes per gradient row
  const int sldp = p.P.scale_ld;                 // N / 32
  const int ldw = p.Q.code_ld;                   // 2 K bytes per weight row
  const int nk = N / XBK;                        // a multiple of 8 (N % 512 == 0)
  const int wrows_max = 0x7FFFFFFF / ldw;        // weight rows one 32-bit range covers

  const bool loader = wave < 4;
  const int lw = wave & 3;                       // index among the loading (or storing) waves
  // Gradient codes: loading wave w fills blocks 4 w + u of 16 rows x 64 B;
  // lane i takes row 16 (4 w + u) + i / 4, physical chunk i % 4, logical
  // chunk (i % 4) ^ p_swz(row) = (i % 4) ^ ((i >> 4) & 3).
  const int pchunk = (lane & 3) ^ ((lane >> 4) & 3);
  const int32_t p_off = (16 * 4 * lw + lane / 4) * ldp + 16 * pchunk;
  // bf16 weight: loading wave w fills blocks 8 w + v of 2 rows x 512 B;
  // lane i takes row n = 16 w + 2 v + i / 32, physical chunk i % 32,
  // logical chunk (i % 32) ^ wb_swz(n); the swizzle depends on v's parity
  // only.
  auto w_off = [&](int v) __attribute__((always_inline)) {
    const int n = 16 * lw + 2 * v + lane / 32;
    return (int32_t)((16 * lw + lane / 32) * ldw + 16 * ((lane & 31) ^ wb_swz(n)));
  };
  const int32_t w_off0 = w_off(0), w_off1 = w_off(1);
  const int32_t c_off = (16 * 4 * lw + lane / 4) * sldp + 4 * (lane & 3);   // scale chunk pieces

  // Direct loads of slab kk of tile t into the buffers of stream step sg
  // (every slab of a workgroup's tiles is one step of a single stream; a
  // null tile's loads read nothing and leave zeros).  The contraction is a
  // whole number of scale chunks (N % 512 == 0, which the launch checks),
  // so every slab is full.
  auto issue_g = [&](const WTile& t, int kk, int sg) __attribute__((always_inline)) {
    const int k0 = kk * XBK;
    int64_t range = 0;
    if (t.valid) {
      const int64_t rb = (int64_t)(t.pend - t.p0) * ldp - k0;   // the group's rows only: the rest read as zeros
      range = rb < 0 ? 0 : (rb > 0x7FFFFFFF ? 0x7FFFFFFF : rb);
    }
    const Rsrc r = make_rsrc(p.P.codes + (int64_t)t.p0 * ldp + k0, (int64_t)__builtin_amdgcn_readfirstlane((int)range));
    uint8_t* const gb = lds + kGBase + kGTile * (sg % 3);
#pragma unroll
    for (int u = 0; u < TG; ++u) dma<16>(r, (lds_void*)(gb + 1024 * (4 * lw + u)), p_off, 16 * u * ldp);
  };
  auto issue_w = [&](const WTile& t, int kk, int sg) __attribute__((always_inline)) {
    const int k0 = kk * XBK;
    int rows = t.valid ? N - k0 : 0;
    rows = rows < 0 ? 0 : (rows > wrows_max ? wrows_max : rows);
    const uint8_t* const wg = p.Q.codes + (int64_t)t.g * p.Q.code_batch + 2 * (int64_t)t.q0;
    const Rsrc r = make_rsrc(wg + (int64_t)k0 * ldw, (int64_t)__builtin_amdgcn_readfirstlane(rows * ldw));
    uint8_t* const wb = lds + kWBase + kWTile * (sg % 3);
#pragma unroll
    for (int v = 0; v < TW; ++v)
      dma<16>(r, (lds_void*)(wb + 1024 * (8 * lw + v)), (v & 1) ? w_off1 : w_off0, 2 * v * ldw);
  };
  // Gradient scales of the chunk at slab kk ([256 rows][16 B]) into the
  // chunk buffer of step sg: loading wave w fills 256-byte pieces 4 w + s,
  // lane i taking 4 bytes of row 16 (4 w + s) + i / 4.
  auto issue_chunk = [&](const WTile& t, int kk, int sg) __attribute__((always_inline)) {
    const int64_t rb = t.valid ? (int64_t)(t.pend - t.p0) * sldp : 0;
    const Rsrc r = make_rsrc(p.P.scales + (int64_t)t.p0 * sldp, (int64_t)__builtin_amdgcn_readfirstlane((int)(rb < 0x7FFFFFFF ? rb : 0x7FFFFFFF)));
    uint8_t* const cb = lds + kCBase + kGChunk * ((sg / kChunkSlabs) & 1);
#pragma unroll
    for (int sp = 0; sp < S; ++sp)
      dma<4>(r, (lds_void*)(cb + 256 * (4 * lw + sp)), c_off, 16 * sp * sldp + ((kk * XBK) >> 5));
  };

  // Fragments.  Lane l = 32 h + r (h = l / 32, r = l % 32) of an MFMA
  // operand holds row r's contraction elements 16 h .. 16 h + 15 (bytes
  // 0 .. 15) and 32 + 16 h .. 32 + 16 h + 15 (bytes 16 .. 31); its scale byte
  // is that of block h (elements 32 h .. 32 h + 31).  Gradient fragment f:
  // tile row 32 f + r, two 16-byte reads.  Weight fragment: column
  // 32 w + r of the tile, quantized here from eight transposing reads of
  // the bf16 slab, read t giving rows nb(t) .. nb(t) + 3 (nb = 16 h + 4 t
  // for t < 4, 32 + 16 h + 4 (t - 4) after) as two row pairs; in the read,
  // lane i of each 16 supplies row nb + (i % 16) / 4, columns
  // 4 (i % 4) .. + 3 of the group's 16 (groups: l / 16 = 2 h + column half).
  const int r32 = lane & 31, hh = lane >> 5;
  const int32_t pa0 = r32 * XBK + 16 * (hh ^ p_swz(r32));
  const int32_t pa1 = r32 * XBK + 16 * ((2 + hh) ^ p_swz(r32));
  const int32_t psa = 16 * r32 + hh;
  int32_t wa;
  {
    const int i16 = lane & 15, half = (lane >> 4) & 1;
    const int n = 16 * hh + (i16 >> 2);                       // n % 4 == (i16 >> 2), as for every nb + n
    const int byte = 64 * wave + 32 * half + 8 * (i16 & 3);   // logical byte in the 512-byte row
    wa = n * (WBQ * 2) + 16 * ((byte >> 4) ^ wb_swz(n)) + (byte & 15);
  }
  const uint32_t hsh = 16 * hh;                               // this lane's block in packed pairs

  // Quantization state of the next slab's weight fragment.
  uint32_t d[16];                                // bf16 pairs: d[2t], d[2t + 1] = rows nb(t) + 0, 1 and + 2, 3
  uint32_t m0, m1, amx, bsc, thr0, thr1;
  float sc0, sc1;
  bool special;
  auto q_read = [&](const uint8_t* wb) __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int nb = tt < 4 ? 4 * tt : 32 + 4 * (tt - 4);
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(wb + wa + nb * (WBQ * 2)));
      const u32x2 u = __builtin_bit_cast(u32x2, v);
      d[2 * tt] = u[0];
      d[2 * tt + 1] = u[1];
    }
  };
  // Piece b (0, 1): packed magnitude maxima of block b's 16 rows here.
  auto q_amax = [&](auto bi) __attribute__((always_inline)) {
    constexpr int b = decltype(bi)::value;
    uint32_t m = d[8 * b] & 0x7FFF7FFFu;
#pragma unroll
    for (int j = 1; j < 8; ++j) m = pk_umax16(m, d[8 * b + j] & 0x7FFF7FFFu);
    if constexpr (b == 0) m0 = m;
    else m1 = m;
  };
  // Amax of both blocks (low half: block 0), combined with the lane 32
  // away that holds the other 16 rows of each; scale bytes max(E - 8, 0)
  // (E: exponent field of the bf16 amax; 255 flags a NaN or an infinity);
  // the scale 2^(byte - 127) for the conversion and the bf16 magnitude of
  // 448 times it, the clamp that makes the conversion saturate.
  auto q_scale = [&]() __attribute__((always_inline)) {
    const uint32_t lo = __builtin_amdgcn_perm(m1, m0, 0x05040100u);   // m0.lo, m1.lo
    const uint32_t hi = __builtin_amdgcn_perm(m1, m0, 0x07060302u);   // m0.hi, m1.hi
    amx = pk_umax16(lo, hi);
    const auto sw = __builtin_amdgcn_permlane32_swap(amx, amx, false, false);
    amx = pk_umax16(sw[0], sw[1]);
    const uint32_t e = (amx >> 7) & 0x00FF00FFu;
    special = __builtin_amdgcn_ballot_w64(((e + 0x00010001u) & 0x01000100u) != 0u) != 0;
    bsc = pk_subsat_u16(e, 0x00080008u);
    sc0 = __builtin_bit_cast(float, bsc << 23);
    sc1 = __builtin_bit_cast(float, (bsc >> 16) << 23);
    const uint32_t thr = (pk_add_u16(bsc, 0x00080008u) << 7) | 0x00600060u;
    thr0 = __builtin_amdgcn_perm(thr, thr, 0x01000100u);
    thr1 = __builtin_amdgcn_perm(thr, thr, 0x03020302u);
  };
  // Piece pc (0 .. 3): row pairs 4 pc .. 4 pc + 3 -> fragment dwords
  // 2 pc, 2 pc + 1.  Clamp |v| to the threshold on the bit patterns (signed
  // 16-bit min for positive values, unsigned min against sign | threshold
  // for negative ones), then scale and round to nearest even.
  auto q_codes = [&](auto pci, i32x8& qn) __attribute__((always_inline)) {
    constexpr int pcn = decltype(pci)::value;
    static_for<4>([&](auto jji) __attribute__((always_inline)) {
      constexpr int jj = decltype(jji)::value;
      constexpr int j = 4 * pcn + jj;
      const uint32_t tp = j < 8 ? thr0 : thr1;
      const float sc = j < 8 ? sc0 : sc1;
      const uint32_t c = pk_min_u16(pk_min_s16(d[j], tp), tp | 0x80008000u);
      // The first conversion of a dword fills its low half; its old value
      // (the high half, written next) is any register: its own input.
      const s16x2 old = __builtin_bit_cast(s16x2, (jj & 1) ? (uint32_t)qn[j >> 1] : c);
      const s16x2 r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(old, __builtin_bit_cast(bf16x2e, c), sc, (jj & 1) != 0);
      qn[j >> 1] = __builtin_bit_cast(int, r);
    });
  };
  // A block with a NaN or an infinity (never in finite data): scale byte
  // 0xFF and the E4M3 NaN code with each element's sign, as the standalone
  // quantizer writes them.
  auto q_special = [&](i32x8& qn, uint32_t& qs) __attribute__((always_inline)) {
    const bool bad0 = (amx & 0xFFFFu) >= 0x7F80u, bad1 = (amx >> 16) >= 0x7F80u;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
      if (tt < 4 ? bad0 : bad1) qn[tt] = (int)(nan_e4m3x2(d[2 * tt]) | (nan_e4m3x2(d[2 * tt + 1]) << 16));
    if (hh ? bad1 : bad0) qs = 0xFFu;
  };

  i32x8 qf[2];
  uint32_t qsc[2];
  f32x16 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x16{};

  // Prologue: the first tile's chunk 0, slabs 0, 1 (gradient and weight)
  // and weight slab 2 in flight; chunk 0 and slab 0 landed, weight slab 0
  // quantized.
  WTile cur = tile_at(0), nxt = tile_at(1);
  if (loader) {
    issue_chunk(cur, 0, 0);
    issue_g(cur, 0, 0);
    issue_w(cur, 0, 0);
    issue_w(cur, 1, 1);
    issue_g(cur, 1, 1);
    issue_w(cur, 2, 2);
    barrier_vm<TG + 2 * TW>();
  } else {
    barrier_lgkm();
  }
  q_read(lds + kWBase);
  q_amax(IC<0>{});
  q_amax(IC<1>{});
  q_scale();
  static_for<4>([&](auto pci) { q_codes(pci, qf[0]); });
  qsc[0] = bsc >> hsh;
  if (special) q_special(qf[0], qsc[0]);

  // Step sg = slab k of the current tile (position S8 in its scale chunk):
  // the barrier publishes gradient slab sg and weight slab sg + 1 of the
  // stream; issue gradient slab sg + 2 and weight
  // slab sg + 3 (and at position 4 the next scale chunk), of this tile or,
  // near its end, of the next; read weight slab sg + 1, then run slab sg's
  // eight products with the quantization of slab sg + 1 spread between
  // them.
  auto slab = [&](auto ji, int k, int sg) __attribute__((always_inline)) {
    constexpr int S8 = decltype(ji)::value;
    constexpr int CUR = S8 & 1, NXT = CUR ^ 1;
    if (loader) {
      barrier_vm<TG + TW + (S8 == 5 ? S : 0)>();
      if constexpr (S8 == 4) {
        if (k + 4 < nk) issue_chunk(cur, k + 4, sg + 4);
        else issue_chunk(nxt, k + 4 - nk, sg + 4);
      }
      if (k + 2 < nk) issue_g(cur, k + 2, sg + 2);
      else issue_g(nxt, k + 2 - nk, sg + 2);
      if (k + 3 < nk) issue_w(cur, k + 3, sg + 3);
      else issue_w(nxt, k + 3 - nk, sg + 3);
    } else {
      barrier_lgkm();
    }
    const uint8_t* const gb = lds + kGBase + kGTile * (sg % 3);
    const uint8_t* const cb = lds + kCBase + kGChunk * ((sg / kChunkSlabs) & 1);
    q_read(lds + kWBase + kWTile * ((sg + 1) % 3));
    i32x8 pf[2];
    int32_t psc[2];
    auto read_p = [&](auto fi) __attribute__((always_inline)) {
      constexpr int f = decltype(fi)::value;
      const u32x4 a = *reinterpret_cast<const u32x4*>(gb + pa0 + f * 32 * XBK);
      const u32x4 b = *reinterpret_cast<const u32x4*>(gb + pa1 + f * 32 * XBK);
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        pf[f & 1][dd] = (int)a[dd];
        pf[f & 1][4 + dd] = (int)b[dd];
      }
      psc[f & 1] = cb[psa + 16 * 32 * f + 2 * S8];
    };
    auto mfma = [&](auto fi) __attribute__((always_inline)) {
      constexpr int f = decltype(fi)::value;
      acc[f] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qf[CUR], pf[f & 1], acc[f], 0, 0, 0, (int)qsc[CUR], 0,
                                                               psc[f & 1]);
    };
    read_p(IC<0>{});
    __builtin_amdgcn_sched_barrier(0);
    static_for<NF>([&](auto fi) {
      constexpr int f = decltype(fi)::value;
      if constexpr (f + 1 < NF) read_p(IC<f + 1>{});
      mfma(fi);
      if constexpr (f == 0) q_amax(IC<0>{});
      else if constexpr (f == 1) q_amax(IC<1>{});
      else if constexpr (f == 2) q_scale();
      else if constexpr (f >= 3 && f <= 6) q_codes(IC<f - 3>{}, qf[NXT]);
      else qsc[NXT] = bsc >> hsh;
      __builtin_amdgcn_sched_barrier(0);
    });
    if (__builtin_expect(special, false)) {
      // A use of the products on this path too: otherwise the compiler
      // sinks them past the branch, after the quantization above.
#pragma unroll
      for (int f = 0; f < NF; ++f) asm volatile("" ::"v"(acc[f]));
      q_special(qf[NXT], qsc[NXT]);
    }
  };

  // Results of a tile: fp32 -> bf16 (nearest even) staged through the
  // weight buffer that slab sg - 1 finished with (the stream refills it only
  // at step sg), 64 rows at a time (16-byte chunk c of staged row r at
  // c ^ (r % 32)), then stored by the storing waves as whole 512-byte row
  // segments, 1 KiB per store (register-direct stores of 16-byte pieces
  // cost far more).  Only rows of the tile's group are staged and stored
  // (a column group past K is sent out of range).
  auto store_tile = [&](const WTile& t, uint8_t* stg) __attribute__((always_inline)) {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // every wave done reading the buffer
    const int nrows = t.pend - t.p0;
    const Rsrc out = make_rsrc(p.C + (int64_t)t.p0 * p.ldc, (int64_t)nrows * p.ldc * 2);
    const int ccol = t.q0 + 8 * (lane & 31);
    const bool cok = ccol < K;
#pragma unroll
    for (int rnd = 0; rnd < NF / 2; ++rnd) {
      if (64 * rnd >= nrows) break;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int f = 2 * rnd + h;
        const int r = 32 * h + r32;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int phys = (4 * wave + r4) ^ r32;
          const u32x2 v = {pack_bf16x2(acc[f][4 * r4], acc[f][4 * r4 + 1]),
                           pack_bf16x2(acc[f][4 * r4 + 2], acc[f][4 * r4 + 3])};
          *reinterpret_cast<u32x2*>(stg + r * (WBQ * 2) + 16 * phys + 8 * hh) = v;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if (!loader) {
        // Row r = 16 w + 2 j + h of the round: voffset per lane, the row
        // step 2 j in soffset; r % 32 = (16 (w % 2) + h) | 2 j.
        int y = (lane & 31) ^ (16 * (lw & 1) + hh);
        int32_t voff = cok ? ((16 * lw + hh) * p.ldc + ccol) * 2 : kOOB;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          asm volatile("" : "+v"(y), "+v"(voff));             // recomputed per store, not held eight times
          if (64 * rnd + 16 * lw + 2 * j < nrows) {
            const int r = 16 * lw + 2 * j + hh;
            const u32x4 v = *reinterpret_cast<const u32x4*>(stg + r * (WBQ * 2) + 16 * (y ^ (2 * j)));
            __builtin_amdgcn_raw_buffer_store_b128(v, out, voff, (64 * rnd + 2 * j) * p.ldc * 2, 0);
          }
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = f32x16{};
  };

  int sg = 0;
  for (int i = 0; i < mine; ++i) {
    for (int kt = 0; kt < nk; kt += kChunkSlabs) {
      static_for<kChunkSlabs>([&](auto ji) {
        constexpr int J = decltype(ji)::value;
        slab(ji, kt + J, sg + J);
      });
      sg += kChunkSlabs;
    }
    store_tile(cur, lds + kWBase + kWTile * (sg % 3));
    cur = nxt;
    nxt = tile_at(i + 2);
  }
  // No direct load may still be writing LDS when the workgroup ends.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

// Tiles of the groups listed by p (p.fuse_side == 2: the groups of at most
// p.fuse_rows rows); p.Q describes the bf16 weight [G][N][K].
hipError_t dx_wquant(const Params& prm, hipStream_t s) {
  if (prm.ntiles <= 0) return hipSuccess;
  // Persistent: one workgroup per compute unit (a multiple of the 8 XCDs),
  // fewer when the listed tiles (at most prm.ntiles) are fewer.
  int wg = compute_units() / 8 * 8;
  wg = wg < 8 ? 8 : wg;
  const int cap = (prm.ntiles + 7) / 8 * 8;
  fp8_mfma_wquant_kernel<><<<dim3(wg < cap ? wg : cap), dim3(NT8), 0, s>>>(prm);
  return hipGetLastError();
}

}  // namespace gk
}  // namespace lp
