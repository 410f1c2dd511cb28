"""CPU oracle: block-scaled formats, dequantization and MX re-quantization.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the library never does.

Everything here is written from the definitions, element by element, in
fp64 (exact for every product below), with two explicit IEEE
round-to-nearest-even steps: to fp32 (numpy's float64 -> float32 cast) and
then to bf16 (an integer rounding on the fp32 bit pattern).

Sources:
* "Add Autograd Backward Support for FP4 GEMM Custom Ops", Implementation
  Method: the backward dequantizes the saved packed FP4 operands (E2M1, eight
  magnitudes) to BF16 before the matmuls.
* "Train adapters on top of FP8 weights", `_dequantize_fp8_weight`: an
  E4M3 weight times its per-128x128-block fp32 inverse scale, the scale grid
  expanded over each block and cut at the tensor edge.
* "perf: defer mxfp8 backward quantization", `MXFP8GMMFunction.op_dx` and
  `MXFP8MatMul.backward`: dynamic MX quantization along an axis, E8M0 scale
  (`float8_e8m0fnu`) per group of 32 (`group_sizes=[1, 1, 32]`).
* "AstrAI fp8.py", `FP8_MAX`: the E4M3 maximum is 448.

Readings taken where the source documents are silent (each with the test
that pins it under tests/):
* E2M1, E4M3 (OCP "FN": no infinities, S.1111.111 is NaN) and E8M0
  (2^(b-127), 0xFF = NaN) follow the OCP MX v1.0 element definitions.
* Packed E2M1: element 2j in the low nibble, 2j+1 in the high nibble.
  Parity unpinned by the source documents (no packed example is printed).
* Scales are plain row-major, unswizzled.
* Every decode is RNE_bf16(RNE_fp32(code_value * S)) with S an fp32 block
  multiplier; for NVFP4, S = RNE_fp32(E4M3(s_b) * tensor_scale), the tensor
  scale being a decode multiplier.  Parity of the NVFP4 tensor-scale reading
  is unpinned by the source documents.
* A NaN result is the bf16 quiet NaN 0x7FC0 carrying the code's sign bit.
* MX scale: e = floor(log2(amax)) - emax_elem (8 for E4M3, 2 for E2M1),
  clamped to [-127, 127]; elements rounded to nearest, ties to even, and
  saturated to +-448 / +-6.  A block with a NaN or infinity gets scale 0xFF
  and NaN codes (E4M3 0x7F with the element's sign; E2M1 has no NaN, its
  codes are 0); an all-zero block gets scale 0x00 and signed-zero codes.
"""
from __future__ import annotations

import numpy as np

FMT_BF16 = "bf16"
FMT_MXFP4 = "mxfp4"
FMT_NVFP4 = "nvfp4"
FMT_FP8_B128 = "fp8_b128"
FMT_MXFP8 = "mxfp8"

E4M3_MAX = 448.0   # "AstrAI fp8.py", FP8_MAX
E2M1_MAX = 6.0
MX_BLOCK = 32      # "perf: defer mxfp8 backward quantization", group_sizes [1, 1, 32]
NV_BLOCK = 16
FP8_BLOCK = 128    # "Train adapters on top of FP8 weights", block_size (128, 128)
# Exponent of the largest power of two not above each element format's maximum
# (448 = 1.75 * 2^8, 6 = 1.5 * 2^2): the MX scale puts a block's amax there.
ELEM_EMAX = {"e4m3": 8, "e2m1": 2}


# ---------------------------------------------------------------- element codes

def e2m1_value(code: int) -> float:
    """E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is
    subnormal (0 or 0.5)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def e4m3_value(code: int) -> float:
    """E4M3 (FN): 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
    subnormal; only S.1111.111 is NaN, there are no infinities."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    mag = m * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


def e8m0_value(code: int) -> float:
    """E8M0: a bare biased exponent, 2^(code-127); 0xFF is NaN."""
    return float("nan") if code == 0xFF else 2.0 ** (code - 127)


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


# ---------------------------------------------------------------- rounding

def round_f32(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32, IEEE round to nearest even (subnormals kept, overflow
    to infinity)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(f: np.ndarray, nan_sign: np.ndarray | None = None) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even on the 16 dropped bits.

    NaN becomes 0x7FC0 with the sign bit taken from `nan_sign` (an array of
    0/1) when given, else from the NaN's own sign bit.
    """
    f = np.ascontiguousarray(f, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(f)
    if nan.any():
        sign = (u >> 31).astype(np.uint32) if nan_sign is None else np.broadcast_to(
            np.asarray(nan_sign, dtype=np.uint32), f.shape)
        r = np.where(nan, 0x7FC0 | (sign << 15), r)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- unpacking

def unpack_e2m1(packed: np.ndarray) -> np.ndarray:
    """[..., C/2] bytes -> [..., C] 4-bit codes; even column = low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def pack_e2m1(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] & 0x0F) | ((c[..., 1::2] & 0x0F) << 4)


def _as3d(a: np.ndarray) -> np.ndarray:
    return a.reshape((1,) + a.shape) if a.ndim == 2 else a


def expand_scales(scales: np.ndarray, rows: int, cols: int, block_r: int,
                  block_c: int) -> np.ndarray:
    """Repeat a block grid [b, ceil(R/br), ceil(C/bc)] over the elements and cut
    it at the tensor edge (the slicing of `_dequantize_fp8_weight`)."""
    s = np.repeat(np.repeat(scales, block_r, axis=-2)[..., :rows, :], block_c, axis=-1)
    return s[..., :cols]


# ---------------------------------------------------------------- dequant

def _decode(code_values: np.ndarray, S: np.ndarray, code_sign: np.ndarray) -> np.ndarray:
    """RNE_bf16(RNE_fp32(code_value * S)); the fp64 product is exact."""
    with np.errstate(invalid="ignore", over="ignore"):
        prod = code_values * S
    return f32_to_bf16_bits(round_f32(prod), nan_sign=code_sign)


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 [b,R,C/2] packed codes, E8M0 scales [b,R,C/32] along the columns."""
    c = unpack_e2m1(_as3d(codes))
    R, C = c.shape[-2:]
    S = expand_scales(E8M0_TABLE[_as3d(scales)], R, C, 1, MX_BLOCK)
    return _decode(E2M1_TABLE[c], S, c >> 3)


def dequant_nvfp4(codes: np.ndarray, scales: np.ndarray, tensor_scale: float) -> np.ndarray:
    """NVFP4 [b,R,C/2] packed codes, E4M3 scales [b,R,C/16], fp32 tensor scale."""
    c = unpack_e2m1(_as3d(codes))
    R, C = c.shape[-2:]
    with np.errstate(invalid="ignore", over="ignore"):
        block = round_f32(E4M3_TABLE[_as3d(scales)] * np.float64(np.float32(tensor_scale)))
    S = expand_scales(block.astype(np.float64), R, C, 1, NV_BLOCK)
    return _decode(E2M1_TABLE[c], S, c >> 3)


def dequant_fp8_b128(codes: np.ndarray, scale_inv: np.ndarray) -> np.ndarray:
    """E4M3 [b,R,C] codes, fp32 inverse scales [b, ceil(R/128), ceil(C/128)]."""
    c = _as3d(codes).astype(np.uint8)
    R, C = c.shape[-2:]
    S = expand_scales(_as3d(scale_inv).astype(np.float32).astype(np.float64), R, C,
                      FP8_BLOCK, FP8_BLOCK)
    return _decode(E4M3_TABLE[c], S, c >> 7)


def dequant_mxfp8(codes: np.ndarray, scales: np.ndarray, axis: int) -> np.ndarray:
    """MXFP8 (E4M3 elements) [b,R,C]; E8M0 scales [b,R,C/32] (axis -1) or
    [b,R/32,C] (axis -2)."""
    c = _as3d(codes).astype(np.uint8)
    R, C = c.shape[-2:]
    sv = E8M0_TABLE[_as3d(scales)]
    S = expand_scales(sv, R, C, 1, MX_BLOCK) if axis == -1 else expand_scales(sv, R, C, MX_BLOCK, 1)
    return _decode(E4M3_TABLE[c], S, c >> 7)


def _dequant_one(fmt, codes, scales, tensor_scale, axis):
    if fmt == FMT_MXFP4:
        return dequant_mxfp4(codes, scales)
    if fmt == FMT_NVFP4:
        return dequant_nvfp4(codes, scales, tensor_scale)
    if fmt == FMT_FP8_B128:
        return dequant_fp8_b128(codes, scales)
    if fmt == FMT_MXFP8:
        return dequant_mxfp8(codes, scales, axis)
    raise ValueError(fmt)


def dequant(fmt: str, codes, scales=None, tensor_scale=None, axis: int = -1,
            chunk_rows: int = 512) -> np.ndarray:
    """Dispatch on the format; returns bf16 bits [b,R,C].  Large tensors are
    processed in slabs of about `chunk_rows` rows, rounded up to a whole
    number of scale-block rows so that every slab starts on a block
    boundary; the slabs change nothing in the result."""
    if fmt == FMT_BF16:
        return _as3d(np.asarray(codes, dtype=np.uint16))
    codes = _as3d(np.asarray(codes))
    scales = _as3d(np.asarray(scales))
    b, R = codes.shape[:2]
    C = codes.shape[2] * (2 if fmt in (FMT_MXFP4, FMT_NVFP4) else 1)
    out = np.empty((b, R, C), dtype=np.uint16)
    srow = {FMT_FP8_B128: FP8_BLOCK, FMT_MXFP8: MX_BLOCK if axis == -2 else 1}.get(fmt, 1)
    step = -(-max(1, chunk_rows) // srow) * srow        # slabs start on a scale-block boundary
    for bi in range(b):
        for r0 in range(0, R, step):
            r1 = min(R, r0 + step)
            out[bi, r0:r1] = _dequant_one(fmt, codes[bi:bi + 1, r0:r1],
                                          scales[bi:bi + 1, _scale_rows(r0, r1, srow)],
                                          tensor_scale, axis)[0]
    return out


def _scale_rows(r0: int, r1: int, srow: int) -> slice:
    """Rows of the scale grid that cover tensor rows [r0, r1) when one scale
    row spans `srow` tensor rows (r0 a multiple of srow)."""
    return slice(r0 // srow, -(-r1 // srow))


# ---------------------------------------------------------------- rounding onto a grid

def _grid(table: np.ndarray, ncodes: int):
    """Non-negative finite values of a format with their codes, ascending."""
    codes = np.arange(ncodes // 2)                 # sign bit clear
    vals = table[codes]
    keep = np.isfinite(vals)
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], codes[keep][order]


_E4M3_GRID = _grid(E4M3_TABLE, 256)
_E2M1_GRID = _grid(E2M1_TABLE, 16)


def round_to_grid(t: np.ndarray, elem: str) -> np.ndarray:
    """Nearest element code to each real t (fp64), ties to the even code,
    magnitudes above the largest value saturated to it; the sign bit is
    copied from t (so -0 and small negatives give a negative-zero code)."""
    vals, codes = _E4M3_GRID if elem == "e4m3" else _E2M1_GRID
    sign_bit = 0x80 if elem == "e4m3" else 0x8
    a = np.abs(t)
    lo = np.searchsorted(vals, a, side="right") - 1          # vals[lo] <= a
    lo = np.clip(lo, 0, len(vals) - 1)
    hi = np.minimum(lo + 1, len(vals) - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0) & (hi != lo))
    idx = np.where(pick_hi, hi, lo)
    out = codes[idx].astype(np.uint8)
    neg = np.signbit(t)
    return np.where(neg, out | sign_bit, out).astype(np.uint8)


# ---------------------------------------------------------------- MX quantization

def _mx_quant_blocks(blocks: np.ndarray, elem: str):
    """Quantize rows of 32 values (fp64 [n, 32]) -> (codes [n, 32], scales [n])."""
    emax = ELEM_EMAX[elem]
    sign_bit = 0x80 if elem == "e4m3" else 0x8
    bad = ~np.isfinite(blocks).all(axis=-1)                 # a NaN or infinity
    with np.errstate(invalid="ignore"):
        amax = np.where(bad, 0.0, np.abs(blocks).max(axis=-1))
    zero = (amax == 0) & ~bad
    _, ex = np.frexp(np.where(zero | bad, 1.0, amax))      # amax = m * 2^ex, m in [0.5, 1)
    e = np.clip(ex.astype(np.int64) - 1 - emax, -127, 127)  # floor(log2 amax) - emax
    e = np.where(zero | bad, -127, e)
    scale = np.where(bad, 0xFF, e + 127).astype(np.uint8)

    finite = np.where(bad[:, None], 0.0, blocks)
    t = finite * np.ldexp(1.0, (-e).astype(np.int32))[:, None]   # exact power-of-two scaling
    codes = round_to_grid(t, elem)
    codes = np.where(np.signbit(blocks), codes | sign_bit, codes)
    if elem == "e4m3":
        nan_code = np.where(np.signbit(blocks), 0xFF, 0x7F).astype(np.uint8)
        codes = np.where(bad[:, None], nan_code, codes)
    else:
        codes = np.where(bad[:, None], 0, codes)
    return codes.astype(np.uint8), scale


def _block_chunks(n: int, size: int) -> list[tuple[int, int]]:
    """[start, stop) ranges of at most `size` blocks covering blocks 0..n-1."""
    size = max(1, size)
    return [(i, min(n, i + size)) for i in range(0, n, size)]


def mx_quant(bits: np.ndarray, axis: int, elem: str, chunk_blocks: int = 1 << 16):
    """Dynamic MX quantization of bf16 bits [b,R,C] along `axis` (-1: blocks of
    32 run along the columns, -2: along the rows).

    Returns (codes, scales): E4M3 codes [b,R,C] or packed E2M1 [b,R,C/2], and
    E8M0 scales [b,R,C/32] (axis -1) or [b,R/32,C] (axis -2).
    """
    x = _as3d(np.asarray(bits, dtype=np.uint16))
    if axis == -2:
        x = np.swapaxes(x, -1, -2)
    b, R, C = x.shape
    flat = np.ascontiguousarray(x).reshape(-1, MX_BLOCK)
    codes = np.zeros(flat.shape, dtype=np.uint8)
    scale = np.zeros(flat.shape[0], dtype=np.uint8)
    for i, j in _block_chunks(flat.shape[0], chunk_blocks):
        c, s = _mx_quant_blocks(bf16_bits_to_f64(flat[i:j]), elem)
        codes[i:j] = c
        scale[i:j] = s
    codes = codes.reshape(b, R, C)
    scale = scale.reshape(b, R, C // MX_BLOCK)
    if axis == -2:
        codes = np.ascontiguousarray(np.swapaxes(codes, -1, -2))
        scale = np.ascontiguousarray(np.swapaxes(scale, -1, -2))
    if elem == "e2m1":
        codes = pack_e2m1(codes)
    return codes, scale


# ---------------------------------------------------------------- input generators

def quant_fp8_b128(w: np.ndarray):
    """Generator of FP8 block inputs: per 128x128 block s = RNE_fp32(amax / 448)
    (the amax/FP8_MAX recipe of "AstrAI fp8.py" with margin 0), codes =
    E4M3(RNE_fp32(w / s)).  Returns (codes [b,R,C], scale_inv fp32 grid)."""
    w3 = _as3d(np.asarray(w, dtype=np.float32)).astype(np.float64)
    b, R, C = w3.shape
    gr, gc = -(-R // FP8_BLOCK), -(-C // FP8_BLOCK)
    pad = np.zeros((b, gr * FP8_BLOCK, gc * FP8_BLOCK))
    pad[:, :R, :C] = np.abs(w3)
    amax = pad.reshape(b, gr, FP8_BLOCK, gc, FP8_BLOCK).max(axis=(2, 4))
    s = round_f32(amax / E4M3_MAX)
    s = np.where(s == 0, np.float32(1.0), s).astype(np.float32)
    S = expand_scales(s.astype(np.float64), R, C, FP8_BLOCK, FP8_BLOCK)
    t = round_f32(w3 / S).astype(np.float64)
    return round_to_grid(t, "e4m3"), s


def quant_nvfp4(x: np.ndarray):
    """Generator of NVFP4 inputs (two-level recipe): s_t = amax / (6 * 448);
    per 16 along the columns s_b = E4M3(amax_b / 6 / s_t); codes =
    E2M1(x / (E4M3(s_b) * s_t)); a zero block scale gives zero codes.
    Returns (packed codes, E4M3 scale codes [b,R,C/16], fp32 tensor scale)."""
    x3 = _as3d(np.asarray(x, dtype=np.float32)).astype(np.float64)
    b, R, C = x3.shape
    st = float(np.float32(np.abs(x3).max() / (E2M1_MAX * E4M3_MAX)))
    if st == 0.0:
        st = 1.0
    blocks = x3.reshape(b, R, C // NV_BLOCK, NV_BLOCK)
    sb = round_to_grid(np.abs(blocks).max(axis=-1) / E2M1_MAX / st, "e4m3")
    Sb = round_f32(E4M3_TABLE[sb] * st).astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.where(Sb[..., None] > 0, blocks / Sb[..., None], 0.0)
    codes = round_to_grid(t, "e2m1").reshape(b, R, C)
    return pack_e2m1(codes), sb, np.float32(st)


def quant_mxfp4_f32(x: np.ndarray):
    """Generator of MXFP4 inputs: round the fp32 draws to bf16 (torch's cast,
    as the library's quantizer takes bf16), then MX-quantize along the columns."""
    from workloads import bf16_bits
    return mx_quant(bf16_bits(np.asarray(x, dtype=np.float32)), -1, "e2m1")
