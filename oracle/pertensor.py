"""CPU oracle: per-tensor scaled FP8 backward (E4M3 / E5M2 codes, one fp32
scale per tensor).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the library never does.

Source: "AstrAI fp8.py" (astrai/extension/fp8.py):
* FP8_MAX: E4M3 448, E5M2 57344.  Hybrid format: E4M3 forward, E5M2 for the
  backward pass.
* Every operand's scale is a quantization step derived from amax:
  scale = (amax / FP8_MAX[fmt]) / 2^margin, clamped to at least 1e-12.
  Delayed scaling takes the max over an amax history ring (the amax recorded
  by earlier steps); dynamic scaling takes the current amax of the tensor.
  The ring records an amax at idx, then idx = (idx + 1) % len, and a first
  use fills the whole ring with the tensor's amax.
* _LinearFp8.backward quantizes the gradient once and shares it between the
  dX and dW products, and returns the gradient's amax for the ring.

The native backward kernels are not shown on the page, so three points are
readings (listed with their pins in the design notes):
* Quantization: t = x / scale in fp32 (IEEE division, round to nearest
  even), then the nearest FP8 value, ties to even.  Finite magnitudes and
  infinities beyond the format's maximum saturate to it, with the sign kept;
  NaN becomes a NaN code (0x7F with the sign bit) in both formats.
* A dequantized element is code * scale.  A product of two per-tensor
  operands is scale_a * scale_b * sum(code_a * code_b), with no rounding of
  the dequantized values in between, since the products are FP8 GEMMs.
* amax is max |x| over the tensor, NaN if any element is NaN (torch's
  abs().amax()).
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_TABLE, bf16_bits_to_f64, f32_to_bf16_bits, round_f32

FP8_MAX = {"e4m3": 448.0, "e5m2": 57344.0}
SCALE_FLOOR = np.float32(1e-12)


def e5m2_value(code: int) -> float:
    """E5M2: 1 sign, 5 exponent (bias 15), 2 mantissa bits; exponent 0 is
    subnormal (m / 4 * 2^-14); exponent 31 is infinity (m == 0) or NaN."""
    s, e, m = (code >> 7) & 1, (code >> 2) & 31, code & 3
    if e == 31:
        mag = float("inf") if m == 0 else float("nan")
    elif e == 0:
        mag = m / 4.0 * 2.0 ** -14
    else:
        mag = 2.0 ** (e - 15) * (1.0 + m / 4.0)
    return -mag if s else mag


E5M2_TABLE = np.array([e5m2_value(c) for c in range(256)], dtype=np.float64)
TABLES = {"e4m3": E4M3_TABLE, "e5m2": E5M2_TABLE}


def _finite_grid(table: np.ndarray):
    """Non-negative finite values of a format (sign bit clear) with their
    codes, ascending."""
    codes = np.arange(128)
    vals = table[codes]
    keep = np.isfinite(vals)
    order = np.argsort(vals[keep], kind="stable")
    return vals[keep][order], codes[keep][order]


_GRIDS = {k: _finite_grid(t) for k, t in TABLES.items()}


def round_to_fp8(t: np.ndarray, elem: str) -> np.ndarray:
    """Nearest FP8 code to each real t, ties to the even code; magnitudes
    beyond the largest finite value (infinities included) saturate to it; the
    sign bit follows t; NaN gives 0x7F with t's sign bit."""
    vals, codes = _GRIDS[elem]
    t = np.asarray(t, dtype=np.float64)
    nan = np.isnan(t)
    a = np.where(nan, 0.0, np.abs(t))
    lo = np.clip(np.searchsorted(vals, a, side="right") - 1, 0, len(vals) - 1)
    hi = np.minimum(lo + 1, len(vals) - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (codes[hi] % 2 == 0) & (hi != lo))
    out = codes[np.where(pick_hi, hi, lo)].astype(np.uint8)
    out = np.where(nan, 0x7F, out).astype(np.uint8)
    return np.where(np.signbit(t), out | 0x80, out).astype(np.uint8)


def amax(bits: np.ndarray) -> np.float32:
    """max |x| of bf16 values (bit patterns), NaN if any is NaN."""
    v = np.abs(bf16_bits_to_f64(bits))
    return np.float32(np.nan) if np.isnan(v).any() else np.float32(v.max() if v.size else 0.0)


def scale_from_history(hist, elem: str, margin: int = 0) -> np.float32:
    """scale = (max(hist) / FP8_MAX) / 2^margin, at least 1e-12, each step in
    fp32 (the recipe's tensor arithmetic).  Dynamic scaling is a history of
    one entry, the current amax."""
    peak = np.float32(np.max(np.asarray(hist, dtype=np.float32)))
    s = np.float32(peak / np.float32(FP8_MAX[elem]))
    s = np.float32(s / np.float32(2.0 ** margin))
    return np.float32(max(s, SCALE_FLOOR)) if not np.isnan(s) else s


def record(hist: np.ndarray, idx: int, value) -> int:
    """Ring update: hist[idx] = value, returns the next index."""
    hist[idx] = np.float32(value)
    return (idx + 1) % len(hist)


def quantize(bits: np.ndarray, elem: str, scale) -> np.ndarray:
    """bf16 values -> FP8 codes: t = fp32(x / scale), then the nearest code."""
    x = bf16_bits_to_f64(bits).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        t = x / np.float32(scale)                    # fp32 / fp32, IEEE round to nearest even
    return round_to_fp8(t.astype(np.float64), elem)


def values(codes: np.ndarray, elem: str) -> np.ndarray:
    """Code values (fp64, exact)."""
    return TABLES[elem][np.asarray(codes, dtype=np.uint8)]


def dequant(codes: np.ndarray, elem: str, scale) -> np.ndarray:
    """bf16 bits of RNE_bf16(RNE_fp32(code * scale)); a NaN code gives 0x7FC0
    with the code's sign bit."""
    c = np.asarray(codes, dtype=np.uint8)
    with np.errstate(invalid="ignore", over="ignore"):
        f = round_f32(values(c, elem) * np.float64(np.float32(scale)))
    return f32_to_bf16_bits(f, nan_sign=(c >> 7) & 1)


def linear_dx(g_codes, g_elem, g_scale, w_codes, w_elem, w_scale) -> np.ndarray:
    """grad_X = (g_scale * w_scale) * (g_codes @ w_codes), fp64."""
    return (values(g_codes, g_elem) @ values(w_codes, w_elem)) * (float(np.float32(g_scale)) * float(np.float32(w_scale)))


def linear_dw(g_codes, g_elem, g_scale, x_codes, x_elem, x_scale) -> np.ndarray:
    """grad_W = (g_scale * x_scale) * (g_codes^T @ x_codes), fp64."""
    return (values(g_codes, g_elem).T @ values(x_codes, x_elem)) * (float(np.float32(g_scale)) * float(np.float32(x_scale)))
