"""CPU oracle: the backward contractions, in fp64.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module; the library never does.

* "Add Autograd Backward Support for FP4 GEMM Custom Ops", Implementation
  Method: with the saved operands dequantized to BF16,
  grad_X = grad_output @ W_bf16 and grad_W = grad_output.T @ X_bf16.
* "Train adapters on top of FP8 weights", `FP8LinearFunction.backward`: a
  frozen weight returns only grad_X; `FP8GroupedMatmulFunction.backward`:
  grad_output rows of group g (cumulative int32 end offsets, the first group
  starting at 0) multiply that group's (output_dim, input_dim) weight; the
  EP-sentinel comment in `fp8_grouped_mm_experts_forward`: rows past the last
  offset are not written.

The forward that the backward pairs with ("Add Autograd Backward Support for
FP4 GEMM Custom Ops": FP4 inputs times FP4 weights into BF16, dense and
grouped; "perf: defer mxfp8 backward quantization", MXFP8MatMul.forward) is
y = x @ W^T with the same decoded operands.

The inputs are bf16 values (bit patterns) that the format oracle produced;
every bf16 x bf16 product is exact in fp64 and the sums are fp64 (numpy's
float64 matmul).  Grouped weight gradients of an empty group are the empty
sum, zero.
"""
from __future__ import annotations

import numpy as np

from .formats import FMT_FP8_B128, FMT_NVFP4, bf16_bits_to_f64, dequant


def _f64(bits) -> np.ndarray:
    return bf16_bits_to_f64(bits)


def linear_dx(grad_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """grad_X[m,k] = sum_n grad[m,n] * W[n,k]; grad [M,N], W [N,K]."""
    return _f64(grad_bits) @ _f64(w_bits)


def linear_dw(grad_bits: np.ndarray, x_bits: np.ndarray) -> np.ndarray:
    """grad_W[n,k] = sum_m grad[m,n] * X[m,k]; grad [M,N], X [M,K]."""
    return _f64(grad_bits).T @ _f64(x_bits)


def group_bounds(offsets) -> list[tuple[int, int]]:
    """(start, end) rows of each group from cumulative end offsets."""
    ends = [int(o) for o in np.asarray(offsets).reshape(-1)]
    starts = [0] + ends[:-1]
    return list(zip(starts, ends))


def grouped_dx(grad_bits: np.ndarray, w_bits: np.ndarray, offsets) -> tuple[np.ndarray, int]:
    """Per group g: grad_X[rows of g] = grad[rows of g] @ W[g].

    Returns (dX [M,K] fp64, rows_written): rows at or past the last offset are
    left as NaN here, standing for "not written"."""
    G = _f64(grad_bits)
    W = _f64(w_bits)
    M, K = G.shape[0], W.shape[-1]
    out = np.full((M, K), np.nan)
    for g, (s, e) in enumerate(group_bounds(offsets)):
        if e > s:
            out[s:e] = G[s:e] @ W[g]
    return out, group_bounds(offsets)[-1][1] if len(offsets) else 0


def grouped_dw(grad_bits: np.ndarray, x_bits: np.ndarray, offsets) -> np.ndarray:
    """Per group g: grad_W[g] = grad[rows of g].T @ X[rows of g]; zero when the
    group is empty.  Returns [G, N, K] fp64."""
    G = _f64(grad_bits)
    X = _f64(x_bits)
    bounds = group_bounds(offsets)
    out = np.zeros((len(bounds), G.shape[1], X.shape[1]))
    for g, (s, e) in enumerate(bounds):
        if e > s:
            out[g] = G[s:e].T @ X[s:e]
    return out


def linear_fwd(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """y[m,n] = sum_k x[m,k] * W[n,k]; x [M,K], W [N,K]."""
    return _f64(x_bits) @ _f64(w_bits).T


def grouped_fwd(x_bits: np.ndarray, w_bits: np.ndarray, offsets) -> np.ndarray:
    """Per group g: y[rows of g] = x[rows of g] @ W[g]^T; rows at or past the
    last offset are NaN here ("not written")."""
    X = _f64(x_bits)
    W = _f64(w_bits)
    out = np.full((X.shape[0], W.shape[1]), np.nan)
    for g, (s, e) in enumerate(group_bounds(offsets)):
        if e > s:
            out[s:e] = X[s:e] @ W[g].T
    return out


def rows_dx(grad_bits: np.ndarray, w_bits: np.ndarray, rows) -> np.ndarray:
    """Selected rows of grad_X = grad @ W (for sampled checks at full size)."""
    return _f64(np.asarray(grad_bits)[rows]) @ _f64(w_bits)


def rows_dw(grad_bits: np.ndarray, x_bits: np.ndarray, n_rows) -> np.ndarray:
    """Selected rows n of grad_W = grad.T @ X."""
    return _f64(np.asarray(grad_bits)[:, n_rows]).T @ _f64(x_bits)


# ---------------------------------------------------------------- forwards of quantized layers
# The forward ops that the backward pages pair with take the same saved
# operands.  Neither page gives their arithmetic; the reading here is the
# one the backward states for its own products: decode each quantized
# operand to bf16 exactly as the backward does (formats.dequant), then
# contract in fp64.

def nvfp4_fwd(x_codes, x_scales, x_ts, w_codes, w_scales, w_ts, offsets=None) -> np.ndarray:
    """NVFP4 forward ("Add Autograd Backward Support for FP4 GEMM Custom Ops":
    the f4f4bf16 ops multiply FP4 inputs by FP4 weights into BF16, dense and
    grouped).  x [M][K] and w [G][N][K] (G = 1 for the dense op) are NVFP4:
    packed E2M1 codes, E4M3 scales per 16 along K, an fp32 tensor scale.
    Dense: y = dec(x) @ dec(w)^T; grouped (offsets given): per group as
    grouped_fwd, rows past the last offset NaN ("not written")."""
    xb = dequant(FMT_NVFP4, x_codes, x_scales, x_ts)[0]
    wb = dequant(FMT_NVFP4, w_codes, w_scales, w_ts)
    return linear_fwd(xb, wb[0]) if offsets is None else grouped_fwd(xb, wb, offsets)


def fp8_block_fwd(x_bits, w_codes, w_scale_inv, offsets=None) -> np.ndarray:
    """Block-FP8 forward ("Train adapters on top of FP8 weights":
    FP8LinearFunction.forward through fp8_linear, and
    FP8GroupedMatmulFunction.forward through the kernel's
    grouped_matmul(input, weight, weight_scale_inv, offsets, ...)): a bf16
    input times an E4M3 weight [G][N][K] with fp32 inverse scales per 128 x
    128 block.  The input stays bf16 (the page quantizes nothing else); the
    weight is decoded as `_dequantize_fp8_weight` does for the backward.
    Dense (offsets None, G = 1) or grouped as grouped_fwd."""
    wb = dequant(FMT_FP8_B128, w_codes, w_scale_inv)
    return linear_fwd(x_bits, wb[0]) if offsets is None else grouped_fwd(x_bits, wb, offsets)
