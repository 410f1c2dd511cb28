"""Helpers of the GPU parity tests: move oracle-made inputs to the device,
build the library's tensor descriptors, and compare results."""
from __future__ import annotations

import numpy as np
import torch

import workloads as W
from oracle import formats as F

REL_FRO = 5e-3      # relative Frobenius error bound of every contraction
MAX_ABS = 1e-2      # max |error| bound, as a fraction of max |reference|


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return dev(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def qtensor(lp, fmt, codes, scales=None, ts=None, shape=None, axis=-1):
    """Library descriptor of oracle-made codes / scales (numpy)."""
    c = dev(codes) if fmt != "bf16" else bf16_dev(codes)
    s = dev(scales) if scales is not None else None
    t = torch.tensor([ts], dtype=torch.float32, device="cuda") if ts is not None else None
    return lp.QTensor(fmt, c, s, t, shape=shape, axis=axis)


def quantize(lp, fmt: str, values_f32: np.ndarray, axis: int = -1):
    """Quantize fp32 values [b,R,C] or [R,C] with the oracle's generators.
    Returns (descriptor on the GPU, the oracle's dequantized bf16 bits [b,R,C])."""
    v = np.asarray(values_f32, dtype=np.float32)
    v3 = v.reshape((1,) + v.shape) if v.ndim == 2 else v
    shape = v3.shape
    ts = None
    if fmt == "bf16":
        codes = W.bf16_bits(v3)
        scales = None
    elif fmt == "mxfp4":
        codes, scales = F.quant_mxfp4_f32(v3)
    elif fmt == "nvfp4":
        codes, scales, ts = F.quant_nvfp4(v3)
        ts = float(ts)
    elif fmt == "fp8_b128":
        codes, scales = F.quant_fp8_b128(v3)
    elif fmt == "mxfp8":
        codes, scales = F.mx_quant(W.bf16_bits(v3), axis, "e4m3")
    else:
        raise ValueError(fmt)
    deq = F.dequant(fmt, codes, scales, ts, axis)
    return qtensor(lp, fmt, codes, scales, ts, shape, axis), deq


def errors(got: torch.Tensor, ref: np.ndarray):
    g = got.float().cpu().numpy().astype(np.float64).reshape(ref.shape)
    rel = np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300)
    mx = np.abs(g - ref).max() / max(np.abs(ref).max(), 1e-300)
    return rel, mx


def assert_close(got: torch.Tensor, ref: np.ndarray, what: str = ""):
    rel, mx = errors(got, ref)
    assert rel <= REL_FRO and mx <= MAX_ABS, f"{what}: rel Frobenius {rel:.3e}, max abs ratio {mx:.3e}"


def assert_bits_equal(got: np.ndarray, ref: np.ndarray, what: str = ""):
    got = np.asarray(got).reshape(ref.shape)
    bad = got != ref
    if bad.any():
        idx = np.argwhere(bad)[:5]
        pairs = [(tuple(i), hex(int(got[tuple(i)])), hex(int(ref[tuple(i)]))) for i in idx]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} differ, e.g. {pairs}")
