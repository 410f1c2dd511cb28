"""lp_dequant against the oracle, bit for bit (GPU)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_bits_equal, bits_host, qtensor, quantize
from oracle import formats as F

pytestmark = pytest.mark.gpu


def _run(lp, fmt, codes, scales, ts=None, axis=-1, shape=None):
    q = qtensor(lp, fmt, codes, scales, ts, shape, axis)
    out = lp.lp_dequant(q)
    torch.cuda.synchronize()
    return bits_host(out)


def test_mxfp8_every_code_every_scale(lp):
    """All 256 E4M3 codes x all 256 E8M0 scale bytes, scales along cols."""
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))          # row r, col c -> code c
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, 1)  # row r -> scale r
    got = _run(lp, "mxfp8", codes, scales, shape=(1, 256, 256))
    assert_bits_equal(got, F.dequant("mxfp8", codes, scales, axis=-1), "mxfp8 axis -1")


def test_mxfp8_rows_every_code_every_scale(lp):
    """Scales along rows: 32-row block b uses scale byte b for every column."""
    codes = np.tile(np.arange(256, dtype=np.uint8), (32 * 256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 256, 1)
    got = _run(lp, "mxfp8", codes, scales, axis=-2, shape=(1, 32 * 256, 256))
    assert_bits_equal(got, F.dequant("mxfp8", codes, scales, axis=-2), "mxfp8 axis -2")


def test_mxfp4_every_byte_every_scale(lp):
    """All 256 packed bytes (every nibble pair) x all 256 E8M0 scale bytes."""
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))          # 512 elements per row
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 16, 1)
    got = _run(lp, "mxfp4", codes, scales, shape=(1, 256, 512))
    assert_bits_equal(got, F.dequant("mxfp4", codes, scales), "mxfp4")


@pytest.mark.parametrize("ts", [1.0, 0.0173, 2.0 ** -30, 3.0e5, 6.5e30, float("inf"), float("nan")])
def test_nvfp4_every_byte_every_block_scale(lp, ts):
    """All packed bytes x all 256 E4M3 block-scale bytes (NaN ones included)
    x a range of fp32 tensor scales."""
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 32, 1)
    got = _run(lp, "nvfp4", codes, scales, ts=ts, shape=(1, 256, 512))
    assert_bits_equal(got, F.dequant("nvfp4", codes, scales, np.float32(ts)), f"nvfp4 ts={ts}")


def test_fp8_b128_every_code_special_scales(lp):
    """All 256 codes in every 128x128 block, block scales covering zero,
    negative, subnormal, tiny, huge, infinite and NaN values."""
    svals = np.array([1.0, 0.0, -1.5, 1e-40, 3e-39, 1e-30, 3.7, 6e4, 1e30, 3e38, np.inf, np.nan,
                      0.00173, -0.0, 2.0 ** -127, 448.0], dtype=np.float32)
    grid = svals.reshape(8, 2)
    codes = np.tile(np.arange(256, dtype=np.uint8), (128 * 8, 1))
    got = _run(lp, "fp8_b128", codes, grid, shape=(1, 1024, 256))
    assert_bits_equal(got, F.dequant("fp8_b128", codes, grid), "fp8_b128")


def test_fp8_b128_partial_blocks_batched(lp):
    """Partial 128-blocks at both edges, two batches with their own grids."""
    g = W.rng(11, "w")
    b, R, C = 2, 300, 208
    codes = g.integers(0, 256, size=(b, R, C), dtype=np.uint8)
    grid = (g.random((b, 3, 2), dtype=np.float32) * 4 + 0.25).astype(np.float32)
    got = _run(lp, "fp8_b128", codes, grid, shape=(b, R, C))
    assert_bits_equal(got, F.dequant("fp8_b128", codes, grid), "fp8_b128 partial")


@pytest.mark.parametrize("name,tensor", [("fp8_frozen", "w"), ("nvfp4_linear", "x"), ("nvfp4_linear", "w"),
                                         ("mxfp4_grouped", "x"), ("mxfp4_grouped", "w")])
def test_workload_operands_full_size(lp, name, tensor):
    """The saved operands of the workloads, at full size, every element."""
    w = W.WORKLOADS[name]
    shape = (w.M, w.K) if tensor == "x" else ((w.groups, w.N, w.K) if w.grouped else (w.N, w.K))
    sigma = w.x_sigma if tensor == "x" else w.w_sigma
    vals = W.normal_f32(w.number, tensor, shape, sigma)
    if w.outliers:
        vals = W.with_outliers(vals, w.number, tensor)
    q, ref = quantize(lp, w.fmt, vals)
    out = lp.lp_dequant(q)
    torch.cuda.synchronize()
    assert_bits_equal(bits_host(out), ref, f"{name}.{tensor}")


def test_empty_is_noop(lp):
    q = lp.QTensor("mxfp4", torch.empty((0, 16), dtype=torch.uint8, device="cuda"),
                   torch.empty((0, 1), dtype=torch.uint8, device="cuda"), shape=(1, 0, 32))
    out = lp.lp_dequant(q)
    assert out.shape == (1, 0, 32)


@pytest.mark.parametrize("fmt,shape,axis", [
    ("nvfp4", (1, 5, 16), -1),          # 80 elements: not a whole 32-element code chunk
    ("nvfp4", (3, 37, 48), -1),         # ragged units of the last workgroup, batched
    ("mxfp4", (1, 1027, 32), -1),
    ("mxfp8", (2, 33, 96), -1),
    ("mxfp8", (2, 64, 48), -2),
    ("fp8_b128", (3, 129, 272), -1),
])
def test_ragged_sizes(lp, fmt, shape, axis):
    """Element counts that leave the last workgroup partly empty and rows
    as short as one scale block."""
    vals = W.rng(12, "x").standard_normal(shape, dtype=np.float32)
    q, ref = quantize(lp, fmt, vals, axis)
    out = lp.lp_dequant(q)
    torch.cuda.synchronize()
    assert_bits_equal(bits_host(out), ref, f"{fmt} {shape}")


def test_binding_rejects_short_and_strided_buffers(lp):
    """A device buffer too small for the call, or a strided view, is refused
    by the binding before any kernel runs (the C calls take bare pointers)."""
    codes = torch.zeros((1, 64, 64), dtype=torch.uint8, device="cuda")
    scales = torch.full((1, 64, 2), 127, dtype=torch.uint8, device="cuda")
    q = lp.QTensor("mxfp8", codes, scales)
    with pytest.raises(ValueError, match="needs"):
        lp.lp_dequant(q, torch.empty((64, 63), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError, match="needs"):
        lp.lp_dequant(lp.QTensor("mxfp8", codes, scales[:, :32], shape=(1, 64, 64)))
    with pytest.raises(ValueError, match="contiguous"):
        lp.lp_dequant(q, torch.empty((64, 128), dtype=torch.bfloat16, device="cuda")[:, ::2])
    src = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="bfloat16"):
        lp.lp_tensor_amax(src)
    out = lp.lp_dequant(q)                                   # and the well-formed call still runs
    torch.cuda.synchronize()
    assert out.shape == (1, 64, 64) and not out.float().abs().any()
