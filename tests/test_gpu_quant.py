"""lp_mx_quant against the oracle, bit for bit (GPU)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_bits_equal, bf16_dev
from oracle import formats as F

pytestmark = pytest.mark.gpu

ELEM = {"mxfp8": "e4m3", "mxfp4": "e2m1"}


def _gpu_quant(lp, bits3, axis, fmt):
    q = lp.lp_mx_quant(bf16_dev(bits3), axis, fmt)
    torch.cuda.synchronize()
    return q.codes.cpu().numpy(), q.scales.cpu().numpy()


def _check(lp, bits3, axis, fmt, what):
    codes, scales = _gpu_quant(lp, bits3, axis, fmt)
    rc, rs = F.mx_quant(bits3, axis, ELEM[fmt])
    assert_bits_equal(scales, rs, f"{what} scales")
    assert_bits_equal(codes, rc, f"{what} codes")


def _every_finite_bf16_in_blocks():
    """Every finite bf16 value once, shuffled into blocks of 32 (so each value
    meets many block maxima), plus structured blocks: one binade per block
    with the mantissa walking through it, to hit every rounding tie."""
    b = np.arange(1 << 16, dtype=np.uint32)
    finite = b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    g = W.rng(20, "x")
    g.shuffle(finite)
    n = len(finite) // 32 * 32
    blocks = [finite[:n].reshape(-1, 32)]
    for e in range(0, 255):
        for sign in (0, 0x8000):
            m = np.arange(128, dtype=np.uint16)
            vals = (sign | (e << 7) | m).astype(np.uint16)
            blocks.append(vals.reshape(4, 32))
    return np.concatenate(blocks).astype(np.uint16)


def _special_blocks():
    z = np.zeros((8, 32), np.uint16)
    z[1, :] = 0x8000                       # all -0
    z[2, 3] = 0x7FC0                       # NaN in a block
    z[3, 5] = 0x7F80                       # +inf
    z[4, 7] = 0xFF80                       # -inf
    z[4, 8] = 0xBF80                       # -1 beside it
    z[5, :] = 0x0001                       # smallest subnormal everywhere
    z[6, :] = np.arange(32) | 0x8000       # negative subnormals
    z[7, :] = 0x7F7F                       # largest finite everywhere
    return z


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("axis", [-1, -2])
def test_every_bf16_value(lp, fmt, axis):
    blocks = np.concatenate([_special_blocks(), _every_finite_bf16_in_blocks()])
    rows = blocks.shape[0] // 32 * 32
    blocks = blocks[:rows]
    if axis == -1:
        bits = blocks.reshape(1, -1, 256)[:, : (rows * 32 // 256)]
    else:
        # blocks run down the columns: block i becomes column i % 256 of row-block i // 256
        nb = rows // 256 * 256
        bits = blocks[:nb].reshape(nb // 256, 256, 32).transpose(0, 2, 1).reshape(1, -1, 256)
    _check(lp, np.ascontiguousarray(bits), axis, fmt, f"{fmt} axis {axis}")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("axis", [-1, -2])
def test_random_magnitudes_batched(lp, fmt, axis):
    g = W.rng(21, "x")
    mags = np.exp2(g.integers(-135, 125, size=(3, 64, 1))).astype(np.float32)
    x = (g.standard_normal((3, 64, 96)).astype(np.float32) * mags)
    _check(lp, W.bf16_bits(x), axis, fmt, f"{fmt} axis {axis} batched")


def test_deferred_grad_full_size(lp):
    """The deferred-quantization gradient (32768 x 2048, along -1), every byte."""
    w = W.WORKLOADS["mxfp8_deferred"]
    bits = W.bf16_bits(W.normal_f32(w.number, "grad", (1, w.M, w.N), 1.0))
    _check(lp, bits, -1, "mxfp8", "grad")


def test_deferred_weight_full_size_sampled(lp):
    """The deferred-quantization weight (64 x 2048 x 7168 bf16, along the
    reduction axis -2), quantized whole on the GPU; 48 sampled 32-row blocks
    compared byte for byte with the oracle."""
    w = W.WORKLOADS["mxfp8_deferred"]
    Wt = W.torch_normal_bf16((w.groups, w.N, w.K), w.w_sigma, seed=5005, device="cuda")
    q = lp.lp_mx_quant(Wt, -2, "mxfp8")
    torch.cuda.synchronize()
    g = W.rng(22, "x")
    for _ in range(48):
        e = int(g.integers(0, w.groups))
        rb = int(g.integers(0, w.N // 32))
        sl = Wt[e, rb * 32:(rb + 1) * 32].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        rc, rs = F.mx_quant(sl[None], -2, "e4m3")
        assert_bits_equal(q.scales[e, rb].cpu().numpy(), rs[0, 0], f"expert {e} block {rb} scales")
        assert_bits_equal(q.codes[e, rb * 32:(rb + 1) * 32].cpu().numpy(), rc[0], f"expert {e} block {rb} codes")


def test_mxfp4_grouped_operand_full_size(lp):
    """MXFP4 along -1 of the grouped workload's X (16384 x 4096), every byte."""
    w = W.WORKLOADS["mxfp4_grouped"]
    bits = W.bf16_bits(W.normal_f32(w.number, "x", (1, w.M, w.K), 1.0))
    _check(lp, bits, -1, "mxfp4", "X")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("shape", [(1, 1, 32), (1, 33, 64), (2, 1029, 32)])
def test_ragged_sizes_along_cols(lp, fmt, shape):
    """Block counts that leave the last workgroup partly empty, down to a
    single 32-element block."""
    g = W.rng(23, "x")
    x = g.standard_normal(shape).astype(np.float32) * np.exp2(g.integers(-20, 20, size=shape[:-1] + (1,)))
    _check(lp, W.bf16_bits(x.astype(np.float32)), -1, fmt, f"{fmt} {shape}")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("data", ["every_bf16", "random_batched"])
def test_dual_axis_equals_single_axis(lp, fmt, data):
    """lp_mx_quant_dual writes exactly the two copies lp_mx_quant writes along
    -1 and along -2, which the oracle checks (every finite bf16 value in
    blocks both ways, special blocks, random magnitudes, batched)."""
    if data == "every_bf16":
        blocks = np.concatenate([_special_blocks(), _every_finite_bf16_in_blocks()])
        n = blocks.size // (256 * 32) * (256 * 32)
        bits = blocks.reshape(-1)[:n].reshape(1, -1, 256)
    else:
        g = W.rng(24, "x")
        mags = np.exp2(g.integers(-30, 30, size=(3, 64, 1))).astype(np.float32)
        bits = W.bf16_bits(g.standard_normal((3, 64, 96)).astype(np.float32) * mags)
    src = bf16_dev(bits)
    qc, qr = lp.lp_mx_quant_dual(src, fmt)
    torch.cuda.synchronize()
    rc, rs = F.mx_quant(bits, -1, ELEM[fmt])
    assert_bits_equal(qc.codes.cpu().numpy(), rc, f"{fmt} dual, codes along -1")
    assert_bits_equal(qc.scales.cpu().numpy(), rs, f"{fmt} dual, scales along -1")
    rc, rs = F.mx_quant(bits, -2, ELEM[fmt])
    assert_bits_equal(qr.codes.cpu().numpy(), rc, f"{fmt} dual, codes along -2")
    assert_bits_equal(qr.scales.cpu().numpy(), rs, f"{fmt} dual, scales along -2")
