"""Forward y = x @ W^T of MX operands scaled along the contraction (the FP4
page's forward ops; the Deferred-MXFP8 page's MXFP8MatMul.forward) on the
block-scaled MFMA, against the oracle's fp64 product of the decoded operands
(GPU)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_close, dev, quantize
from oracle import formats as F
from oracle import gemm as O

pytestmark = pytest.mark.gpu


def _operands(lp, fmt, number, M, N, K, groups=0):
    x = W.with_outliers(W.normal_f32(number, "x", (M, K), 1.0), number, "x")
    w = W.normal_f32(number, "w", (groups, N, K) if groups else (N, K), 0.02)
    xq, xd = quantize(lp, fmt, x)
    wq, wd = quantize(lp, fmt, w)
    return xq, xd[0], wq, (wd if groups else wd[0])


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("M,N,K", [(300, 272, 384), (1, 16, 128), (513, 528, 1024), (64, 1040, 256)])
def test_linear_fwd(lp, fmt, M, N, K):
    xq, xd, wq, wd = _operands(lp, fmt, 41, M, N, K)
    y = lp.lp_linear_fwd(xq, wq)
    torch.cuda.synchronize()
    assert_close(y, O.linear_fwd(xd, wd), f"{fmt} forward {M}x{N}x{K}")


@pytest.mark.parametrize("K", [64, 320])
def test_linear_fwd_mxfp8_short_slabs(lp, K):
    """MXFP8 contracts in 64-deep slabs: K = 64 (one slab) and an odd count."""
    xq, xd, wq, wd = _operands(lp, "mxfp8", 42, 200, 48, K)
    y = lp.lp_linear_fwd(xq, wq)
    torch.cuda.synchronize()
    assert_close(y, O.linear_fwd(xd, wd), f"mxfp8 forward K={K}")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("sizes", [[100, 0, 300, 37, 1], [0, 0, 513], [256, 256]])
def test_grouped_fwd(lp, fmt, sizes):
    G, N, K = len(sizes), 272, 256
    M = int(sum(sizes)) + 29
    xq, xd, wq, wd = _operands(lp, fmt, 43, M, N, K, groups=G)
    ends = W.cumulative_ends(sizes)
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    lp.lp_grouped_fwd(xq, wq, dev(ends), y=y)
    torch.cuda.synchronize()
    ref = O.grouped_fwd(xd, wd, ends)
    end = int(ends[-1])
    for g, (s, e) in enumerate(O.group_bounds(ends)):
        if e > s:
            assert_close(y[s:e], ref[s:e], f"{fmt} group {g}")
    assert (y[end:].float() == 7.0).all(), "rows past the last end are not written"


def test_grouped_fwd_one_group_equals_linear(lp):
    xq, _, wq, _ = _operands(lp, "mxfp4", 44, 700, 256, 512)
    y1 = lp.lp_linear_fwd(xq, wq)
    wq3 = lp.QTensor("mxfp4", wq.codes, wq.scales, shape=(1, 256, 512))
    y2 = lp.lp_grouped_fwd(xq, wq3, dev(np.array([700], np.int32)))
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_more_tiles_than_cus(lp, fmt):
    """More 256 x 256 tiles than compute units (a second dispatch round): a
    grouped forward of 34 row tiles of 8 column tiles (272 tiles; an empty
    group, a 1-row group, rows past the last end kept) bit-identical to a
    linear forward per group and within tolerance of the oracle, and a dense
    one with ragged last row and column tiles (M = 9000, N = 2000: 36 x 8 =
    288 tiles)."""
    sizes = [4000, 0, 4300, 1]
    G, N, K = len(sizes), 2048, 256
    M = int(sum(sizes)) + 40
    xq, xd, wq, wd = _operands(lp, fmt, 47, M, N, K, groups=G)
    ends = W.cumulative_ends(sizes)
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    lp.lp_grouped_fwd(xq, wq, dev(ends), y=y)
    per = []
    for g, (s, e) in enumerate(O.group_bounds(ends)):
        if e > s:
            # copies, so that every pointer keeps the library's alignment
            xs = lp.QTensor(fmt, xq.codes.view(M, -1)[s:e].clone(), xq.scales.view(M, -1)[s:e].clone(),
                            shape=(1, e - s, K))
            wg = lp.QTensor(fmt, wq.codes.view(G, -1)[g].clone(), wq.scales.view(G, -1)[g].clone(), shape=(1, N, K))
            per.append((g, s, e, lp.lp_linear_fwd(xs, wg)))
    torch.cuda.synchronize()
    for g, s, e, yg in per:
        assert torch.equal(y[s:e].view(torch.int16), yg.view(torch.int16)), f"group {g} differs from the linear call"
    end = int(ends[-1])
    assert_close(y[:end], O.grouped_fwd(xd, wd, ends)[:end], f"{fmt} grouped forward, 272 tiles")
    assert (y[end:].float() == 7.0).all(), "rows past the last end are not written"

    Md, Nd = 9000, 2000
    xq, xd, wq, wd = _operands(lp, fmt, 48, Md, Nd, K)
    y = lp.lp_linear_fwd(xq, wq)
    torch.cuda.synchronize()
    assert_close(y, O.linear_fwd(xd, wd), f"{fmt} dense forward, 288 tiles")


@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_nan_scale_blocks(lp, fmt):
    """An E8M0 NaN scale (0xFF) makes its block NaN: the output column of a
    NaN weight block and the output row of a NaN input block are NaN, as in
    the decoded product."""
    M, N, K = 96, 64, 256
    x = W.normal_f32(45, "x", (M, K), 1.0)
    w = W.normal_f32(45, "w", (N, K), 0.02)
    xb, wb = W.bf16_bits(x)[None], W.bf16_bits(w)[None]
    elem = "e2m1" if fmt == "mxfp4" else "e4m3"
    xc, xs = F.mx_quant(xb, -1, elem)
    wc, ws = F.mx_quant(wb, -1, elem)
    xs[0, 5, 3] = 0xFF
    ws[0, 17, 1] = 0xFF
    xd = F.dequant(fmt, xc, xs, axis=-1)[0]
    wd = F.dequant(fmt, wc, ws, axis=-1)[0]
    xq = lp.QTensor(fmt, dev(xc), dev(xs), shape=(1, M, K))
    wq = lp.QTensor(fmt, dev(wc), dev(ws), shape=(1, N, K))
    y = lp.lp_linear_fwd(xq, wq)
    torch.cuda.synchronize()
    ref = O.linear_fwd(xd, wd)
    got = y.float().cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    rel = np.linalg.norm(got[ok] - ref[ok]) / np.linalg.norm(ref[ok])
    assert rel <= 5e-3


def test_rejects(lp):
    xq, _, wq, _ = _operands(lp, "mxfp4", 46, 64, 32, 128)
    wb = lp.QTensor("bf16", torch.zeros((1, 32, 128), dtype=torch.bfloat16, device="cuda"), shape=(1, 32, 128))
    with pytest.raises(lp.LpError, match="LP_ERR_FORMAT"):
        lp.lp_linear_fwd(xq, wb)
    x8, _, _, _ = _operands(lp, "mxfp8", 46, 64, 32, 128)
    with pytest.raises(lp.LpError, match="LP_ERR_FORMAT"):
        lp.lp_linear_fwd(x8, wq)                             # formats must agree


def test_mxfp4_forward_full_size(lp):
    """The benchmark's forward workload (8192 x 4096 @ (4096 x 4096)^T, MXFP4)
    through the same call, on sampled output rows."""
    w = W.WORKLOADS["mxfp4_forward"]
    x = W.normal_f32(w.number, "x", (w.M, w.K), w.x_sigma)
    wt = W.normal_f32(w.number, "w", (w.N, w.K), w.w_sigma)
    xc, xs = F.quant_mxfp4_f32(x[None])
    wc, ws = F.quant_mxfp4_f32(wt[None])
    xq = lp.QTensor("mxfp4", dev(xc), dev(xs), shape=(1, w.M, w.K))
    wq = lp.QTensor("mxfp4", dev(wc), dev(ws), shape=(1, w.N, w.K))
    y = lp.lp_linear_fwd(xq, wq)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, w.M, 67), [w.M - 1]]))
    xd = F.dequant("mxfp4", xc[:, rows], xs[:, rows])[0]
    wd = F.dequant("mxfp4", wc, ws)[0]
    assert_close(y[torch.from_numpy(rows).cuda()], O.linear_fwd(xd, wd), "full-size forward rows")
