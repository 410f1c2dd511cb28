"""Forward y = x @ W^T through bf16 tiles with both operands k-major (GPU):
a bf16 input with a bf16, block-FP8 or NVFP4 weight ("Train adapters on top of FP8
weights", FP8LinearFunction.forward and FP8GroupedMatmulFunction.forward)
and NVFP4 operands on both sides ("Add Autograd Backward Support for FP4 GEMM
Custom Ops", the f4f4bf16 forward ops), dense and grouped, against the
oracle's forwards (oracle.gemm.fp8_block_fwd, nvfp4_fwd, linear_fwd,
grouped_fwd) within the contraction tolerance."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_close, bits_host, dev, qtensor
from oracle import formats as F
from oracle import gemm as O

pytestmark = pytest.mark.gpu

PAIRS = [("bf16", "bf16"), ("bf16", "fp8_b128"), ("nvfp4", "nvfp4"), ("bf16", "nvfp4")]


def _make(lp, fmt, v):
    """Oracle-generated codes of fp32 values v ([R,C] or [b,R,C]) and their
    library descriptor.  Returns (descriptor, host tuple)."""
    v3 = np.asarray(v, dtype=np.float32)
    v3 = v3.reshape((1,) + v3.shape) if v3.ndim == 2 else v3
    if fmt == "bf16":
        host = (W.bf16_bits(v3),)
        return qtensor(lp, "bf16", host[0], shape=v3.shape), host
    if fmt == "fp8_b128":
        host = F.quant_fp8_b128(v3)
        return qtensor(lp, fmt, host[0], host[1], shape=v3.shape), host
    c, s, ts = F.quant_nvfp4(v3)
    return qtensor(lp, fmt, c, s, float(ts), shape=v3.shape), (c, s, ts)


def _reference(fx, fw, xh, wh, offsets=None):
    if fx == "nvfp4":
        return O.nvfp4_fwd(xh[0][0], xh[1][0], xh[2], wh[0], wh[1], wh[2], offsets)
    if fw == "nvfp4":
        wb = F.dequant("nvfp4", wh[0], wh[1], wh[2])
        return O.linear_fwd(xh[0][0], wb[0]) if offsets is None else O.grouped_fwd(xh[0][0], wb, offsets)
    if fw == "fp8_b128":
        return O.fp8_block_fwd(xh[0][0], wh[0], wh[1], offsets)
    return O.linear_fwd(xh[0][0], wh[0][0]) if offsets is None else O.grouped_fwd(xh[0][0], wh[0], offsets)


def _operands(lp, fx, fw, number, M, N, K, groups=0):
    x = W.with_outliers(W.normal_f32(number, "x", (M, K), 1.0), number, "x")
    w = W.normal_f32(number, "w", (groups, N, K) if groups else (N, K), 0.02)
    xq, xh = _make(lp, fx, x)
    wq, wh = _make(lp, fw, w)
    return xq, xh, wq, wh


def _shapes(fx, fw=None):
    # several tiles with ragged edges, one row, partial 128-blocks along N and
    # K, a contraction shorter than one 64-deep slab
    base = [(300, 272, 384), (1, 16, 32), (513, 528, 1024), (64, 1040, 256)]
    nv = "nvfp4" in (fx, fw)
    return base + ([(200, 144, 352), (70, 48, 96)] if nv else [(200, 144, 336), (70, 48, 16)])


@pytest.mark.parametrize("fx,fw", PAIRS)
def test_linear_fwd(lp, fx, fw):
    for i, (M, N, K) in enumerate(_shapes(fx, fw)):
        xq, xh, wq, wh = _operands(lp, fx, fw, 50 + i, M, N, K)
        y = lp.lp_linear_fwd(xq, wq)
        torch.cuda.synchronize()
        assert_close(y, _reference(fx, fw, xh, wh), f"{fx} x {fw} forward {M}x{N}x{K}")


@pytest.mark.parametrize("fx,fw", PAIRS)
@pytest.mark.parametrize("sizes", [[100, 0, 300, 37, 1], [0, 0, 513], [256, 256]])
def test_grouped_fwd(lp, fx, fw, sizes):
    G, N, K = len(sizes), 272, 256
    M = int(sum(sizes)) + 29
    xq, xh, wq, wh = _operands(lp, fx, fw, 57, M, N, K, groups=G)
    ends = W.cumulative_ends(sizes)
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    lp.lp_grouped_fwd(xq, wq, dev(ends), y=y)
    torch.cuda.synchronize()
    ref = _reference(fx, fw, xh, wh, ends)
    end = int(ends[-1])
    for g, (s, e) in enumerate(O.group_bounds(ends)):
        if e > s:
            assert_close(y[s:e], ref[s:e], f"{fx} x {fw} group {g}")
    assert (y[end:].float() == 7.0).all(), "rows past the last end are not written"


@pytest.mark.parametrize("fx,fw,N", [("bf16", "fp8_b128", 2048), ("bf16", "fp8_b128", 1936), ("nvfp4", "nvfp4", 2048),
                                     ("bf16", "nvfp4", 2048), ("bf16", "nvfp4", 1936)])
def test_grouped_fwd_round_split(lp, fx, fw, N):
    """A grouped forward over a 4096-long contraction with more 256 x 256
    tiles than one round of the 256 CUs: 34 row tiles of 8 column tiles,
    272 tiles, the last 16 run as 256 x 128 tiles in a second launch (N =
    1936 ends on a single 128-wide tile).  Bit-identical to a linear forward
    per group, within tolerance of the oracle on sampled rows of every group,
    rows past the last end kept."""
    sizes = [4000, 0, 4300, 1]
    G, K = len(sizes), 4096
    M = int(sum(sizes)) + 40
    xq, xh, wq, wh = _operands(lp, fx, fw, 59, M, N, K, groups=G)
    ends = W.cumulative_ends(sizes)
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    lp.lp_grouped_fwd(xq, wq, dev(ends), y=y)
    per = []
    for g, (s, e) in enumerate(O.group_bounds(ends)):
        if e > s:
            # copies, so that every pointer keeps the library's alignment
            xsc = xq.scales.view(M, -1)[s:e].clone() if xq.scales is not None else None
            xs = lp.QTensor(fx, xq.codes.view(M, -1)[s:e].clone(), xsc, xq.tensor_scale, shape=(1, e - s, K))
            ws = wq.scales.view(G, -1)[g].clone() if wq.scales is not None else None
            wg = lp.QTensor(fw, wq.codes.view(G, -1)[g].clone(), ws, wq.tensor_scale, shape=(1, N, K))
            per.append((g, s, e, lp.lp_linear_fwd(xs, wg)))
    torch.cuda.synchronize()
    for g, s, e, yg in per:
        assert np.array_equal(bits_host(y[s:e]), bits_host(yg)), f"group {g} differs from the linear forward"
        rows = s + np.sort(W.rng(59 + g, "x").choice(e - s, size=min(24, e - s), replace=False))
        xr = tuple(a[:, rows] if np.ndim(a) == 3 else a for a in xh)
        wr = tuple(a[g:g + 1] if np.ndim(a) == 3 else a for a in wh)
        assert_close(y[torch.from_numpy(rows).cuda()], _reference(fx, fw, xr, wr), f"{fx} x {fw} group {g}, N = {N}")
    end = int(ends[-1])
    assert (y[end:].float() == 7.0).all(), "rows past the last end are not written"


@pytest.mark.parametrize("fx,fw", [("bf16", "fp8_b128"), ("nvfp4", "nvfp4"), ("bf16", "nvfp4")])
def test_fused_decode_equals_decoded_copy(lp, fx, fw):
    """Decoding inside the contraction gives the same bits as decoding the
    operands first (lp_dequant) and running the bf16 x bf16 forward: the
    decode equals the standalone dequantization, and the fp32 sums run in the
    same order."""
    M, N, K = 513, 528, 1024
    xq, _, wq, _ = _operands(lp, fx, fw, 58, M, N, K)
    y = lp.lp_linear_fwd(xq, wq)
    xb = xq if fx == "bf16" else lp.QTensor("bf16", lp.lp_dequant(xq), shape=(1, M, K))
    wb = lp.QTensor("bf16", lp.lp_dequant(wq), shape=(1, N, K))
    y2 = lp.lp_linear_fwd(xb, wb)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(y), bits_host(y2))


def test_nan_codes_and_scales(lp):
    """A NaN E4M3 weight code makes its output column NaN (block-FP8); a NaN
    E4M3 block scale of x makes its output row NaN (NVFP4), and one of an
    NVFP4 weight its output column (bf16 x), as in the oracle."""
    M, N, K = 96, 64, 256
    x = W.normal_f32(59, "x", (M, K), 1.0)
    w = W.normal_f32(59, "w", (N, K), 0.02)
    xb = W.bf16_bits(x)[None]
    wc, ws = F.quant_fp8_b128(w[None])
    wc[0, 17, 5] = 0x7F
    y = lp.lp_linear_fwd(qtensor(lp, "bf16", xb, shape=(1, M, K)), qtensor(lp, "fp8_b128", wc, ws, shape=(1, N, K)))
    torch.cuda.synchronize()
    ref = O.fp8_block_fwd(xb[0], wc, ws)
    got = y.float().cpu().numpy()
    assert np.isnan(ref[:, 17]).all() and np.array_equal(np.isnan(got), np.isnan(ref))
    xc, xs, xts = F.quant_nvfp4(x[None])
    wc4, ws4, wts = F.quant_nvfp4(w[None])
    xs[0, 5, 3] = 0x7F
    y = lp.lp_linear_fwd(qtensor(lp, "nvfp4", xc, xs, float(xts), shape=(1, M, K)),
                         qtensor(lp, "nvfp4", wc4, ws4, float(wts), shape=(1, N, K)))
    torch.cuda.synchronize()
    ref = O.nvfp4_fwd(xc[0], xs[0], xts, wc4, ws4, wts)
    got = y.float().cpu().numpy()
    assert np.isnan(ref[5]).all() and np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.linalg.norm(got[ok] - ref[ok]) / np.linalg.norm(ref[ok]) <= 5e-3
    # bf16 x with an NVFP4 weight: a NaN block scale of W makes its output column NaN
    ws4[0, 40, 2] = 0x7F
    y = lp.lp_linear_fwd(qtensor(lp, "bf16", xb, shape=(1, M, K)),
                         qtensor(lp, "nvfp4", wc4, ws4, float(wts), shape=(1, N, K)))
    torch.cuda.synchronize()
    ref = O.linear_fwd(xb[0], F.dequant("nvfp4", wc4, ws4, wts)[0])
    got = y.float().cpu().numpy()
    assert np.isnan(ref[:, 40]).all() and np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.linalg.norm(got[ok] - ref[ok]) / np.linalg.norm(ref[ok]) <= 5e-3


def test_rejects(lp):
    xq, _, wq, _ = _operands(lp, "nvfp4", "nvfp4", 60, 64, 32, 96)
    xb, _, wf, _ = _operands(lp, "bf16", "fp8_b128", 60, 64, 32, 96)
    with pytest.raises(lp.LpError, match="LP_ERR_FORMAT"):
        lp.lp_linear_fwd(xq, wf)                             # NVFP4 x needs an NVFP4 weight
    with pytest.raises(lp.LpError, match="LP_ERR_FORMAT"):
        lp.lp_linear_fwd(wf, xb)                             # the block-FP8 operand is the weight
    x48, _, w48, _ = _operands(lp, "nvfp4", "nvfp4", 60, 64, 32, 48)
    with pytest.raises(lp.LpError, match="LP_ERR_SHAPE"):
        lp.lp_linear_fwd(x48, w48)                           # NVFP4: K % 32


def test_nvfp4_forward_full_size(lp):
    """The NVFP4 forward workload (8192 x 4096 @ (4096 x 4096)^T, 1% outliers)
    through the fused call, on sampled output rows; the timed order (X
    decoded once with lp_dequant, then the bf16 x NVFP4 forward) gives the
    same bits."""
    w = W.WORKLOADS["nvfp4_forward"]
    x = W.with_outliers(W.normal_f32(w.number, "x", (w.M, w.K), w.x_sigma), w.number, "x")
    wt = W.with_outliers(W.normal_f32(w.number, "w", (w.N, w.K), w.w_sigma), w.number, "w")
    xq, xh = _make(lp, "nvfp4", x)
    wq, wh = _make(lp, "nvfp4", wt)
    y = lp.lp_linear_fwd(xq, wq)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, w.M, 67), [w.M - 1]]))
    ref = O.nvfp4_fwd(xh[0][0][rows], xh[1][0][rows], xh[2], wh[0], wh[1], wh[2])
    assert_close(y[torch.from_numpy(rows).cuda()], ref, "full-size NVFP4 forward rows")
    xb = lp.lp_dequant(xq)
    y2 = lp.lp_linear_fwd(lp.QTensor("bf16", xb, shape=(1, w.M, w.K)), wq)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "decode-once forward differs"


def test_fp8_grouped_forward_full_size(lp):
    """The block-FP8 grouped forward workload (8 experts, 16384 tokens,
    W 8 x 2048 x 4096) through the same call, on sampled rows of every group."""
    w = W.WORKLOADS["fp8_grouped_forward"]
    ends = W.cumulative_ends(W.group_sizes(w))
    x = W.normal_f32(w.number, "x", (w.M, w.K), w.x_sigma)
    wt = W.normal_f32(w.number, "w", (w.groups, w.N, w.K), w.w_sigma)
    xq, xh = _make(lp, "bf16", x)
    wq, wh = _make(lp, "fp8_b128", wt)
    y = lp.lp_grouped_fwd(xq, wq, dev(ends))
    torch.cuda.synchronize()
    for g, (s, e) in enumerate(O.group_bounds(ends)):
        if e <= s:
            continue
        rows = np.unique(np.concatenate([np.arange(s, e, 97), [e - 1]]))
        wd = F.dequant("fp8_b128", wh[0][g:g + 1], wh[1][g:g + 1])[0]
        ref = O.linear_fwd(xh[0][0][rows], wd)
        assert_close(y[torch.from_numpy(rows).cuda()], ref, f"full-size block-FP8 forward, group {g}")
