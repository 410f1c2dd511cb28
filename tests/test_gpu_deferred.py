"""lp_grouped_dx_deferred: grad_X of the deferred MXFP8 recipe with the bf16
weight quantized as part of the call (small groups inside the product).

It must give the same bits as quantizing the weight with lp_mx_quant
(axis -2) and calling lp_grouped_bwd, for any split of the groups between
the two ways, and the oracle's result within the contraction tolerance."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_bits_equal, assert_close, bf16_dev, bits_host, dev
from oracle import formats as F
from oracle import gemm as O

pytestmark = pytest.mark.gpu


def _sentinel(shape):
    return torch.full(shape, -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)


def _case(lp, number, M, N, K, sizes, special=False):
    gbits = W.bf16_bits(W.normal_f32(number, "grad", (1, M, N), 1.0))
    gc, gs = F.mx_quant(gbits, -1, "e4m3")
    g = lp.QTensor("mxfp8", dev(gc[0]), dev(gs[0]), shape=(1, M, N), axis=-1)
    G = len(sizes)
    wv = W.normal_f32(number, "w", (G, N, K), 0.02)
    if special:
        wv[0, 40, 3] = np.inf            # group 0, column 3, block rows 32..63: scale 0xFF
        wv[2, 7, 100] = np.nan           # group 2, column 100, block rows 0..31
        wv[2, 64:96, 9] = 0.0            # an all-zero block: scale 0
        wv[2, 96:128, 11] = 2.0 ** -130  # a block of bf16 subnormals
    wbits = W.bf16_bits(wv)
    offsets = W.cumulative_ends(sizes)
    return g, F.dequant("mxfp8", gc, gs, axis=-1)[0], wbits, offsets


def _two_calls(lp, g, w, offs, dx0):
    wq = lp.lp_mx_quant(w, -2, "mxfp8")
    dx, _ = lp.lp_grouped_bwd(g, None, wq, offs, need_dw=False, grad_x=dx0)
    return dx


@pytest.mark.parametrize("fuse_rows", [0, 256, 100000])
def test_deferred_matches_quantize_then_product(lp, fuse_rows):
    """Nine groups (empty ones, a 1-row group, groups of 256 and 257 rows,
    one of 500), rows past the last offset kept, N = 1536 (a contraction of
    24 slabs), K = 416 (a partial 128-column tile), and weight blocks with
    an infinity, a NaN, all zeros and bf16 subnormals.  fuse_rows 0: every
    weight quantized first; 256: groups of up to 256 rows fused; 100000:
    every group fused."""
    M, N, K = 1500, 1536, 416
    sizes = [100, 0, 300, 1, 256, 257, 40, 500, 0]
    g, gd, wbits, offsets = _case(lp, 70, M, N, K, sizes, special=True)
    w = bf16_dev(wbits)
    offs = torch.from_numpy(offsets).cuda()
    ref = _two_calls(lp, g, w, offs, _sentinel((M, K)))
    G = len(sizes)
    codes = torch.full((G, N, K), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((G, N // 32, K), 0x5A, dtype=torch.uint8, device="cuda")
    dx = lp.lp_grouped_dx_deferred(g, w, offs, fuse_rows=fuse_rows, grad_x=_sentinel((M, K)), w_codes=codes,
                                   w_scales=scales)
    torch.cuda.synchronize()
    assert_bits_equal(bits_host(dx), bits_host(ref), f"fuse_rows={fuse_rows} vs quantize-then-product")
    end = int(offsets[-1])
    assert np.all(bits_host(dx[end:]) == 0xFFFF), "rows past the last offset were written"
    wc, ws = F.mx_quant(wbits, -2, "e4m3")
    # The weight copy: written (the oracle's codes and scales) for the groups
    # quantized first (all of them when fuse_rows is 0), left as it was for
    # the groups quantized inside the product.
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    for gi, (s0, e0) in enumerate(O.group_bounds(offsets)):
        if fuse_rows == 0 or e0 - s0 > fuse_rows:
            assert np.array_equal(got_c[gi], wc[gi]) and np.array_equal(got_s[gi], ws[gi]), f"group {gi} codes"
        else:
            assert np.all(got_c[gi] == 0xA5) and np.all(got_s[gi] == 0x5A), f"group {gi} copy was written"
    wd = F.dequant("mxfp8", wc, ws, axis=-2)
    exp, _ = O.grouped_dx(gd, wd, offsets)
    got = dx[:end].float().cpu().numpy()
    nan = np.isnan(exp[:end])
    assert np.array_equal(np.isnan(got), nan), "NaN outputs differ from the oracle's"
    rows_ok = ~nan.any(axis=1)
    assert rows_ok.sum() > 0
    cols_ok = ~nan.any(axis=0)
    sel = np.ix_(rows_ok, cols_ok)
    assert_close(dx[:end][torch.from_numpy(np.where(rows_ok)[0]).cuda()][:, torch.from_numpy(np.where(cols_ok)[0]).cuda()],
                 exp[:end][sel], f"fuse_rows={fuse_rows} vs oracle")


def test_deferred_many_groups(lp):
    """150 groups, most small, with groups above the threshold at indices
    past 64 and 128 (the quantize-first pass lists its groups 64 at a time,
    carrying the running end across), an empty group among them, and rows
    past the last offset: dX bit for bit equal to quantize-then-product, the
    weight copy written for exactly the large groups."""
    N, K, G = 512, 64, 150
    rng = W.rng(72, "route")
    sizes = rng.integers(0, 60, size=G)
    for gi, n in ((3, 700), (70, 300), (64, 257), (129, 513), (149, 400), (100, 0)):
        sizes[gi] = n
    M = int(sizes.sum()) + 37
    g, gd, wbits, offsets = _case(lp, 72, M, N, K, sizes.tolist())
    w = bf16_dev(wbits)
    offs = torch.from_numpy(offsets).cuda()
    ref = _two_calls(lp, g, w, offs, _sentinel((M, K)))
    codes = torch.full((G, N, K), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full((G, N // 32, K), 0x5A, dtype=torch.uint8, device="cuda")
    dx = lp.lp_grouped_dx_deferred(g, w, offs, fuse_rows=256, grad_x=_sentinel((M, K)), w_codes=codes,
                                   w_scales=scales)
    torch.cuda.synchronize()
    assert_bits_equal(bits_host(dx), bits_host(ref), "150 groups vs quantize-then-product")
    wc, ws = F.mx_quant(wbits, -2, "e4m3")
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    large = [gi for gi, (s0, e0) in enumerate(O.group_bounds(offsets)) if e0 - s0 > 256]
    assert large == [3, 64, 70, 129, 149]
    for gi in range(G):
        if gi in large:
            assert np.array_equal(got_c[gi], wc[gi]) and np.array_equal(got_s[gi], ws[gi]), f"group {gi} codes"
        else:
            assert np.all(got_c[gi] == 0xA5) and np.all(got_s[gi] == 0x5A), f"group {gi} copy was written"


@pytest.mark.parametrize("N,K", [(800, 272), (1024, 400)])
def test_deferred_other_widths_fall_back(lp, N, K):
    """N % 512 != 0 or K % 32 != 0: every weight is quantized first; the
    result is still the quantize-then-product one."""
    M = 700
    sizes = [130, 0, 17, 300, 203]
    g, gd, wbits, offsets = _case(lp, 71, M, N, K, sizes)
    w = bf16_dev(wbits)
    offs = torch.from_numpy(offsets).cuda()
    ref = _two_calls(lp, g, w, offs, _sentinel((M, K)))
    dx = lp.lp_grouped_dx_deferred(g, w, offs, fuse_rows=256, grad_x=_sentinel((M, K)))
    torch.cuda.synchronize()
    assert_bits_equal(bits_host(dx), bits_host(ref), f"N = {N}, K = {K}")


def test_deferred_full_size(lp):
    """The 64-expert deferred workload (32768 tokens, Zipf(1.1) sizes, W
    64 x 2048 x 7168): the fused call equals quantize-then-product bit for
    bit over the whole 32768 x 7168 output."""
    w = W.WORKLOADS["mxfp8_deferred"]
    offs = torch.from_numpy(W.cumulative_ends(W.group_sizes(w))).cuda()
    Wt = W.torch_normal_bf16((w.groups, w.N, w.K), w.w_sigma, seed=5105, device="cuda")
    Gt = W.torch_normal_bf16((w.M, w.N), 1.0, seed=5106, device="cuda")
    gq = lp.lp_mx_quant(Gt, -1, "mxfp8")
    gq.shape = (1, w.M, w.N)
    ref = _two_calls(lp, gq, Wt, offs, torch.empty((w.M, w.K), dtype=torch.bfloat16, device="cuda"))
    # the benchmark's threshold (1536: experts of up to six row tiles fused) and 256
    for fr in (1536, 256):
        dx = lp.lp_grouped_dx_deferred(gq, Wt, offs, fuse_rows=fr)
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16), ref.view(torch.int16)), f"fused call (fuse_rows {fr}) differs"
