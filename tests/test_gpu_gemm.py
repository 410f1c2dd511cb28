"""lp_linear_bwd / lp_grouped_bwd against the fp64 oracle (GPU).

Tolerance on every output tensor: relative Frobenius error <= 5e-3 and
max |error| <= 1e-2 * max |reference|; both sides consume the same
quantized operands, so the bound covers only accumulation order and the
final bf16 rounding (about 1e-3 relative on its own).
"""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_bits_equal, assert_close, bf16_dev, bits_host, dev, quantize
from oracle import formats as F
from oracle import gemm as O

pytestmark = pytest.mark.gpu

FORMATS = [("bf16", -1), ("mxfp4", -1), ("nvfp4", -1), ("fp8_b128", -1), ("mxfp8", -1), ("mxfp8", -2)]


def _grad(lp, number, M, N, fmt="bf16"):
    bits = W.bf16_bits(W.normal_f32(number, "grad", (M, N), 1.0))
    if fmt == "bf16":
        return lp.QTensor("bf16", bf16_dev(bits), shape=(1, M, N)), bits
    q, deq = quantize(lp, "mxfp8", F.bf16_bits_to_f64(bits).astype(np.float32)[None], axis=-1)
    return q, deq[0]


def _operand(lp, number, tensor, shape, fmt, axis, sigma=1.0):
    vals = W.normal_f32(number, tensor, shape, sigma)
    q, deq = quantize(lp, fmt, vals, axis)
    return q, deq


@pytest.mark.parametrize("fmt,axis", FORMATS)
def test_linear_small_ragged(lp, fmt, axis):
    """M = 300 (ragged), N = 320, K = 288: several tiles, partial tiles in
    every dimension, the narrow-tile configuration."""
    M, N, K = 300, 320, 288
    if fmt == "mxfp8" and axis == -2:
        M = 320                       # X scales along rows need M % 32
    g, gb = _grad(lp, 31, M, N)
    x, xd = _operand(lp, 31, "x", (M, K), fmt, axis)
    w, wd = _operand(lp, 31, "w", (N, K), fmt, axis)
    dx, dw = lp.lp_linear_bwd(g, x, w)
    torch.cuda.synchronize()
    assert_close(dx, O.linear_dx(gb, wd[0]), f"{fmt}{axis} dX")
    assert_close(dw, O.linear_dw(gb, xd[0]), f"{fmt}{axis} dW")


@pytest.mark.parametrize("fmt,axis", FORMATS)
def test_linear_wide_tiles(lp, fmt, axis):
    """Shapes that select the 256x256 configuration for both products:
    dX 4100 x 4096 (ragged M) over N = 272; dW 4096 x 4096 over M = 160."""
    g, gb = _grad(lp, 32, 4100, 272)
    w, wd = _operand(lp, 32, "w", (272, 4096), fmt, -1 if axis == -2 else axis)
    dx, _ = lp.lp_linear_bwd(g, None, w, need_dw=False)
    g2, gb2 = _grad(lp, 33, 160, 4096)
    x, xd = _operand(lp, 33, "x", (160, 4096), fmt, axis)
    _, dw = lp.lp_linear_bwd(g2, x, None, need_dx=False)
    torch.cuda.synchronize()
    assert_close(dx, O.linear_dx(gb, wd[0]), f"{fmt} dX")
    assert_close(dw, O.linear_dw(gb2, xd[0]), f"{fmt}{axis} dW")


def test_linear_mxfp8_grad(lp):
    """MX-quantized gradient (along its last axis) times an MXFP8 weight
    quantized along its reduction axis, as in the deferred backward."""
    M, N, K = 520, 384, 448
    g, gd = _grad(lp, 34, M, N, fmt="mxfp8")
    w, wd = _operand(lp, 34, "w", (N, K), "mxfp8", -2, sigma=0.02)
    dx, _ = lp.lp_linear_bwd(g, None, w, need_dw=False)
    torch.cuda.synchronize()
    assert_close(dx, O.linear_dx(gd, wd[0]), "mxfp8 x mxfp8 dX")


def _workspace(lp, g, x, w, need_dx=True, need_dw=True):
    n = lp.lp_linear_bwd_workspace(g, x, w, need_dx, need_dw)
    assert n > 0, "shape expected to split its contraction"
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def _counters_zero(ws, tiles):
    assert int(ws[: 4 * tiles].count_nonzero()) == 0, "per-tile counters not cleared"


@pytest.mark.parametrize("fmt,axis", FORMATS)
def test_split_dx(lp, fmt, axis):
    """dX over a long contraction with few output tiles: M = 300 (ragged),
    N = 4096, K = 544 -> 2 x 3 tiles of 256 x 256, four splits of 16 slabs.
    Two calls in a row give the same bits (the sum does not depend on which
    split finishes last) and leave the counters at zero."""
    M, N, K = 300, 4096, 544
    g, gb = _grad(lp, 35, M, N)
    w, wd = _operand(lp, 35, "w", (N, K), fmt, axis)
    ws = _workspace(lp, g, None, w, need_dw=False)
    dx1, _ = lp.lp_linear_bwd(g, None, w, need_dw=False, workspace=ws)
    dx2, _ = lp.lp_linear_bwd(g, None, w, need_dw=False, workspace=ws)
    torch.cuda.synchronize()
    _counters_zero(ws, 6)
    assert_close(dx1, O.linear_dx(gb, wd[0]), f"{fmt}{axis} split dX")
    assert_bits_equal(bits_host(dx2), bits_host(dx1), "second call")


@pytest.mark.parametrize("fmt,axis", FORMATS)
def test_split_dw(lp, fmt, axis):
    """dW over a long, ragged token axis: M = 4100 (4128 for X scaled along
    rows), N = 272, K = 544 -> 2 x 3 tiles, 65 slabs in four splits, the last
    one short and ragged."""
    M = 4128 if (fmt == "mxfp8" and axis == -2) else 4100
    N, K = 272, 544
    g, gb = _grad(lp, 36, M, N)
    x, xd = _operand(lp, 36, "x", (M, K), fmt, axis)
    ws = _workspace(lp, g, x, None, need_dx=False)
    _, dw1 = lp.lp_linear_bwd(g, x, None, need_dx=False, workspace=ws)
    _, dw2 = lp.lp_linear_bwd(g, x, None, need_dx=False, workspace=ws)
    torch.cuda.synchronize()
    _counters_zero(ws, 6)
    assert_close(dw1, O.linear_dw(gb, xd[0]), f"{fmt}{axis} split dW")
    assert_bits_equal(bits_host(dw2), bits_host(dw1), "second call")


def test_split_mxfp8_grad(lp):
    """Split dX with an MX-quantized gradient and an MXFP4 weight (decoded
    to bf16 in the mainloop)."""
    M, N, K = 520, 4096, 448
    g, gd = _grad(lp, 37, M, N, fmt="mxfp8")
    w, wd = _operand(lp, 37, "w", (N, K), "mxfp4", -1, sigma=0.02)
    ws = _workspace(lp, g, None, w, need_dw=False)
    dx, _ = lp.lp_linear_bwd(g, None, w, need_dw=False, workspace=ws)
    torch.cuda.synchronize()
    _counters_zero(ws, 3 * 2)
    assert_close(dx, O.linear_dx(gd, wd[0]), "mxfp8 x mxfp4 split dX")


def test_native_mx_needs_no_workspace(lp):
    """MXFP8 gradient x MXFP8 weight along its reduction axis runs on the
    block-scaled MFMA, which does not split."""
    g, _ = _grad(lp, 45, 520, 4096, fmt="mxfp8")
    w, _ = _operand(lp, 45, "w", (4096, 448), "mxfp8", -2, sigma=0.02)
    assert lp.lp_linear_bwd_workspace(g, None, w, True, False) == 0


@pytest.mark.parametrize("N", [288, 2048, 4608])
def test_native_mx_grouped_edges(lp, N):
    """Block-scaled MFMA path, grouped: an empty group, a group smaller than
    a tile, ragged group ends, rows past the last offset kept, output width
    336 (a partial 256-column tile).  N = 288: a contraction ending half way
    through a 64-deep slab (scale bytes gathered per slab); N = 2048, 4608:
    scale rows loaded in 512-deep chunks, 4608 ending mid-way through the
    16-slab main-loop block."""
    M, K, G = 700, 336, 5
    sizes = [130, 0, 17, 300, 203]
    offsets = W.cumulative_ends(sizes)
    g, gd = _grad(lp, 46, M, N, fmt="mxfp8")
    w, wd = _operand(lp, 46, "w", (G, N, K), "mxfp8", -2, sigma=0.02)
    dx0 = _sentinel((M, K))
    dx, _ = lp.lp_grouped_bwd(g, None, w, torch.from_numpy(offsets).cuda(), need_dw=False, grad_x=dx0)
    torch.cuda.synchronize()
    ref, end = O.grouped_dx(gd, wd, offsets)
    assert_close(dx[:end], ref[:end], f"native mx grouped dX N={N}")
    assert np.all(bits_host(dx[end:]) == 0xFFFF), "rows past the last offset were written"


def _mx_grad_with_nan_rows(lp, number, M, N, nan_rows):
    """MXFP8 gradient (scales along -1) whose listed rows each get one NaN
    scale block; returns the descriptor and the oracle's decoded bits."""
    gbits = W.bf16_bits(W.normal_f32(number, "grad", (1, M, N), 1.0))
    gc, gs = F.mx_quant(gbits, -1, "e4m3")
    gs = gs.copy()
    for i, r in enumerate(nan_rows):
        gs[0, r, (7 * i) % (N // 32)] = 0xFF
    g = lp.QTensor("mxfp8", dev(gc[0]), dev(gs[0]), shape=(1, M, N), axis=-1)
    return g, F.dequant("mxfp8", gc, gs, axis=-1)[0]


def test_native_mx_persistent_grouped(lp):
    """More tiles than compute units: one workgroup per compute unit walks the
    tile list, issuing each tile's first loads before the previous tile's
    results are written (about 2.5 tiles per workgroup here).  37 groups
    (empty ones, groups of a few rows, groups spanning several row tiles),
    rows past the last offset kept, a contraction of 24 slabs (N = 1536, not
    a whole number of 16-slab passes), a partial last column tile (K =
    2064), and two gradient rows
    with a NaN scale block, which must come out NaN and leave every other
    row finite."""
    M, N, K, G = 10000, 1536, 2064, 37
    sizes = W.rng(48, "route").integers(0, 400, size=G)
    sizes[10] = 900
    sizes = (sizes * (M - 150) // sizes.sum()).astype(np.int64)
    sizes[[3, 4, 20]] = 0
    sizes[[5, 6]] = [1, 31]
    assert 0 < sizes.sum() < M
    offsets = W.cumulative_ends(sizes)
    end = int(offsets[-1])
    nan_rows = [int(offsets[9]) + 3, end - 1]
    g, gd = _mx_grad_with_nan_rows(lp, 48, M, N, nan_rows)
    w, wd = _operand(lp, 48, "w", (G, N, K), "mxfp8", -2, sigma=0.02)
    dx0 = _sentinel((M, K))
    dx, _ = lp.lp_grouped_bwd(g, None, w, torch.from_numpy(offsets).cuda(), need_dw=False, grad_x=dx0)
    torch.cuda.synchronize()
    got = dx.float().cpu().numpy()
    assert np.all(bits_host(dx[end:]) == 0xFFFF), "rows past the last offset were written"
    assert np.isnan(got[nan_rows]).all(), "a NaN scale block must make its output row NaN"
    fin = np.setdiff1d(np.arange(end), nan_rows)
    assert not np.isnan(got[fin]).any(), "NaN outside the rows with a NaN scale block"
    ref, _ = O.grouped_dx(gd, wd, offsets)
    assert_close(dx[torch.from_numpy(fin).cuda()], ref[fin], "persistent grouped dX")


def test_native_mx_persistent_dense(lp):
    """Dense dX with 17 x 17 output tiles (ragged M, partial tiles on both
    sides) through the persistent walk."""
    M, N, K = 4100, 1024, 4336
    g, gd = _grad(lp, 49, M, N, fmt="mxfp8")
    w, wd = _operand(lp, 49, "w", (N, K), "mxfp8", -2, sigma=0.02)
    dx, _ = lp.lp_linear_bwd(g, None, w, need_dw=False)
    torch.cuda.synchronize()
    assert_close(dx, O.linear_dx(gd, wd[0]), "persistent dense dX")


def test_native_mx_matches_decode_path_with_nan_blocks(lp):
    """The block-scaled MFMA and the decode-to-bf16 path agree: on finite
    blocks within the tolerance, and a gradient block with scale 0xFF (NaN)
    makes the same output rows NaN in both."""
    M, N, K = 300, 512, 288
    gbits = W.bf16_bits(W.normal_f32(47, "grad", (1, M, N), 1.0))
    gc, gs = F.mx_quant(gbits, -1, "e4m3")
    gs = gs.copy()
    gs[0, 7, 3] = 0xFF                           # row 7, columns 96..127
    gs[0, 200, 15] = 0xFF                        # row 200, columns 480..511
    g = lp.QTensor("mxfp8", dev(gc[0]), dev(gs[0]), shape=(1, M, N), axis=-1)
    w, wd = _operand(lp, 47, "w", (N, K), "mxfp8", -2, sigma=0.02)
    dx_native, _ = lp.lp_linear_bwd(g, None, w, need_dw=False)
    gbf = lp.lp_dequant(g)
    gq = lp.QTensor("bf16", gbf.view(M, N), shape=(1, M, N))
    dx_decode, _ = lp.lp_linear_bwd(gq, None, w, need_dw=False)
    torch.cuda.synchronize()
    a = dx_native.float().cpu().numpy()
    b = dx_decode.float().cpu().numpy()
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.isnan(a[7]).all() and np.isnan(a[200]).all() and not np.isnan(np.delete(a, [7, 200], 0)).any()
    fin = np.delete(np.arange(M), [7, 200])
    ref = O.linear_dx(F.dequant("mxfp8", gc, gs, axis=-1)[0][fin], wd[0])
    assert_close(dx_native[torch.from_numpy(fin).cuda()], ref, "native vs oracle, finite rows")


def test_split_workspace_too_small_falls_back(lp):
    """A workspace smaller than reported: the call does not split, same result
    within tolerance, workspace untouched."""
    M, N, K = 300, 4096, 544
    g, gb = _grad(lp, 38, M, N)
    w, wd = _operand(lp, 38, "w", (N, K), "fp8_b128", -1)
    n = lp.lp_linear_bwd_workspace(g, None, w, True, False)
    ws = torch.zeros(n - 256, dtype=torch.uint8, device="cuda")
    dx, _ = lp.lp_linear_bwd(g, None, w, need_dw=False, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0
    assert_close(dx, O.linear_dx(gb, wd[0]), "fallback dX")


@pytest.mark.parametrize("M,N,K", [(4128, 272, 336), (2048, 512, 768)])
def test_native_mx_dw(lp, M, N, K):
    """Dense dW of an MXFP8 gradient and an MXFP8 input both scaled along
    their rows (the token axis): the block-scaled MFMA's dW form.  4128
    tokens end half way through a 64-deep slab; 272 x 336 leaves partial
    256 x 256 tiles."""
    gbits = W.bf16_bits(W.normal_f32(48, "grad", (1, M, N), 1.0))
    gc, gs = F.mx_quant(gbits, -2, "e4m3")
    g = lp.QTensor("mxfp8", dev(gc[0]), dev(gs[0]), shape=(1, M, N), axis=-2)
    x, xd = _operand(lp, 48, "x", (M, K), "mxfp8", -2)
    _, dw = lp.lp_linear_bwd(g, x, None, need_dx=False)
    torch.cuda.synchronize()
    gd = F.dequant("mxfp8", gc, gs, axis=-2)[0]
    assert_close(dw, O.linear_dw(gd, xd[0]), f"native mx dW {M}x{N}x{K}")


def test_native_mx_dw_matches_decode_path_with_nan_blocks(lp):
    """A gradient block with scale 0xFF makes the same dW rows NaN
    in the block-scaled path as in the decode path (grad decoded to bf16)."""
    M, N, K = 512, 256, 288
    gbits = W.bf16_bits(W.normal_f32(49, "grad", (1, M, N), 1.0))
    gc, gs = F.mx_quant(gbits, -2, "e4m3")
    gs = gs.copy()
    gs[0, 3, 17] = 0xFF                          # rows 96..127 of grad column 17 -> dW row 17
    g = lp.QTensor("mxfp8", dev(gc[0]), dev(gs[0]), shape=(1, M, N), axis=-2)
    x, xd = _operand(lp, 49, "x", (M, K), "mxfp8", -2)
    _, dw_native = lp.lp_linear_bwd(g, x, None, need_dx=False)
    gq = lp.QTensor("bf16", lp.lp_dequant(g).view(M, N), shape=(1, M, N))
    _, dw_decode = lp.lp_linear_bwd(gq, x, None, need_dx=False)
    torch.cuda.synchronize()
    a = dw_native.float().cpu().numpy()
    b = dw_decode.float().cpu().numpy()
    assert np.array_equal(np.isnan(a), np.isnan(b))
    assert np.isnan(a[17]).all() and not np.isnan(np.delete(a, 17, 0)).any()
    keep = np.delete(np.arange(N), 17)
    gd = F.dequant("mxfp8", gc, gs, axis=-2)[0]
    assert_close(dw_native[torch.from_numpy(keep).cuda()], O.rows_dw(gd, xd[0], keep), "native dW, finite rows")


def _sentinel(shape):
    return torch.full(shape, -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)   # 0xFFFF (NaN)


@pytest.mark.parametrize("fmt,axis", [("bf16", -1), ("mxfp4", -1), ("fp8_b128", -1), ("nvfp4", -1), ("mxfp8", -2)])
def test_grouped_edges(lp, fmt, axis):
    """Five groups: an empty one, one smaller than a tile, ragged ends, and
    rows past the last offset that must keep their sentinel value.  bf16
    operands take the path that loads both tiles straight into LDS."""
    M, N, K, G = 700, 256, 320, 5
    sizes = [130, 0, 17, 300, 203]            # sum 650 < M: rows 650.. untouched
    offsets = W.cumulative_ends(sizes)
    g, gb = _grad(lp, 35, M, N)
    x, xd = _operand(lp, 35, "x", (M, K), fmt, -1 if axis == -2 else axis)
    w, wd = _operand(lp, 35, "w", (G, N, K), fmt, axis)
    off = torch.from_numpy(offsets).cuda()
    dx0 = _sentinel((M, K))
    dw0 = _sentinel((G, N, K))
    dx, dw = lp.lp_grouped_bwd(g, x, w, off, grad_x=dx0, grad_w=dw0)
    torch.cuda.synchronize()
    ref_dx, end = O.grouped_dx(gb, wd, offsets)
    ref_dw = O.grouped_dw(gb, xd[0], offsets)
    assert_close(dx[:end], ref_dx[:end], f"{fmt} grouped dX")
    assert np.all(bits_host(dx[end:]) == 0xFFFF), "rows past the last offset were written"
    assert_close(dw, ref_dw, f"{fmt} grouped dW")
    assert np.all(bits_host(dw[1]) == 0), "empty group's dW is not zero"


@pytest.mark.parametrize("sizes_kind", ["ties", "many"])
def test_grouped_orders(lp, sizes_kind):
    """Grouped dW tile orders: equal group sizes (the size ranking breaks ties
    by group index) and 300 groups (more than are ranked by size, so tiles
    are dealt round-robin), with empty groups among them."""
    if sizes_kind == "ties":
        sizes = [96, 96, 0, 96, 96, 96, 0, 96]
        M = 640
    else:
        g0 = W.rng(44, "route")
        sizes = g0.integers(0, 9, size=300)
        sizes[g0.choice(300, size=30, replace=False)] = 0
        M = int(sizes.sum()) + 20
    G = len(sizes)
    N, K = 128, 256
    offsets = W.cumulative_ends(np.asarray(sizes))
    g, gb = _grad(lp, 44, M, N)
    x, xd = _operand(lp, 44, "x", (M, K), "mxfp4", -1)
    w, wd = _operand(lp, 44, "w", (G, N, K), "mxfp4", -1)
    dx, dw = lp.lp_grouped_bwd(g, x, w, torch.from_numpy(offsets).cuda())
    torch.cuda.synchronize()
    ref_dx, end = O.grouped_dx(gb, wd, offsets)
    assert_close(dx[:end], ref_dx[:end], f"{sizes_kind} grouped dX")
    assert_close(dw, O.grouped_dw(gb, xd[0], offsets), f"{sizes_kind} grouped dW")


def test_grouped_one_group_equals_linear(lp):
    """One group spanning all rows gives bit-identical results to the linear
    backward (same kernels, same tile order)."""
    M, N, K = 600, 256, 512
    g, _ = _grad(lp, 36, M, N)
    x, _ = _operand(lp, 36, "x", (M, K), "mxfp4", -1)
    w, _ = _operand(lp, 36, "w", (1, N, K), "mxfp4", -1)
    off = torch.tensor([M], dtype=torch.int32, device="cuda")
    dx1, dw1 = lp.lp_grouped_bwd(g, x, w, off)
    dx2, dw2 = lp.lp_linear_bwd(g, x, w)
    torch.cuda.synchronize()
    assert_bits_equal(bits_host(dx1), bits_host(dx2), "dX")
    assert_bits_equal(bits_host(dw1)[0], bits_host(dw2), "dW")


def _group_slice(lp, q, gi):
    """Group gi of a grouped descriptor [G, R, C] as a [1, R, C] descriptor
    (copies, so that every pointer keeps the library's alignment)."""
    G, R, C = q.shape
    scales = q.scales.view(G, -1)[gi].clone() if q.scales is not None else None
    return lp.QTensor(q.fmt, q.codes.view(G, -1)[gi].clone(), scales, q.tensor_scale, shape=(1, R, C), axis=q.axis)


@pytest.mark.parametrize("fmt,K,sizes", [("mxfp4", 2048, [4000, 0, 4300, 1]), ("fp8_b128", 1904, [4000, 0, 4300, 1]),
                                         ("mxfp4", 2048, [7000, 0, 7800])])
def test_grouped_round_split(lp, fmt, K, sizes):
    """Grouped dX over a 4096-long contraction with more 256 x 256 tiles than
    one round of the 256 CUs.  Sizes 4000, 0, 4300, 1: 34 row tiles of 8
    column tiles, 272 tiles, 256 of them in whole rounds and the other 16 as
    256 x 128 tiles of a second launch (K = 1904 ends on a single 128-wide
    tile).  Sizes 7000, 0, 7800: 59 row tiles, 472 tiles, a last round of 216
    tiles, too many to split.  Bit-identical to a linear call per group,
    within the contraction tolerance of the oracle on sampled rows of every
    group, rows past the last offset kept."""
    N = 4096
    G = len(sizes)
    M = int(sum(sizes)) + 40
    offsets = W.cumulative_ends(sizes)
    g, gb = _grad(lp, 39, M, N)
    w, wd = _operand(lp, 39, "w", (G, N, K), fmt, -1)
    dx = lp.lp_grouped_bwd(g, None, w, torch.from_numpy(offsets).cuda(), need_dw=False,
                           grad_x=_sentinel((M, K)))[0]
    per = []
    for gi, (s0, e0) in enumerate(O.group_bounds(offsets)):
        if e0 > s0:
            gq = lp.QTensor("bf16", g.codes.view(M, N)[s0:e0], shape=(1, e0 - s0, N))
            per.append((gi, s0, e0, lp.lp_linear_bwd(gq, None, _group_slice(lp, w, gi), need_dw=False)[0]))
    torch.cuda.synchronize()
    for gi, s0, e0, d in per:
        assert_bits_equal(bits_host(dx[s0:e0]), bits_host(d), f"{fmt} group {gi} vs the linear call")
        rows = s0 + _sample_rows(e0 - s0, 24, 39 + gi)
        sel = torch.from_numpy(rows).cuda()
        assert_close(dx[sel], O.rows_dx(gb, wd[gi], rows), f"{fmt} group {gi}, sampled rows")
    end = int(offsets[-1])
    assert np.all(bits_host(dx[end:]) == 0xFFFF), "rows past the last offset were written"


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4"])
def test_grouped_pair_launch(lp, fmt):
    """Grouped dX + dW with FP4 X and W and more 256 x 256 tiles than compute
    units in both products (dX 34 row tiles x 8 column tiles, dW 4 groups x
    8 x 8 tiles) run as one launch, grad_X's tiles first: both results equal
    the dX-only and dW-only calls bit for bit (rows past the last offset
    kept, an empty group's grad_W zero) and the oracle on sampled rows."""
    sizes = [4000, 0, 4300, 1]
    G, N, K = len(sizes), 2048, 2048
    M = int(sum(sizes)) + 40
    offsets = W.cumulative_ends(sizes)
    off = torch.from_numpy(offsets).cuda()
    g, gb = _grad(lp, 49, M, N)
    x, xd = _operand(lp, 49, "x", (M, K), fmt, -1)
    w, wd = _operand(lp, 49, "w", (G, N, K), fmt, -1)
    dx, dw = lp.lp_grouped_bwd(g, x, w, off, grad_x=_sentinel((M, K)), grad_w=_sentinel((G, N, K)))
    dx1 = lp.lp_grouped_bwd(g, None, w, off, need_dw=False, grad_x=_sentinel((M, K)))[0]
    dw1 = lp.lp_grouped_bwd(g, x, None, off, need_dx=False, grad_w=_sentinel((G, N, K)))[1]
    torch.cuda.synchronize()
    assert_bits_equal(bits_host(dx), bits_host(dx1), f"{fmt} paired dX vs dX alone")
    assert_bits_equal(bits_host(dw), bits_host(dw1), f"{fmt} paired dW vs dW alone")
    end = int(offsets[-1])
    assert np.all(bits_host(dx[end:]) == 0xFFFF), "rows past the last offset were written"
    assert np.all(bits_host(dw[1]) == 0), "the empty group's dW is not zero"
    for gi, (s0, e0) in enumerate(O.group_bounds(offsets)):
        if e0 == s0:
            continue
        rows = s0 + _sample_rows(e0 - s0, 8, 49 + gi)
        assert_close(dx[torch.from_numpy(rows).cuda()], O.rows_dx(gb, wd[gi], rows), f"{fmt} group {gi} dX rows")
        nrows = _sample_rows(N, 8, 59 + gi)
        assert_close(dw[gi][torch.from_numpy(nrows).cuda()], O.rows_dw(gb[s0:e0], xd[0][s0:e0], nrows),
                     f"{fmt} group {gi} dW rows")


def test_grouped_pair_launch_many_groups(lp):
    """The one-launch grouped dX + dW with 300 groups (more than grad_W ranks
    by size, so its tiles are dealt round-robin), empty ones among them, and
    258 grad_X / 600 grad_W tiles of 256 x 256: both results equal the
    dX-only and dW-only calls bit for bit, and the oracle on sampled rows."""
    rng = W.rng(50, "route")
    sizes = rng.integers(0, 221, size=300)
    sizes[rng.choice(300, size=25, replace=False)] = 0
    M = int(sizes.sum())
    if (M + 255) // 256 < 129:                                 # keep 129 row tiles: 258 dX tiles
        sizes[0] += 129 * 256 - 255 - M
        M = int(sizes.sum())
    M += 20
    G, N, K = len(sizes), 256, 512
    offsets = W.cumulative_ends(sizes)
    off = torch.from_numpy(offsets).cuda()
    g, gb = _grad(lp, 50, M, N)
    x, xd = _operand(lp, 50, "x", (M, K), "mxfp4", -1)
    w, wd = _operand(lp, 50, "w", (G, N, K), "mxfp4", -1)
    dx, dw = lp.lp_grouped_bwd(g, x, w, off)
    dx1 = lp.lp_grouped_bwd(g, None, w, off, need_dw=False)[0]
    dw1 = lp.lp_grouped_bwd(g, x, None, off, need_dx=False)[1]
    torch.cuda.synchronize()
    end = int(offsets[-1])
    assert_bits_equal(bits_host(dx[:end]), bits_host(dx1[:end]), "paired dX vs dX alone")
    assert_bits_equal(bits_host(dw), bits_host(dw1), "paired dW vs dW alone")
    bounds = O.group_bounds(offsets)
    for gi in [int(i) for i in np.flatnonzero(sizes)[::37]]:
        s0, e0 = bounds[gi]
        rows = s0 + _sample_rows(e0 - s0, 4, 60 + gi)
        assert_close(dx[torch.from_numpy(rows).cuda()], O.rows_dx(gb, wd[gi], rows), f"group {gi} dX rows")
        nrows = _sample_rows(N, 4, 70 + gi)
        assert_close(dw[gi][torch.from_numpy(nrows).cuda()], O.rows_dw(gb[s0:e0], xd[0][s0:e0], nrows),
                     f"group {gi} dW rows")
    for gi in np.flatnonzero(sizes == 0)[:5]:
        assert np.all(bits_host(dw[int(gi)]) == 0), f"empty group {gi}'s dW is not zero"


def test_grouped_bad_offsets_are_clamped(lp):
    """Offsets out of order or past M are clamped (end_g = clamp(o_g,
    end_{g-1}, M)): the kernels stay in bounds and compute those groups."""
    M, N, K, G = 256, 128, 256, 4
    offsets = np.array([100, 40, 9999, 300], dtype=np.int32)   # -> ends 100, 100, 256, 256
    g, gb = _grad(lp, 37, M, N)
    x, xd = _operand(lp, 37, "x", (M, K), "bf16", -1)
    w, wd = _operand(lp, 37, "w", (G, N, K), "bf16", -1)
    dx, dw = lp.lp_grouped_bwd(g, x, w, torch.from_numpy(offsets).cuda())
    torch.cuda.synchronize()
    clamped = np.array([100, 100, 256, 256], dtype=np.int32)
    assert_close(dx, O.grouped_dx(gb, wd, clamped)[0], "dX")
    assert_close(dw, O.grouped_dw(gb, xd[0], clamped), "dW")


def test_empty_tokens(lp):
    g = lp.QTensor("bf16", torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"), shape=(1, 0, 128))
    w, _ = _operand(lp, 38, "w", (128, 64), "mxfp4", -1)
    dx, _ = lp.lp_linear_bwd(g, None, w, need_dw=False)
    assert dx.shape == (0, 64)


# ------------------------------------------------------------------ full sizes, sampled

def _sample_rows(n, k, seed):
    return np.sort(W.rng(seed, "x").choice(n, size=min(k, n), replace=False))


def test_fp8_frozen_full_size(lp):
    """4096 x 8192 grad, 8192 x 2048 E4M3 weight: dX, 64 sampled rows (the
    256 x 128 tiles fill the GPU, so no workspace is asked for)."""
    w = W.WORKLOADS["fp8_frozen"]
    X, Wt, G = W.dense_inputs(w)
    wq, wd = quantize(lp, "fp8_b128", Wt)
    g = lp.QTensor("bf16", bf16_dev(G), shape=(1, w.M, w.N))
    assert lp.lp_linear_bwd_workspace(g, None, wq, True, False) == 0
    dx, _ = lp.lp_linear_bwd(g, None, wq, need_dw=False)
    torch.cuda.synchronize()
    rows = _sample_rows(w.M, 64, 40)
    assert_close(dx[torch.from_numpy(rows).cuda()], O.rows_dx(G, wd[0], rows), "fp8 frozen dX")


def test_fp8_frozen_full_size_two_step(lp):
    """The benchmark's form of the same step: lp_dequant of the weight to a
    bf16 copy, then dX against it (bf16 x bf16, both operands loaded straight
    into LDS).  Bit-identical to the fused decode, and 64 sampled rows against
    the oracle."""
    w = W.WORKLOADS["fp8_frozen"]
    X, Wt, G = W.dense_inputs(w)
    wq, wd = quantize(lp, "fp8_b128", Wt)
    g = lp.QTensor("bf16", bf16_dev(G), shape=(1, w.M, w.N))
    wbf = lp.lp_dequant(wq)
    dx2, _ = lp.lp_linear_bwd(g, None, lp.QTensor("bf16", wbf, shape=(1, w.N, w.K)), need_dw=False)
    dx1, _ = lp.lp_linear_bwd(g, None, wq, need_dw=False)
    torch.cuda.synchronize()
    assert torch.equal(dx1, dx2), "two-step dX differs from the fused decode"
    rows = _sample_rows(w.M, 64, 41)
    assert_close(dx2[torch.from_numpy(rows).cuda()], O.rows_dx(G, wd[0], rows), "fp8 frozen dX, two-step")


def test_split_dw_full_contraction(lp):
    """A low-rank-adapter-sized dW: N = 256, K = 512 over all 16384 tokens of
    an NVFP4 input (two 256 x 256 tiles, 256 slabs in 16 splits); 32 sampled
    rows of dW against the oracle."""
    M, N, K = 16384, 256, 512
    g, gb = _grad(lp, 39, M, N)
    x, xd = _operand(lp, 39, "x", (M, K), "nvfp4", -1)
    ws = _workspace(lp, g, x, None, need_dx=False)
    _, dw = lp.lp_linear_bwd(g, x, None, need_dx=False, workspace=ws)
    torch.cuda.synchronize()
    _counters_zero(ws, 2)
    nrows = _sample_rows(N, 32, 43)
    assert_close(dw[torch.from_numpy(nrows).cuda()], O.rows_dw(gb, xd[0], nrows), "split dW 16384 tokens")


def test_nvfp4_linear_full_size(lp):
    """8192 x 4096 NVFP4 X and 4096 x 4096 NVFP4 W: dX and dW, sampled rows."""
    w = W.WORKLOADS["nvfp4_linear"]
    X, Wt, G = W.dense_inputs(w)
    xq, xd = quantize(lp, "nvfp4", X)
    wq, wd = quantize(lp, "nvfp4", Wt)
    g = lp.QTensor("bf16", bf16_dev(G), shape=(1, w.M, w.N))
    dx, dw = lp.lp_linear_bwd(g, xq, wq)
    torch.cuda.synchronize()
    rows = _sample_rows(w.M, 48, 41)
    assert_close(dx[torch.from_numpy(rows).cuda()], O.rows_dx(G, wd[0], rows), "nvfp4 dX")
    nrows = _sample_rows(w.N, 48, 42)
    assert_close(dw[torch.from_numpy(nrows).cuda()], O.rows_dw(G, xd[0], nrows), "nvfp4 dW")


def test_mxfp4_grouped_full_size(lp):
    """8 experts, 16384 tokens routed by Dirichlet(1): grouped dX and dW,
    sampled rows of every group."""
    w = W.WORKLOADS["mxfp4_grouped"]
    X, Wt, G = W.dense_inputs(w)
    offsets = W.cumulative_ends(W.group_sizes(w))
    xq, xd = quantize(lp, "mxfp4", X)
    wq, wd = quantize(lp, "mxfp4", Wt)
    g = lp.QTensor("bf16", bf16_dev(G), shape=(1, w.M, w.N))
    dx, dw = lp.lp_grouped_bwd(g, xq, wq, torch.from_numpy(offsets).cuda())
    torch.cuda.synchronize()
    for gi, (s, e) in enumerate(O.group_bounds(offsets)):
        if e == s:
            continue
        rows = s + _sample_rows(e - s, 8, 43 + gi)
        assert_close(dx[torch.from_numpy(rows).cuda()], O.rows_dx(G, wd[gi], rows), f"group {gi} dX")
        nrows = _sample_rows(w.N, 6, 60 + gi)
        ref = O.rows_dw(G[s:e], xd[0][s:e], nrows)
        assert_close(dw[gi][torch.from_numpy(nrows).cuda()], ref, f"group {gi} dW")


def test_mxfp4_grouped_forced_empty_full_size(lp):
    """The 8-expert MXFP4 grouped layer at full size with one expert's
    tokens all moved to the largest (an empty group inside the offsets):
    its grad_W is all zeros, and sampled rows of every other group's dX and
    dW (the grown group's included) match the oracle."""
    w = W.WORKLOADS["mxfp4_grouped"]
    X, Wt, G = W.dense_inputs(w)
    sizes = W.group_sizes(w)
    empty = int(np.argmin(sizes))
    sizes = W.force_empty(sizes, empty)
    assert sizes[empty] == 0 and sizes.sum() == w.M
    offsets = W.cumulative_ends(sizes)
    xq, xd = quantize(lp, "mxfp4", X)
    wq, wd = quantize(lp, "mxfp4", Wt)
    g = lp.QTensor("bf16", bf16_dev(G), shape=(1, w.M, w.N))
    dx, dw = lp.lp_grouped_bwd(g, xq, wq, torch.from_numpy(offsets).cuda())
    torch.cuda.synchronize()
    assert not torch.any(dw[empty].view(torch.int16) != 0), "the emptied group's dW is not all zeros"
    for gi, (s, e) in enumerate(O.group_bounds(offsets)):
        if e == s:
            continue
        rows = s + _sample_rows(e - s, 8, 143 + gi)
        assert_close(dx[torch.from_numpy(rows).cuda()], O.rows_dx(G, wd[gi], rows), f"group {gi} dX")
        nrows = _sample_rows(w.N, 6, 160 + gi)
        ref = O.rows_dw(G[s:e], xd[0][s:e], nrows)
        assert_close(dw[gi][torch.from_numpy(nrows).cuda()], ref, f"group {gi} dW")


def test_mxfp8_deferred_full_size(lp):
    """64 experts, 32768 tokens with Zipf(1.1) sizes: the GPU quantizes grad
    (along -1) and W (along the reduction axis) and runs grouped dX.  Every
    non-empty expert is checked on 3 sampled rows x 96 sampled output
    columns against the oracle's own quantization of the same bf16 inputs
    (a column of W quantized along the reduction axis depends on that
    column alone), and the two largest experts on 8 whole rows."""
    w = W.WORKLOADS["mxfp8_deferred"]
    offsets = W.cumulative_ends(W.group_sizes(w))
    Wt = W.torch_normal_bf16((w.groups, w.N, w.K), w.w_sigma, seed=5005, device="cuda")
    Gt = W.torch_normal_bf16((w.M, w.N), 1.0, seed=5006, device="cuda")
    gq = lp.lp_mx_quant(Gt, -1, "mxfp8")
    wq = lp.lp_mx_quant(Wt, -2, "mxfp8")
    gq.shape = (1, w.M, w.N)
    dx, _ = lp.lp_grouped_bwd(gq, None, wq, torch.from_numpy(offsets).cuda(), need_dw=False)
    torch.cuda.synchronize()
    bounds = O.group_bounds(offsets)
    sizes = np.diff([0] + list(offsets))
    biggest = set(int(i) for i in np.argsort(-sizes)[:2])
    cols = np.sort(W.rng(44, "x").choice(w.K, 96, replace=False))
    tcols = torch.from_numpy(cols).cuda()
    checked = 0
    for gi, (s, e) in enumerate(bounds):
        if e == s:
            continue
        full = gi in biggest
        rows = s + _sample_rows(e - s, 8 if full else 3, 45 + gi)
        trows = torch.from_numpy(rows).cuda()
        gbits = Gt[trows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        gc, gs = F.mx_quant(gbits[None], -1, "e4m3")
        g_deq = F.dequant("mxfp8", gc, gs, axis=-1)[0]
        wsel = Wt[gi] if full else Wt[gi][:, tcols]
        wbits = wsel.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        wc, ws = F.mx_quant(wbits[None], -2, "e4m3")
        w_deq = F.dequant("mxfp8", wc, ws, axis=-2)[0]
        got = dx[trows] if full else dx[trows][:, tcols]
        assert_close(got, O.linear_dx(g_deq, w_deq), f"expert {gi} dX")
        checked += 1
    assert checked == int((sizes > 0).sum())


def test_mxfp8_dense_full_size(lp):
    """The dense deferred MXFP8 backward at 8192 tokens x 4096 x 4096: the GPU
    quantizes grad along both axes and W, X along their rows, then runs dX and
    dW on the block-scaled MFMA.  Sampled outputs (rows x columns) are checked
    against the oracle's own quantization of the same bf16 inputs; every
    quantization involved is local to the sampled rows or columns."""
    w = W.WORKLOADS["mxfp8_dense"]
    M, N, K = w.M, w.N, w.K
    Gt = W.torch_normal_bf16((M, N), 1.0, seed=6006, device="cuda")
    Wt = W.torch_normal_bf16((N, K), w.w_sigma, seed=6007, device="cuda")
    Xt = W.torch_normal_bf16((M, K), 1.0, seed=6008, device="cuda")
    gc, gr = lp.lp_mx_quant_dual(Gt, "mxfp8")
    wq = lp.lp_mx_quant(Wt, -2, "mxfp8")
    xq = lp.lp_mx_quant(Xt, -2, "mxfp8")
    dx, _ = lp.lp_linear_bwd(gc, None, wq, need_dw=False)
    _, dw = lp.lp_linear_bwd(gr, xq, None, need_dx=False)
    torch.cuda.synchronize()

    def host(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    rows, cols = _sample_rows(M, 16, 50), _sample_rows(K, 32, 51)
    ic = torch.from_numpy(cols).cuda()
    g = host(Gt[torch.from_numpy(rows).cuda()])
    gq, gs = F.mx_quant(g[None], -1, "e4m3")
    wcol = host(Wt[:, ic])
    wc, ws = F.mx_quant(wcol[None], -2, "e4m3")
    ref = O.linear_dx(F.dequant("mxfp8", gq, gs, axis=-1)[0], F.dequant("mxfp8", wc, ws, axis=-2)[0])
    assert_close(dx[torch.from_numpy(rows).cuda()][:, ic], ref, "mxfp8 dense dX")

    nrows = _sample_rows(N, 16, 52)
    gcol = host(Gt[:, torch.from_numpy(nrows).cuda()])
    gq, gs = F.mx_quant(gcol[None], -2, "e4m3")
    xcol = host(Xt[:, ic])
    xc, xs = F.mx_quant(xcol[None], -2, "e4m3")
    ref = O.linear_dw(F.dequant("mxfp8", gq, gs, axis=-2)[0], F.dequant("mxfp8", xc, xs, axis=-2)[0])
    assert_close(dw[torch.from_numpy(nrows).cuda()][:, ic], ref, "mxfp8 dense dW")


def test_mxfp8_persistent_partial_tiles(lp):
    """The persistent block-scaled grad_X (more output tiles than compute
    units: 17 x 17 = 289 here) with a ragged last row tile (M = 4133) and a
    partial last column tile (K = 4160, 64 columns past 16 tiles of 256),
    dense and grouped (five groups with ragged ends, an empty one, sentinel
    rows past the last offset), on sampled rows and every column of the
    partial tile against the oracle."""
    M, N, K = 4133, 1024, 4160
    Gt = W.torch_normal_bf16((M, N), 1.0, seed=6106, device="cuda")
    Wt = W.torch_normal_bf16((3, N, K), 0.02, seed=6107, device="cuda")
    gc = lp.lp_mx_quant(Gt, -1, "mxfp8")
    gc.shape = (1, M, N)
    wq = lp.lp_mx_quant(Wt, -2, "mxfp8")

    def host(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    rows = np.unique(np.concatenate([_sample_rows(M, 12, 60), [M - 1, 4095, 4096]]))
    cols = np.unique(np.concatenate([_sample_rows(K, 24, 61), np.arange(4096, K)]))
    ic = torch.from_numpy(cols).cuda()
    g = host(Gt[torch.from_numpy(rows).cuda()])
    gq, gs = F.mx_quant(g[None], -1, "e4m3")
    gd = F.dequant("mxfp8", gq, gs, axis=-1)[0]
    wd = []
    for e in range(3):
        wc, ws = F.mx_quant(host(Wt[e][:, ic])[None], -2, "e4m3")
        wd.append(F.dequant("mxfp8", wc, ws, axis=-2)[0])

    w1 = lp.QTensor("mxfp8", wq.codes[:1], wq.scales[:1], shape=(1, N, K), axis=-2)
    dx, _ = lp.lp_linear_bwd(gc, None, w1, need_dw=False)
    torch.cuda.synchronize()
    assert_close(dx[torch.from_numpy(rows).cuda()][:, ic], O.linear_dx(gd, wd[0]), "dense persistent dX")

    # four groups; group 3 reuses expert 0's weight (a copy)
    sizes = [1500, 0, 1201, 900]
    ends = W.cumulative_ends(sizes)
    wq4 = lp.QTensor("mxfp8", torch.cat([wq.codes, wq.codes[:1]]), torch.cat([wq.scales, wq.scales[:1]]),
                     shape=(4, N, K), axis=-2)
    sent = torch.full((M, K), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    dxg, _ = lp.lp_grouped_bwd(gc, None, wq4, dev(ends), need_dw=False, grad_x=sent)
    torch.cuda.synchronize()
    for gi, (s0, e0) in enumerate(O.group_bounds(ends)):
        sel = (rows >= s0) & (rows < e0)
        if not sel.any():
            continue
        ref = O.linear_dx(gd[sel], wd[gi if gi < 3 else 0])
        r = torch.from_numpy(rows[sel]).cuda()
        assert_close(dxg[r][:, ic], ref, f"grouped persistent dX, group {gi}")
    tail = rows[rows >= int(ends[-1])]
    assert (host(dxg[torch.from_numpy(tail).cuda()]) == 0xFFFF).all(), "rows past the last offset were written"
