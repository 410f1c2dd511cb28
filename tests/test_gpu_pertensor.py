"""Per-tensor scaled FP8 (the AstrAI page's hybrid E4M3 / E5M2 recipe) on the
GPU against oracle/pertensor.py: amax, scale from history, quantization and
decoding bit for bit; the dX / dW products (dense and grouped) within the
contraction tolerance."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_bits_equal, assert_close, bf16_dev, bits_host, dev
from oracle import pertensor as PT

pytestmark = pytest.mark.gpu

ELEM = {"fp8t_e4m3": "e4m3", "fp8t_e5m2": "e5m2"}


def _f32_dev(x) -> torch.Tensor:
    return torch.tensor(np.asarray(x, dtype=np.float32).reshape(-1), device="cuda")


def _f32_bits(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def _same_f32(got: torch.Tensor, want, what: str):
    g = got.cpu().numpy().astype(np.float32).reshape(-1)
    w = np.asarray(want, dtype=np.float32).reshape(-1)
    nan_ok = np.isnan(g) & np.isnan(w)
    bad = (g.view(np.uint32) != w.view(np.uint32)) & ~nan_ok
    assert not bad.any(), f"{what}: got {g[bad][:4]}, want {w[bad][:4]}"


def _every_bf16() -> np.ndarray:
    """Every bf16 bit pattern once (NaNs and infinities included), shuffled."""
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    W.rng(30, "x").shuffle(b)
    return b


@pytest.mark.parametrize("fmt", ["fp8t_e4m3", "fp8t_e5m2"])
@pytest.mark.parametrize("scale", [1.0, 0.01234, 3.0517578e-05, 1e-12, 7.5e3])
def test_quant_every_bf16(lp, fmt, scale):
    bits = _every_bf16()
    s = _f32_dev([scale])
    amax = torch.full((1,), -1.0, device="cuda")
    q = lp.lp_tensor_quant(bf16_dev(bits).view(256, 256), fmt, s, amax=amax)
    torch.cuda.synchronize()
    want = PT.quantize(bits, ELEM[fmt], np.float32(scale))
    assert_bits_equal(q.codes.cpu().numpy().reshape(-1), want, f"{fmt} codes at scale {scale}")
    assert np.isnan(amax.item()), "a NaN input makes the amax NaN"


def _scales_across_ranges() -> np.ndarray:
    """Random fp32 scales, log-uniform over 2^-80 .. 2^100 with random
    mantissas, plus the ends of that range and their neighbours outside it,
    and a few far outside (the quantizer forms its quotients differently
    inside and outside the range)."""
    g = W.rng(39, "w")
    e = g.uniform(-80.0, 100.0, 48)
    r = (2.0 ** e).astype(np.float32)
    r = (r.view(np.uint32) ^ (g.integers(0, 1 << 23, 48, dtype=np.uint32))).view(np.float32)
    edges = np.array([2.0 ** -80, 2.0 ** 100, 1e-12, 1e30, 2.0 ** -100, 2.0 ** 120], np.float32)
    near = np.concatenate([np.nextafter(edges[:2], np.float32(0)), np.nextafter(edges[:2], np.float32(np.inf))])
    return np.concatenate([r, edges, near.astype(np.float32)])


@pytest.mark.parametrize("fmt", ["fp8t_e4m3", "fp8t_e5m2"])
def test_quant_every_bf16_many_scales(lp, fmt):
    """Every bf16 value at 58 scales, against fp32 IEEE division on the host."""
    bits = _every_bf16()
    src = bf16_dev(bits)
    for scale in _scales_across_ranges():
        q = lp.lp_tensor_quant(src, fmt, _f32_dev([scale]))
        torch.cuda.synchronize()
        assert_bits_equal(q.codes.cpu().numpy().reshape(-1), PT.quantize(bits, ELEM[fmt], scale),
                          f"{fmt} codes at scale {scale!r}")


@pytest.mark.parametrize("fmt", ["fp8t_e4m3", "fp8t_e5m2"])
@pytest.mark.parametrize("scale", [1.0, 0.37, 1e-12, 2.0 ** -140, 3.0e38, 0.0, float("nan")])
def test_dequant_every_code(lp, fmt, scale):
    codes = np.tile(np.arange(256, dtype=np.uint8), 4).reshape(16, 64)
    q = lp.QTensor(fmt, dev(codes), None, _f32_dev([scale]), shape=(1, 16, 64))
    out = lp.lp_dequant(q)
    torch.cuda.synchronize()
    want = PT.dequant(codes, ELEM[fmt], np.float32(scale))
    assert_bits_equal(bits_host(out).reshape(16, 64), want, f"{fmt} decode at scale {scale}")


@pytest.mark.parametrize("n", [8, 1000, 8192, 65536 * 3 + 40, 1 << 22])
def test_amax_sizes(lp, n):
    x = W.normal_f32(31, "x", (n,), 2.0)
    x[n // 3] = -1000.5                      # the largest magnitude is negative
    bits = W.bf16_bits(x)
    got = lp.lp_tensor_amax(bf16_dev(bits))
    torch.cuda.synchronize()
    _same_f32(got, PT.amax(bits), f"amax of {n}")


def test_amax_special(lp):
    z = np.zeros(64, np.uint16)
    _same_f32(lp.lp_tensor_amax(bf16_dev(z)), 0.0, "all zeros")
    z[5] = 0x8000
    _same_f32(lp.lp_tensor_amax(bf16_dev(z)), 0.0, "signed zero")
    z[9] = 0xFF80                            # -inf
    _same_f32(lp.lp_tensor_amax(bf16_dev(z)), np.inf, "-inf")
    z[11] = 0xFFC1                           # a negative NaN
    assert np.isnan(lp.lp_tensor_amax(bf16_dev(z)).item())
    z = np.full(64, 0x0001, np.uint16)      # smallest subnormal
    _same_f32(lp.lp_tensor_amax(bf16_dev(z)), PT.amax(z), "subnormal")
    empty = torch.empty(0, dtype=torch.bfloat16, device="cuda")
    amax = torch.full((1,), 5.0, device="cuda")
    lp.lp_tensor_amax(empty, amax)
    _same_f32(amax, 0.0, "empty tensor")


@pytest.mark.parametrize("fmt", ["fp8t_e4m3", "fp8t_e5m2"])
@pytest.mark.parametrize("length,margin", [(1, 0), (16, 0), (16, 2), (1024, -3), (65536, 1), (300, 64), (5, -64)])
def test_scale_from_history(lp, fmt, length, margin):
    g = W.rng(32, "w")
    hist = (g.random(length).astype(np.float32) * np.float32(10.0) ** g.integers(-8, 6, length)).astype(np.float32)
    got = lp.lp_scale_from_history(_f32_dev(hist), fmt, margin)
    _same_f32(got, PT.scale_from_history(hist, ELEM[fmt], margin), f"{fmt} len {length} margin {margin}")


def test_scale_from_history_special(lp):
    for hist, what in (([0.0] * 16, "zero history -> floor"), ([1e-20], "tiny -> floor"),
                       ([3.0, float("inf")], "inf"), ([1.0, float("nan"), 2.0], "NaN")):
        for fmt in ELEM:
            got = lp.lp_scale_from_history(_f32_dev(hist), fmt, 0)
            _same_f32(got, PT.scale_from_history(np.asarray(hist, np.float32), ELEM[fmt], 0), f"{what} {fmt}")


def test_quant_records_amax_into_ring_slot(lp):
    """Delayed scaling: quantize with the ring's scale and record the amax in
    slot idx, in one call; the other slots are untouched."""
    x = W.normal_f32(33, "grad", (96, 64), 1e-3)
    bits = W.bf16_bits(x)
    hist = np.array([2e-3, 5e-3, 1e-3, 4e-3], np.float32)
    ring = _f32_dev(hist)
    scale = lp.lp_scale_from_history(ring, "fp8t_e5m2")
    idx = 2
    q = lp.lp_tensor_quant(bf16_dev(bits), "fp8t_e5m2", scale, amax=ring[idx:idx + 1])
    torch.cuda.synchronize()
    want_scale = PT.scale_from_history(hist, "e5m2")
    want_hist = hist.copy()
    PT.record(want_hist, idx, PT.amax(bits))
    _same_f32(scale, want_scale, "ring scale")
    _same_f32(ring, want_hist, "ring after record")
    assert_bits_equal(q.codes.cpu().numpy().reshape(-1), PT.quantize(bits, "e5m2", want_scale).reshape(-1), "codes")


@pytest.mark.parametrize("fmt", ["fp8t_e5m2", "fp8t_e4m3"])
def test_quant_delayed_equals_scale_then_quant(lp, fmt):
    """20 delayed-scaling steps on a 16-entry ring: the one-call step and the
    two-call sequence agree bit for bit (codes, scale, ring) every step, and
    the first step equals the oracle's."""
    L, shape = W.AMAX_RING, (96, 512)
    ring_a = torch.zeros(L, device="cuda")
    first = W.bf16_bits(W.normal_f32(47, "grad", shape, 1e-3))
    ring_a.copy_(torch.tensor([PT.amax(first)] * L, device="cuda"))
    ring_b = ring_a.clone()
    hist = ring_a.cpu().numpy().copy()
    for step in range(20):
        bits = W.bf16_bits(W.normal_f32(47, "grad", shape, 10.0 ** ((step % 7) - 4)))
        src = bf16_dev(bits)
        slot = step % L
        qa = lp.lp_tensor_quant_delayed(src, fmt, ring_a, slot)
        sb = lp.lp_scale_from_history(ring_b, fmt)
        qb = lp.lp_tensor_quant(src, fmt, sb, amax=ring_b[slot:slot + 1])
        torch.cuda.synchronize()
        assert torch.equal(qa.codes, qb.codes), f"codes differ at step {step}"
        assert torch.equal(qa.tensor_scale.view(torch.int32), sb.view(torch.int32)), f"scale differs at step {step}"
        assert torch.equal(ring_a.view(torch.int32), ring_b.view(torch.int32)), f"ring differs at step {step}"
        if step == 0:
            s = PT.scale_from_history(hist, ELEM[fmt])
            _same_f32(qa.tensor_scale, s, "oracle scale")
            assert_bits_equal(qa.codes.cpu().numpy().reshape(shape), PT.quantize(bits, ELEM[fmt], s), "oracle codes")
            PT.record(hist, slot, PT.amax(bits))
            _same_f32(ring_a, hist, "oracle ring")


def _pt_operand(lp, number, tensor, shape, sigma, fmt, outliers=False):
    """bf16 values -> the oracle's per-tensor codes with the dynamic scale of
    their amax; returns (descriptor on the GPU, codes, scale)."""
    v = W.normal_f32(number, tensor, shape, sigma)
    if outliers:
        v = W.with_outliers(v, number, tensor)
    bits = W.bf16_bits(v)
    s = PT.scale_from_history([PT.amax(bits)], ELEM[fmt])
    codes = PT.quantize(bits, ELEM[fmt], s)
    shp = (1,) + tuple(shape) if len(shape) == 2 else tuple(shape)
    return lp.QTensor(fmt, dev(codes.reshape(shp)), None, _f32_dev([s]), shape=shp), codes, s


FMT_PAIRS = [("fp8t_e5m2", "fp8t_e4m3"), ("fp8t_e4m3", "fp8t_e4m3"), ("fp8t_e4m3", "fp8t_e5m2"),
             ("fp8t_e5m2", "fp8t_e5m2")]


@pytest.mark.parametrize("gfmt,ofmt", FMT_PAIRS)
@pytest.mark.parametrize("M,N,K", [(300, 272, 400), (64, 16, 16), (513, 1040, 272), (1, 48, 512)])
def test_linear_dx_dw(lp, gfmt, ofmt, M, N, K):
    g, gc, gs = _pt_operand(lp, 34, "grad", (M, N), 1e-3, gfmt, outliers=True)
    w, wc, ws = _pt_operand(lp, 34, "w", (N, K), 0.02, ofmt)
    x, xc, xs = _pt_operand(lp, 34, "x", (M, K), 1.0, ofmt, outliers=True)
    dx, dw = lp.lp_linear_bwd(g, x, w)
    torch.cuda.synchronize()
    assert_close(dx, PT.linear_dx(gc, ELEM[gfmt], gs, wc, ELEM[ofmt], ws), f"dX {gfmt}x{ofmt} {M}x{N}x{K}")
    assert_close(dw, PT.linear_dw(gc, ELEM[gfmt], gs, xc, ELEM[ofmt], xs), f"dW {gfmt}x{ofmt} {M}x{N}x{K}")


def test_linear_x_and_w_in_different_formats(lp):
    """X and W of different per-tensor formats: the two products are launched
    one after the other instead of together; same results as the oracle."""
    M, N, K = 300, 272, 400
    g, gc, gs = _pt_operand(lp, 48, "grad", (M, N), 1e-3, "fp8t_e5m2")
    w, wc, ws = _pt_operand(lp, 48, "w", (N, K), 0.02, "fp8t_e4m3")
    x, xc, xs = _pt_operand(lp, 48, "x", (M, K), 1.0, "fp8t_e5m2")
    dx, dw = lp.lp_linear_bwd(g, x, w)
    torch.cuda.synchronize()
    assert_close(dx, PT.linear_dx(gc, "e5m2", gs, wc, "e4m3", ws), "dX, W in E4M3")
    assert_close(dw, PT.linear_dw(gc, "e5m2", gs, xc, "e5m2", xs), "dW, X in E5M2")


def test_linear_each_output_alone(lp):
    M, N, K = 320, 256, 288
    g, gc, gs = _pt_operand(lp, 35, "grad", (M, N), 1e-3, "fp8t_e5m2")
    w, wc, ws = _pt_operand(lp, 35, "w", (N, K), 0.02, "fp8t_e4m3")
    x, xc, xs = _pt_operand(lp, 35, "x", (M, K), 1.0, "fp8t_e4m3")
    dx, none = lp.lp_linear_bwd(g, None, w, need_dw=False)
    assert none is None
    none, dw = lp.lp_linear_bwd(g, x, None, need_dx=False)
    assert none is None
    torch.cuda.synchronize()
    assert_close(dx, PT.linear_dx(gc, "e5m2", gs, wc, "e4m3", ws), "dX alone")
    assert_close(dw, PT.linear_dw(gc, "e5m2", gs, xc, "e4m3", xs), "dW alone")


@pytest.mark.parametrize("sizes", [[100, 0, 300, 37, 1], [0, 0, 513], [256, 256]])
def test_grouped(lp, sizes):
    G, N, K = len(sizes), 272, 320
    M = int(sum(sizes)) + 29                             # rows past the last end stay unwritten
    ends = W.cumulative_ends(sizes)
    g, gc, gs = _pt_operand(lp, 36, "grad", (M, N), 1e-3, "fp8t_e5m2")
    w, wc, ws = _pt_operand(lp, 36, "w", (G, N, K), 0.02, "fp8t_e4m3")
    x, xc, xs = _pt_operand(lp, 36, "x", (M, K), 1.0, "fp8t_e4m3")
    sentinel = torch.full((M, K), 7.0, dtype=torch.bfloat16, device="cuda")
    dx, dw = lp.lp_grouped_bwd(g, x, w, dev(ends), grad_x=sentinel)
    torch.cuda.synchronize()
    start = 0
    for e, end in enumerate(ends):
        rows = slice(start, int(end))
        if end > start:
            assert_close(dx[rows], PT.linear_dx(gc[rows], "e5m2", gs, wc[e], "e4m3", ws), f"dX group {e}")
        ref_w = PT.linear_dw(gc[rows], "e5m2", gs, xc[rows], "e4m3", xs)
        if end > start:
            assert_close(dw[e], ref_w, f"dW group {e}")
        else:
            assert not dw[e].float().abs().any(), f"empty group {e} must get zeros"
        start = int(end)
    assert (dx[int(ends[-1]):].float() == 7.0).all(), "rows past the last end are not written"


def test_rejects_mixed_formats(lp):
    g, _, _ = _pt_operand(lp, 37, "grad", (64, 64), 1e-3, "fp8t_e5m2")
    wb = lp.QTensor("bf16", torch.zeros((1, 64, 64), dtype=torch.bfloat16, device="cuda"), shape=(1, 64, 64))
    with pytest.raises(lp.LpError, match="LP_ERR_FORMAT"):
        lp.lp_linear_bwd(g, None, wb, need_dw=False)
    gb = lp.QTensor("bf16", torch.zeros((1, 64, 64), dtype=torch.bfloat16, device="cuda"), shape=(1, 64, 64))
    w, _, _ = _pt_operand(lp, 37, "w", (64, 64), 0.02, "fp8t_e4m3")
    with pytest.raises(lp.LpError, match="LP_ERR_FORMAT"):
        lp.lp_linear_bwd(gb, None, w, need_dw=False)


def test_hybrid_step_dynamic_scaling(lp):
    """The page's backward step on the device: amax of the bf16 gradient ->
    dynamic scale -> E5M2 codes (amax recorded once more by the quantizer) ->
    dX and dW against E4M3 saved operands, every stage against the oracle."""
    M, N, K = 512, 384, 256
    gbits = W.bf16_bits(W.normal_f32(38, "grad", (M, N), 1e-4))
    w, wc, ws = _pt_operand(lp, 38, "w", (N, K), 0.02, "fp8t_e4m3")
    x, xc, xs = _pt_operand(lp, 38, "x", (M, K), 1.0, "fp8t_e4m3")
    gdev = bf16_dev(gbits)
    amax = lp.lp_tensor_amax(gdev)
    scale = lp.lp_scale_from_history(amax, "fp8t_e5m2")
    rec = torch.empty(1, device="cuda")
    g = lp.lp_tensor_quant(gdev, "fp8t_e5m2", scale, amax=rec)
    dx, dw = lp.lp_linear_bwd(g, x, w)
    torch.cuda.synchronize()
    a = PT.amax(gbits)
    s = PT.scale_from_history([a], "e5m2")
    codes = PT.quantize(gbits, "e5m2", s)
    _same_f32(amax, a, "amax")
    _same_f32(rec, a, "recorded amax")
    _same_f32(scale, s, "scale")
    assert_bits_equal(g.codes.cpu().numpy().reshape(M, N), codes, "gradient codes")
    assert_close(dx, PT.linear_dx(codes, "e5m2", s, wc, "e4m3", ws), "dX")
    assert_close(dw, PT.linear_dw(codes, "e5m2", s, xc, "e4m3", xs), "dW")


def test_fp8_hybrid_full_size(lp):
    """The benchmark's workload at full size, through the same calls: every
    code of the three quantizations against the oracle, then sampled rows of
    dX and dW (all tiles' row and column ranges, the last rows included)."""
    w = W.WORKLOADS["fp8_hybrid"]
    M, N, K = w.M, w.N, w.K
    gb = W.bf16_bits(W.normal_f32(w.number, "grad", (M, N), 1.0))
    xb = W.bf16_bits(W.normal_f32(w.number, "x", (M, K), w.x_sigma))
    wb = W.bf16_bits(W.normal_f32(w.number, "w", (N, K), w.w_sigma))
    ops = {}
    for name, bits, fmt in (("grad", gb, "fp8t_e5m2"), ("x", xb, "fp8t_e4m3"), ("w", wb, "fp8t_e4m3")):
        t = bf16_dev(bits)
        hist = torch.empty(W.AMAX_RING, device="cuda")
        hist.copy_(lp.lp_tensor_amax(t).expand(W.AMAX_RING))
        scale = lp.lp_scale_from_history(hist, fmt)
        q = lp.lp_tensor_quant(t, fmt, scale, amax=hist[3:4])
        torch.cuda.synchronize()
        a = PT.amax(bits)
        s = PT.scale_from_history(np.full(W.AMAX_RING, a, np.float32), ELEM[fmt])
        codes = PT.quantize(bits, ELEM[fmt], s)
        _same_f32(scale, s, f"{name} scale")
        _same_f32(hist[3:4], a, f"{name} recorded amax")
        assert_bits_equal(q.codes.cpu().numpy().reshape(bits.shape), codes, f"{name} codes")
        ops[name] = (q, codes, s)
    (gq, gc, gs), (xq, xc, xs), (wq, wc, ws) = ops["grad"], ops["x"], ops["w"]
    dx, _ = lp.lp_linear_bwd(gq, None, wq, need_dw=False)
    _, dw = lp.lp_linear_bwd(gq, xq, None, need_dx=False)
    torch.cuda.synchronize()
    rs = np.unique(np.concatenate([np.arange(0, M, 61), [M - 1]]))
    ns = np.unique(np.concatenate([np.arange(0, N, 97), [N - 1]]))
    assert_close(dx[torch.from_numpy(rs).cuda()], PT.linear_dx(gc[rs], "e5m2", gs, wc, "e4m3", ws), "dX rows")
    assert_close(dw[torch.from_numpy(ns).cuda()], PT.linear_dw(gc[:, ns], "e5m2", gs, xc, "e4m3", xs), "dW rows")
