"""Pins of the CPU oracle to things other than itself.

Each `pin_*` function raises AssertionError when the oracle disagrees with
the format definitions, an independent library (torch's CPU casts and
ops), a closed form, a brute-force search or a structural invariant of the
method.  `test_oracle_pins.py` runs them; `test_oracle_mutations.py` plants
plausible mistakes in the oracle and checks that some pin fails.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import workloads as W
from oracle import formats as F
from oracle import gemm as O
from oracle import pertensor as PT

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def _bits_f32(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def _torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).bfloat16() \
        .view(torch.int16).numpy().view(np.uint16)


def _same_bits_or_both_nan(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.all((a == b) & (np.signbit(a) == np.signbit(b)) | (np.isnan(a) & np.isnan(b)))


# ------------------------------------------------------------------ element tables

def pin_e4m3_table():
    """All 256 E4M3 codes against torch's CPU float8_e4m3fn decode; max 448
    (AstrAI FP8_MAX)."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert _same_bits_or_both_nan(F.E4M3_TABLE, ref), "E4M3 table differs from torch"
    assert np.nanmax(F.E4M3_TABLE) == GOLDEN["e4m3_max"]["value"]
    assert F.E4M3_TABLE[0x7E] == 448.0 and np.isnan(F.E4M3_TABLE[0x7F]) and np.isnan(F.E4M3_TABLE[0xFF])
    assert F.E4M3_TABLE[0x01] == 2.0 ** -9 and F.E4M3_TABLE[0x08] == 2.0 ** -6


def pin_e8m0_table():
    """All 256 E8M0 codes against torch's CPU float8_e8m0fnu decode."""
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    assert _same_bits_or_both_nan(F.E8M0_TABLE, ref), "E8M0 table differs from torch"
    assert F.E8M0_TABLE[127] == 1.0 and F.E8M0_TABLE[0] == 2.0 ** -127


def pin_e2m1_table():
    """The 16 E2M1 codes against the OCP value list; eight distinct
    magnitudes, as the FP4 page states."""
    ocp = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    expect = np.array(ocp + [-v for v in ocp])
    assert _same_bits_or_both_nan(F.E2M1_TABLE, expect), "E2M1 table differs from the OCP list"
    assert len(set(np.abs(F.E2M1_TABLE).tolist())) == GOLDEN["e2m1_magnitudes"]["value"]


# ------------------------------------------------------------------ rounding

def pin_bf16_rounding():
    """fp32 -> bf16 RNE against torch's CPU cast on every high half with
    low halves at and around the tie; NaN gives 0x7FC0 with the sign."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    f = _bits_f32(u)
    ok = ~np.isnan(f)
    got = F.f32_to_bf16_bits(f[ok])
    ref = _torch_bf16_bits(f[ok])
    assert np.array_equal(got, ref), "bf16 rounding differs from torch"
    nan = F.f32_to_bf16_bits(np.array([np.nan, -np.nan], dtype=np.float32))
    assert nan[0] in (0x7FC0, 0xFFC0) and (nan[0] & 0x7FFF) == 0x7FC0
    signed = F.f32_to_bf16_bits(np.array([np.nan, np.nan], dtype=np.float32), nan_sign=np.array([0, 1]))
    assert list(signed) == [0x7FC0, 0xFFC0]


def _all_bf16_finite() -> np.ndarray:
    b = np.arange(1 << 16, dtype=np.uint32) << 16
    f = _bits_f32(b)
    return f[np.isfinite(f)].astype(np.float64)


def pin_e4m3_rounding():
    """RNE onto the E4M3 grid against torch's float8_e4m3fn cast for every
    finite bf16 value below 464 in magnitude (torch does not saturate beyond
    that point); at and above 448 the oracle saturates to +-448."""
    v = _all_bf16_finite()
    small = np.abs(v) < 464
    got = F.round_to_grid(v[small], "e4m3")
    ref = torch.from_numpy(v[small].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref), "E4M3 rounding differs from torch"
    big = F.round_to_grid(v[~small], "e4m3")
    assert np.all((big & 0x7F) == 0x7E), "E4M3 does not saturate to 448"
    assert np.all((big >> 7) == np.signbit(v[~small]))


def _brute_nearest(t: np.ndarray, table: np.ndarray, sign_bit: int) -> np.ndarray:
    """Brute force: distance to every finite non-negative grid point, the
    nearest wins, a tie goes to the code with a clear last bit."""
    codes = np.array([c for c in range(sign_bit) if np.isfinite(table[c])])
    vals = table[codes]
    a = np.abs(t)[:, None]
    d = np.abs(a - vals[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    top = np.argmax(vals)
    pick = np.where(np.abs(t) >= vals[top], top, pick)
    out = codes[pick]
    return np.where(np.signbit(t), out | sign_bit, out).astype(np.uint8)


def pin_e2m1_rounding():
    """RNE onto the E2M1 grid against a brute-force nearest search over a
    dense set of points including every midpoint, and the tie table
    0.25->0, 0.75->1, 1.25->1, 1.75->2, 2.5->2, 3.5->4, 5->4, 7->6."""
    t = np.concatenate([np.arange(-8, 8, 1 / 64), np.arange(0, 8, 0.25) + 1 / 1024, [1e30, -1e30]])
    got = F.round_to_grid(t, "e2m1")
    ref = _brute_nearest(t, F.E2M1_TABLE, 0x8)
    assert np.array_equal(got, ref), "E2M1 rounding differs from brute force"
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])
    expect = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0]
    assert F.E2M1_TABLE[F.round_to_grid(ties, "e2m1")].tolist() == expect


def pin_e4m3_brute():
    """E4M3 rounding against brute force, including values far past the
    saturation point and subnormal midpoints."""
    t = np.concatenate([np.arange(0, 16, 2.0 ** -10), np.linspace(-600, 600, 4001), [1e9, -1e9]])
    assert np.array_equal(F.round_to_grid(t, "e4m3"), _brute_nearest(t, F.E4M3_TABLE, 0x80))


# ------------------------------------------------------------------ dequant

def _torch_decode_e4m3(codes_u8: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes_u8)).view(torch.float8_e4m3fn).float()


def _torch_decode_e8m0(codes_u8: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes_u8)).view(torch.float8_e8m0fnu).float()


def _bits_equal_nan_aware(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.asarray(a, np.uint16)
    b = np.asarray(b, np.uint16)
    an = ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
    bn = ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    return bool(np.all(np.where(an | bn, an & bn, a == b)))


def pin_fp8_b128_dequant():
    """FP8 block dequant as the FP8-adapter page's own test writes it:
    weight.float() * scale repeated over 128x128 blocks (cut at the edge),
    in fp32 torch ops, then torch's bf16 cast; partial blocks included."""
    g = W.rng(90, "w")
    R, C = 300, 200
    codes = g.integers(0, 256, size=(R, C), dtype=np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x10
    scale = (g.random((3, 2), dtype=np.float32) * 2 + 0.5).astype(np.float32)
    got = F.dequant(F.FMT_FP8_B128, codes, scale)[0]
    s = torch.from_numpy(scale).repeat_interleave(128, dim=0)[:R].repeat_interleave(128, dim=1)[:, :C]
    ref = (_torch_decode_e4m3(codes) * s).bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert _bits_equal_nan_aware(got, ref), "FP8 block dequant differs from the page's formulation"


def pin_fp8_b128_page_rounding():
    """The page's implementation rounds the scale to bf16 before a bf16
    multiply; the reading taken (one fp32 multiply, then bf16) stays within
    two bf16 ulps of it."""
    g = W.rng(91, "w")
    codes = g.integers(0, 0x7E, size=(256, 256), dtype=np.uint8)
    scale = (g.random((2, 2), dtype=np.float32) + 0.5).astype(np.float32)
    ours = F.bf16_bits_to_f64(F.dequant(F.FMT_FP8_B128, codes, scale)[0])
    s = torch.from_numpy(scale).bfloat16().repeat_interleave(128, 0).repeat_interleave(128, 1)
    page = (_torch_decode_e4m3(codes).bfloat16() * s).double().numpy()
    ulp = np.maximum(np.abs(page), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(ours - page) <= 2 * ulp)


def pin_mxfp8_dequant():
    """MXFP8 dequant against torch: float8_e4m3fn x float8_e8m0fnu in fp32,
    then bf16; both scale axes."""
    g = W.rng(92, "w")
    R, C = 64, 96
    codes = g.integers(0, 256, size=(R, C), dtype=np.uint8)
    for axis in (-1, -2):
        shape = (R, C // 32) if axis == -1 else (R // 32, C)
        sc = g.integers(100, 150, size=shape, dtype=np.uint8)
        sc.flat[0] = 0xFF
        got = F.dequant(F.FMT_MXFP8, codes, sc, axis=axis)[0]
        s = _torch_decode_e8m0(sc)
        s = s.repeat_interleave(32, dim=1) if axis == -1 else s.repeat_interleave(32, dim=0)
        ref = (_torch_decode_e4m3(codes) * s).bfloat16().view(torch.int16).numpy().view(np.uint16)
        assert _bits_equal_nan_aware(got, ref), f"MXFP8 axis {axis} differs from torch"


def pin_fp4_dequant_closed_forms():
    """Hand-built packed blocks: byte 0x21 is [0.5, 1.0] (low nibble first);
    MXFP4 scale byte 130 multiplies by 8; NVFP4 code 1.0 with block scale
    E4M3 2.0 (0x40) and tensor scale 0.25 is 0.5; an E8M0 NaN scale makes
    NaN."""
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 1] = 0xF7                                      # [6, -6]
    mx = F.bf16_bits_to_f64(F.dequant(F.FMT_MXFP4, codes, np.array([[127]], np.uint8))[0])
    assert mx[0, :4].tolist() == [0.5, 1.0, 6.0, -6.0]
    mx8 = F.bf16_bits_to_f64(F.dequant(F.FMT_MXFP4, codes, np.array([[130]], np.uint8))[0])
    assert mx8[0, :4].tolist() == [4.0, 8.0, 48.0, -48.0]
    nan = F.dequant(F.FMT_MXFP4, codes, np.array([[255]], np.uint8))[0]
    assert np.all((nan & 0x7FFF) == 0x7FC0)
    nv_codes = np.full((1, 8), 0x22, dtype=np.uint8)       # all 1.0
    nv_scale = np.array([[0x40]], dtype=np.uint8)          # E4M3 2.0
    nv = F.bf16_bits_to_f64(F.dequant(F.FMT_NVFP4, nv_codes, nv_scale, np.float32(0.25))[0])
    assert np.all(nv == 0.5)


def pin_nvfp4_dequant_torch():
    """NVFP4 dequant against torch ops: the block scale (torch E4M3 decode)
    times the tensor scale in fp32, times the E2M1 value (OCP list) in fp32,
    then bf16."""
    g = W.rng(93, "w")
    R, C = 32, 64
    packed = g.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
    sc = g.integers(0, 0x7F, size=(R, C // 16), dtype=np.uint8)
    ts = np.float32(0.0173)
    got = F.dequant(F.FMT_NVFP4, packed, sc, ts)[0]
    ocp = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])
    p = torch.from_numpy(packed).long()
    vals = torch.stack([ocp[p & 15], ocp[p >> 4]], dim=-1).reshape(R, C)
    S = (_torch_decode_e4m3(sc) * torch.tensor(ts)).repeat_interleave(16, dim=1)
    ref = (vals * S).bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref), "NVFP4 dequant differs from torch"


# ------------------------------------------------------------------ MX quant

def pin_mx_scale_rule():
    """A block whose amax is exactly 448 * 2^5 (E4M3) or 6 * 2^5 (E2M1) gets
    scale byte 127 + 5 and its codes back unchanged."""
    g = W.rng(94, "x")
    for elem, table, top in (("e4m3", F.E4M3_TABLE, 0x7E), ("e2m1", F.E2M1_TABLE, 0x7)):
        n = 256 if elem == "e4m3" else 16
        pool = np.array([c for c in range(n) if np.isfinite(table[c])])
        codes = g.choice(pool, size=32).astype(np.uint8)
        codes[3] = top
        vals = (table[codes] * 32.0).astype(np.float32)
        q, s = F.mx_quant(W.bf16_bits(vals[None, :]), -1, elem)
        assert s.reshape(-1)[0] == 132, (elem, s)
        qc = F.unpack_e2m1(q)[0, 0] if elem == "e2m1" else q[0, 0]
        assert np.array_equal(table[qc], table[codes])


def pin_mx_invariants():
    """For random blocks across magnitudes (bf16 subnormals included): the
    scaled amax lies in [2^emax, 2^(emax+1)) unless clamped; quantizing the
    dequantized result returns the same bytes; the error is within half a
    grid step of the top binade, or the clipped excess for saturated elements;
    axis -2 equals axis -1 on the transpose."""
    g = W.rng(95, "x")
    mags = np.exp2(g.integers(-140, 120, size=(64, 1))).astype(np.float32)
    x = (g.standard_normal((64, 64)).astype(np.float32) * mags)
    bits = W.bf16_bits(x)
    v = F.bf16_bits_to_f64(bits)
    for elem, emax, fmt in (("e4m3", 8, F.FMT_MXFP8), ("e2m1", 2, F.FMT_MXFP4)):
        q, s = F.mx_quant(bits, -1, elem)
        amax = np.abs(v.reshape(64, 2, 32)).max(-1)
        e = s[0].astype(np.int64) - 127
        scaled = amax / np.exp2(e.astype(np.float64))
        ok = (e > -127) & (amax > 0)
        assert np.all((scaled[ok] >= 2.0 ** emax) & (scaled[ok] < 2.0 ** (emax + 1)))
        deq = F.dequant(fmt, q, s, axis=-1)
        q2, s2 = F.mx_quant(deq, -1, elem)
        assert np.array_equal(q, q2) and np.array_equal(s, s2), f"{elem} not idempotent"
        dv = F.bf16_bits_to_f64(deq[0])
        step = np.exp2(e.astype(np.float64))[:, :, None] * (2.0 ** (emax - 3 if elem == "e4m3" else emax - 1))
        err = np.abs(dv - v).reshape(64, 2, 32)
        top = 448.0 if elem == "e4m3" else 6.0
        sat = np.abs(v).reshape(64, 2, 32) - top * np.exp2(e.astype(np.float64))[:, :, None]
        bound = np.maximum(step / 2, sat) * (1 + 1e-12) + 2.0 ** -133
        assert np.all(err[ok] <= bound[ok])
        qT, sT = F.mx_quant(np.ascontiguousarray(bits.T), -2, elem)
        if elem == "e4m3":
            assert np.array_equal(qT[0].T, q[0]) and np.array_equal(sT[0].T, s[0])
        else:
            assert np.array_equal(sT[0].T, s[0])


def pin_mx_special_blocks():
    """All-zero block -> scale 0 and signed zero codes; a NaN or an infinity
    -> scale 0xFF and NaN codes (E4M3); a block of bf16 subnormals clamps the
    exponent at -127."""
    z = np.zeros((1, 32), np.float32)
    z[0, 1] = -0.0
    q, s = F.mx_quant(W.bf16_bits(z), -1, "e4m3")
    assert s[0, 0, 0] == 0 and q[0, 0, 0] == 0 and q[0, 0, 1] == 0x80
    n = np.ones((1, 32), np.float32)
    n[0, 5] = np.nan
    n[0, 6] = -1
    q, s = F.mx_quant(W.bf16_bits(n), -1, "e4m3")
    assert s[0, 0, 0] == 0xFF and q[0, 0, 0] == 0x7F and q[0, 0, 6] == 0xFF
    i = np.ones((1, 32), np.float32)
    i[0, 0] = np.inf
    assert F.mx_quant(W.bf16_bits(i), -1, "e2m1")[1][0, 0, 0] == 0xFF
    tiny = np.full((1, 32), 2.0 ** -130, np.float32)
    q, s = F.mx_quant(W.bf16_bits(tiny), -1, "e4m3")
    assert s[0, 0, 0] == 0
    assert F.E4M3_TABLE[q[0, 0, 0]] * 2.0 ** -127 == 2.0 ** -130


# ------------------------------------------------------------------ contractions

def _tiny_bf16(number, tensor, shape):
    return W.bf16_bits(W.normal_f32(number, tensor, shape, 1.0))


def pin_gemm_brute_force():
    """dX and dW against pure-Python triple loops on tiny shapes."""
    M, N, K = 5, 7, 3
    g = _tiny_bf16(96, "grad", (M, N))
    w = _tiny_bf16(96, "w", (N, K))
    x = _tiny_bf16(96, "x", (M, K))
    gv, wv, xv = (F.bf16_bits_to_f64(a).tolist() for a in (g, w, x))
    dx = [[sum(gv[m][n] * wv[n][k] for n in range(N)) for k in range(K)] for m in range(M)]
    dw = [[sum(gv[m][n] * xv[m][k] for m in range(M)) for k in range(K)] for n in range(N)]
    assert np.allclose(O.linear_dx(g, w), dx, rtol=1e-13, atol=0)
    assert np.allclose(O.linear_dw(g, x), dw, rtol=1e-13, atol=0)


def pin_gemm_transpose_identity():
    """dW(grad, X) equals dX(grad^T, X): the two contractions agree on which
    operand is transposed."""
    g = _tiny_bf16(97, "grad", (33, 17))
    x = _tiny_bf16(97, "x", (33, 9))
    assert np.allclose(O.linear_dw(g, x), O.linear_dx(np.ascontiguousarray(g.T), x), rtol=1e-13)


def _page_fp8_weight(number, rows, cols, grid, low):
    g = W.rng(number, "w")
    w = torch.from_numpy(g.standard_normal((rows, cols)).astype(np.float32)).to(torch.float8_e4m3fn)
    scale = torch.from_numpy(g.random(grid).astype(np.float32) + np.float32(low))
    return w.view(torch.uint8).numpy(), scale.numpy()


def pin_fp8_adapter_linear_closed_form():
    """The FP8-adapter page's linear test: with grad_out all ones, every row
    of grad_X equals ones @ (W.float() * scale) within rtol 1e-2, atol 1e-1."""
    c = GOLDEN["fp8_linear_test"]
    codes, scale = _page_fp8_weight(98, c["out_features"], c["in_features"], tuple(c["scale_grid"]), c["scale_low"])
    wd = F.dequant(F.FMT_FP8_B128, codes, scale)[0]
    ones = W.bf16_bits(np.ones((c["tokens"], c["out_features"]), np.float32))
    got = O.linear_dx(ones, wd)
    s = torch.from_numpy(scale).repeat_interleave(128, 0).repeat_interleave(128, 1)
    expected = torch.ones(c["tokens"], c["out_features"]) @ (_torch_decode_e4m3(codes) * s)
    torch.testing.assert_close(torch.from_numpy(got).float(), expected, rtol=c["rtol"], atol=c["atol"])


def pin_fp8_adapter_grouped_closed_form():
    """The FP8-adapter page's grouped test: 2 groups of 3 tokens, W 512x256
    viewed as 2 x 256 x 256; with ones as grad_out each token's grad_X is
    ones @ W_deq[its group]."""
    c = GOLDEN["fp8_grouped_test"]
    G, tpg = c["groups"], c["tokens_per_group"]
    codes, scale = _page_fp8_weight(99, c["out_features"], c["in_features"], tuple(c["scale_grid"]), c["scale_low"])
    per = c["out_features"] // G
    wd = np.stack([F.dequant(F.FMT_FP8_B128, codes[g * per:(g + 1) * per],
                             scale[g * per // 128:(g + 1) * per // 128])[0] for g in range(G)])
    offsets = np.arange(1, G + 1, dtype=np.int32) * tpg
    ones = W.bf16_bits(np.ones((G * tpg, per), np.float32))
    got, _ = O.grouped_dx(ones, wd, offsets)
    s = torch.from_numpy(scale).repeat_interleave(128, 0).repeat_interleave(128, 1)
    weight = (_torch_decode_e4m3(codes) * s).view(G, per, c["in_features"])
    expected = (torch.ones(tpg, G, 1, per) @ weight).squeeze(2)      # [token, group, K]
    expected = expected.permute(1, 0, 2).reshape(G * tpg, -1)
    torch.testing.assert_close(torch.from_numpy(got).float(), expected, rtol=c["rtol"], atol=c["atol"])


def pin_grouped_equals_dense():
    """Grouped dX / dW equal the per-group dense results stacked; an empty
    group gets dW = 0; rows past the last offset are not written; one group
    spanning all rows equals the linear backward."""
    M, N, K, G = 40, 24, 16, 4
    g = _tiny_bf16(100, "grad", (M, N))
    x = _tiny_bf16(100, "x", (M, K))
    w = _tiny_bf16(100, "w", (G, N, K))
    offsets = np.array([7, 7, 30, 36], dtype=np.int32)      # group 1 empty, rows 36.. untouched
    dx, end = O.grouped_dx(g, w, offsets)
    dw = O.grouped_dw(g, x, offsets)
    assert end == 36 and np.all(np.isnan(dx[36:]))
    bounds = [(0, 7), (7, 7), (7, 30), (30, 36)]
    for gi, (s, e) in enumerate(bounds):
        if e > s:
            assert np.allclose(dx[s:e], O.linear_dx(g[s:e], w[gi]), rtol=1e-13)
            assert np.allclose(dw[gi], O.linear_dw(g[s:e], x[s:e]), rtol=1e-13)
    assert np.all(dw[1] == 0)
    one_dx, _ = O.grouped_dx(g, w[:1], np.array([M], np.int32))
    assert np.allclose(one_dx, O.linear_dx(g, w[0]), rtol=1e-13)


# ------------------------------------------------------------------ per-tensor FP8 ("AstrAI fp8.py")

def pin_fp8_max_table_matches_page():
    assert PT.FP8_MAX["e4m3"] == GOLDEN["e4m3_max"]["value"]
    assert PT.FP8_MAX["e5m2"] == GOLDEN["e5m2_max"]["value"]
    for elem in ("e4m3", "e5m2"):
        t = PT.TABLES[elem]
        assert np.nanmax(np.where(np.isinf(t), np.nan, t)) == PT.FP8_MAX[elem]


def pin_e5m2_table_against_torch():
    """All 256 E5M2 codes against torch's float8_e5m2 decode."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).double().numpy()
    assert _same_bits_or_both_nan(PT.E5M2_TABLE, ref)
    assert np.isinf(PT.E5M2_TABLE[0x7C]) and np.isnan(PT.E5M2_TABLE[0x7D])


def pin_tensor_quantize_against_torch():
    """Every finite bf16 value x, several scales: codes equal torch's
    (x.float() / scale).to(float8) wherever the quotient is below the
    format's maximum (torch does not saturate, so larger ones are left to
    the saturation pin)."""
    b = np.arange(1 << 16, dtype=np.uint32)
    bits = b[((b >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    xf = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float()
    for elem, dt in (("e4m3", torch.float8_e4m3fn), ("e5m2", torch.float8_e5m2)):
        for scale in (1.0, 0.0173, 3.0e-3, 97.0, 2.0 ** -20):
            q = (xf / torch.tensor(scale, dtype=torch.float32))
            ok = (q.abs() <= PT.FP8_MAX[elem]).numpy()
            ref = q.to(dt).view(torch.uint8).numpy()
            got = PT.quantize(bits, elem, np.float32(scale))
            assert np.array_equal(got[ok], ref[ok]), (elem, scale)


def pin_tensor_quantize_saturates():
    """Brute force: beyond the maximum (infinities included) the code is the
    signed maximum; NaN keeps its sign on the 0x7F pattern; otherwise the
    code is the nearest value by exhaustive search, ties to the even code."""
    for elem in ("e4m3", "e5m2"):
        mx = PT.FP8_MAX[elem]
        t = np.array([mx * 1.01, -mx * 4, np.inf, -np.inf, np.nan, -np.nan, mx, -0.0, 0.0])
        c = PT.round_to_fp8(t, elem)
        vals = PT.TABLES[elem]
        assert vals[c[0]] == mx and vals[c[1]] == -mx and vals[c[2]] == mx and vals[c[3]] == -mx
        assert c[4] == 0x7F and c[5] == 0xFF and vals[c[6]] == mx and c[7] == 0x80 and c[8] == 0x00
        g = W.rng(60, "x")
        r = g.standard_normal(4000) * g.choice([1e-6, 1e-3, 1.0, 10.0, 100.0, 1e4], 4000)
        r = r[np.abs(r) < mx]
        codes = PT.round_to_fp8(r, elem)
        fin = np.arange(256)[np.isfinite(vals)]
        d = np.abs(r[:, None] - vals[fin][None, :])
        best = d.min(axis=1)
        got = np.abs(r - vals[codes])
        assert np.array_equal(got, best)


def pin_scale_from_history_formula():
    """scale = (max(history) / FP8_MAX) / 2^margin, at least 1e-12
    (fp32), as the page's DelayedScaling / DynamicScaling define it."""
    assert PT.scale_from_history([1.0, 57344.0, 2.0], "e5m2") == np.float32(1.0)
    assert PT.scale_from_history([57344.0], "e5m2", margin=2) == np.float32(0.25)
    assert PT.scale_from_history([448.0, 3.0], "e4m3") == np.float32(1.0)
    assert PT.scale_from_history([0.0, 0.0], "e4m3") == np.float32(1e-12)
    s = PT.scale_from_history([7.25], "e4m3", margin=1)
    assert s == np.float32(np.float32(7.25 / 448.0) / 2)
    hist = np.ones(4, np.float32)
    i = 0
    for v in (5.0, 9.0, 2.0, 3.0, 4.0):
        i = PT.record(hist, i, v)
    assert i == 1 and list(hist) == [4.0, 9.0, 2.0, 3.0]
    assert PT.scale_from_history(hist, "e5m2") == np.float32(np.float32(9.0) / np.float32(57344.0))


def pin_tensor_amax_and_dequant():
    bits = W.bf16_bits(np.array([1.5, -7.0, 0.25, -0.0], dtype=np.float32))
    assert PT.amax(bits) == np.float32(7.0)
    assert np.isnan(PT.amax(np.array([0x3F80, 0x7FC0], dtype=np.uint16)))
    # E5M2 0x3C = 1.0, 0x42 = 3.0, 0xBF = -1.75; times 3.0 -> 3.0, 9.0, -5.25
    d = PT.dequant(np.array([0x3C, 0x42, 0xBF, 0x7F, 0xFF, 0x7C], dtype=np.uint8), "e5m2", 3.0)
    assert list(d) == [0x4040, 0x4110, 0xC0A8, 0x7FC0, 0xFFC0, 0x7F80]


def pin_tensor_gemms_brute_force():
    """Pure-Python triple loops with the scales applied to the sums."""
    g = W.rng(61, "grad")
    gc = g.integers(0, 256, size=(3, 5), dtype=np.uint8) & 0x7B          # finite E5M2 codes
    wc = g.integers(0, 256, size=(5, 4), dtype=np.uint8) & 0x77          # finite E4M3 codes
    xc = g.integers(0, 256, size=(3, 4), dtype=np.uint8) & 0x7B
    sg, sw, sx = 0.375, 1.5, 0.0625
    dx = PT.linear_dx(gc, "e5m2", sg, wc, "e4m3", sw)
    dw = PT.linear_dw(gc, "e5m2", sg, xc, "e5m2", sx)
    for m in range(3):
        for k in range(4):
            acc = 0.0
            for n in range(5):
                acc += PT.e5m2_value(int(gc[m, n])) * sg * F.e4m3_value(int(wc[n, k])) * sw
            assert abs(dx[m, k] - acc) <= 1e-12 * max(1.0, abs(acc))
    for n in range(5):
        for k in range(4):
            acc = 0.0
            for m in range(3):
                acc += PT.e5m2_value(int(gc[m, n])) * sg * PT.e5m2_value(int(xc[m, k])) * sx
            assert abs(dw[n, k] - acc) <= 1e-12 * max(1.0, abs(acc))


# ------------------------------------------------------------------ forward (FP4 page; Deferred-MXFP8 page)

def pin_forward_triple_loop_and_adjoint():
    """y = x @ W^T against a pure-Python triple loop, and the adjoint identity
    that ties the forward to the backward: sum(y * g) = sum(x * grad_X) for
    grad_X = g @ W, and = sum(W * grad_W) for grad_W = g^T @ x.  A transposed
    operand in either direction breaks one of them."""
    M, N, K = 3, 5, 4
    x = _tiny_bf16(102, "x", (M, K))
    w = _tiny_bf16(102, "w", (N, K))
    g = _tiny_bf16(102, "grad", (M, N))
    y = O.linear_fwd(x, w)
    xv, wv = F.bf16_bits_to_f64(x), F.bf16_bits_to_f64(w)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += float(xv[m, k]) * float(wv[n, k])
            assert abs(y[m, n] - acc) <= 1e-12 * max(1.0, abs(acc))
    gv = F.bf16_bits_to_f64(g)
    lhs = float(np.sum(y * gv))
    assert abs(lhs - float(np.sum(xv * O.linear_dx(g, w)))) <= 1e-12 * max(1.0, abs(lhs))
    assert abs(lhs - float(np.sum(wv * O.linear_dw(g, x)))) <= 1e-12 * max(1.0, abs(lhs))


def pin_grouped_forward_equals_dense():
    """Grouped forward equals the per-group dense forward; rows past the last
    offset stay unwritten; an empty group writes nothing."""
    M, N, K, G = 30, 8, 16, 3
    x = _tiny_bf16(103, "x", (M, K))
    w = _tiny_bf16(103, "w", (G, N, K))
    offsets = np.array([9, 9, 25], dtype=np.int32)
    y = O.grouped_fwd(x, w, offsets)
    assert np.all(np.isnan(y[25:]))
    assert np.allclose(y[0:9], O.linear_fwd(x[0:9], w[0]), rtol=1e-13)
    assert np.allclose(y[9:25], O.linear_fwd(x[9:25], w[2]), rtol=1e-13)


def _nv_scalar_decode(packed, scales, ts):
    """Element-by-element NVFP4 decode from the scalar code functions: low
    nibble = even column, one E4M3 scale per 16 columns, S = fp32(s * ts),
    value = bf16(fp32(code * S)) through torch's CPU casts."""
    packed = np.asarray(packed, dtype=np.uint8)
    R, C = packed.shape[0], packed.shape[1] * 2
    out = np.empty((R, C), dtype=np.float64)
    for r in range(R):
        for c in range(C):
            byte = int(packed[r, c // 2])
            code = byte & 0xF if c % 2 == 0 else byte >> 4
            S = float(np.float32(F.e4m3_value(int(scales[r, c // 16])) * float(np.float32(ts))))
            f = np.float32(F.e2m1_value(code) * S)
            out[r, c] = float(torch.tensor(float(f), dtype=torch.float32).bfloat16().double())
    return out


def pin_nvfp4_forward_scalar_loop():
    """NVFP4 forward against a triple loop over scalar-decoded operands, dense
    and grouped (an empty group; rows past the last offset unwritten), with
    distinct tensor scales so that dropping or swapping one shows."""
    M, N, K, G = 6, 4, 32, 3
    xc, xs, xts = F.quant_nvfp4(W.normal_f32(106, "x", (M, K), 1.0))
    wc, ws, wts = F.quant_nvfp4(W.normal_f32(106, "w", (G, N, K), 3.0))
    assert float(xts) != float(wts)
    xv = _nv_scalar_decode(xc[0], xs[0], xts)
    wv = [_nv_scalar_decode(wc[g], ws[g], wts) for g in range(G)]

    def loop(rows, wg):
        return np.array([[sum(xv[m, k] * wg[n, k] for k in range(K)) for n in range(N)] for m in rows])

    dense = O.nvfp4_fwd(xc[0], xs[0], xts, wc[:1], ws[:1], wts)
    assert dense.shape == (M, N)
    assert np.allclose(dense, loop(range(M), wv[0]), rtol=1e-12, atol=0), "dense NVFP4 forward"
    offsets = np.array([2, 2, 5], dtype=np.int32)
    y = O.nvfp4_fwd(xc[0], xs[0], xts, wc, ws, wts, offsets)
    assert np.allclose(y[0:2], loop(range(0, 2), wv[0]), rtol=1e-12, atol=0), "grouped NVFP4 forward, group 0"
    assert np.allclose(y[2:5], loop(range(2, 5), wv[2]), rtol=1e-12, atol=0), "grouped NVFP4 forward, group 2"
    assert np.all(np.isnan(y[5:]))


def pin_fp8_block_forward_page_formulation():
    """Block-FP8 forward on the FP8-adapter page's grouped test shapes (2
    groups, weight 512 x 256 viewed as 2 x 256 x 256, scale grid 4 x 2) and on
    a weight with partial 128-blocks: equal to the page's test formulation in
    torch (codes decoded by torch's float8_e4m3fn, times the scale grid
    repeated over 128 x 128 blocks and cut at the edge, rounded to bf16,
    contracted in float64), and tied to the backward by the adjoint identity
    sum(y * g) = sum(x * grad_X)."""
    c = GOLDEN["fp8_grouped_test"]
    G, tpg = c["groups"], c["tokens_per_group"]
    codes, scale = _page_fp8_weight(107, c["out_features"], c["in_features"], tuple(c["scale_grid"]), c["scale_low"])
    per = c["out_features"] // G
    wc = codes.reshape(G, per, c["in_features"])
    wsc = scale.reshape(G, per // 128, -1)
    x = _tiny_bf16(107, "x", (G * tpg + 2, c["in_features"]))        # two rows past the last offset
    offsets = np.arange(1, G + 1, dtype=np.int32) * tpg
    y = O.fp8_block_fwd(x, wc, wsc, offsets)
    s = torch.from_numpy(scale).repeat_interleave(128, 0).repeat_interleave(128, 1)
    wt = (_torch_decode_e4m3(codes) * s).bfloat16().double().view(G, per, -1)
    xt = torch.from_numpy(F.bf16_bits_to_f64(x))
    for g in range(G):
        ref = xt[g * tpg:(g + 1) * tpg] @ wt[g].T
        assert np.allclose(y[g * tpg:(g + 1) * tpg], ref.numpy(), rtol=1e-12, atol=0), f"group {g}"
    assert np.all(np.isnan(y[G * tpg:]))
    gr = _tiny_bf16(107, "grad", (G * tpg, per))
    wd = F.dequant(F.FMT_FP8_B128, wc, wsc)
    dx, _ = O.grouped_dx(gr, wd, offsets)
    lhs = float(np.sum(y[:G * tpg] * F.bf16_bits_to_f64(gr)))
    rhs = float(np.sum(F.bf16_bits_to_f64(x)[:G * tpg] * dx[:G * tpg]))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs)), "forward and backward disagree on orientation"
    # dense, partial blocks: 300 x 200 weight, 3 x 2 grid
    R, C = 300, 200
    codes2, scale2 = _page_fp8_weight(108, R, C, (3, 2), 0.5)
    x2 = _tiny_bf16(108, "x", (5, C))
    y2 = O.fp8_block_fwd(x2, codes2, scale2)
    s2 = torch.from_numpy(scale2).repeat_interleave(128, 0)[:R].repeat_interleave(128, 1)[:, :C]
    w2 = (_torch_decode_e4m3(codes2) * s2).bfloat16().double()
    ref2 = torch.from_numpy(F.bf16_bits_to_f64(x2)) @ w2.T
    assert np.allclose(y2, ref2.numpy(), rtol=1e-12, atol=0), "dense block-FP8 forward with partial blocks"


# ------------------------------------------------------------------ sampled and chunked paths

def pin_rows_dx_dw_brute_force():
    """The sampled contractions that full-size checks use: rows_dx on an
    unsorted row subset (one row twice) and rows_dw on an unsorted subset of
    n, against pure-Python triple loops and against the rows of the whole
    products."""
    M, N, K = 9, 7, 5
    g = _tiny_bf16(104, "grad", (M, N))
    w = _tiny_bf16(104, "w", (N, K))
    x = _tiny_bf16(104, "x", (M, K))
    gv, wv, xv = (F.bf16_bits_to_f64(a).tolist() for a in (g, w, x))
    rows = np.array([8, 0, 3, 3])
    ns = np.array([6, 1, 0])
    dx = [[sum(gv[m][n] * wv[n][k] for n in range(N)) for k in range(K)] for m in rows.tolist()]
    dw = [[sum(gv[m][n] * xv[m][k] for m in range(M)) for k in range(K)] for n in ns.tolist()]
    got_dx, got_dw = O.rows_dx(g, w, rows), O.rows_dw(g, x, ns)
    assert got_dx.shape == (len(rows), K) and got_dw.shape == (len(ns), K)
    assert np.allclose(got_dx, dx, rtol=1e-13, atol=0), "rows_dx differs from the triple loop"
    assert np.allclose(got_dw, dw, rtol=1e-13, atol=0), "rows_dw differs from the triple loop"
    assert np.allclose(got_dx, O.linear_dx(g, w)[rows], rtol=1e-13, atol=0)
    assert np.allclose(got_dw, O.linear_dw(g, x)[ns], rtol=1e-13, atol=0)


def pin_dequant_row_slabs():
    """Dequantization in row slabs: slabs of 32, 100 (rounded up to whole
    scale-block rows) and 128 rows give the same bits as one pass, and the
    slabbed FP8 block result equals the FP8-adapter page's formulation in
    torch (scale grid repeated over 128 x 128 blocks, cut at the edge) on a
    300-row tensor whose last block row is partial; MXFP8 scaled along the
    rows is checked against torch on 96 rows in slabs of 32."""
    g = W.rng(105, "w")
    R, C = 300, 200
    codes = g.integers(0, 256, size=(R, C), dtype=np.uint8)
    codes[codes & 0x7F == 0x7F] = 0x10
    scale = (g.random((3, 2), dtype=np.float32) * 2 + 0.5).astype(np.float32)
    whole = F.dequant(F.FMT_FP8_B128, codes, scale, chunk_rows=1 << 30)[0]
    s = torch.from_numpy(scale).repeat_interleave(128, dim=0)[:R].repeat_interleave(128, dim=1)[:, :C]
    ref = (_torch_decode_e4m3(codes) * s).bfloat16().view(torch.int16).numpy().view(np.uint16)
    for rows in (32, 100, 128):
        got = F.dequant(F.FMT_FP8_B128, codes, scale, chunk_rows=rows)[0]
        assert np.array_equal(got, whole), f"FP8 block dequant in slabs of {rows} rows differs"
        assert _bits_equal_nan_aware(got, ref), f"FP8 block dequant in slabs of {rows} rows differs from torch"
    R8, C8 = 96, 64
    c8 = g.integers(0, 256, size=(R8, C8), dtype=np.uint8)
    sc8 = g.integers(100, 150, size=(R8 // 32, C8), dtype=np.uint8)
    got8 = F.dequant(F.FMT_MXFP8, c8, sc8, axis=-2, chunk_rows=32)[0]
    ref8 = (_torch_decode_e4m3(c8) * _torch_decode_e8m0(sc8).repeat_interleave(32, dim=0))
    ref8 = ref8.bfloat16().view(torch.int16).numpy().view(np.uint16)
    assert _bits_equal_nan_aware(got8, ref8), "MXFP8 axis -2 dequant in slabs differs from torch"
    for fmt, ncols_s in ((F.FMT_MXFP4, 32), (F.FMT_NVFP4, 16)):
        packed = g.integers(0, 256, size=(70, 32), dtype=np.uint8)
        sc = g.integers(0, 0x7F if fmt == F.FMT_NVFP4 else 140, size=(70, 64 // ncols_s), dtype=np.uint8)
        ts = np.float32(0.37) if fmt == F.FMT_NVFP4 else None
        a = F.dequant(fmt, packed, sc, ts, chunk_rows=7)
        b = F.dequant(fmt, packed, sc, ts, chunk_rows=1 << 30)
        assert np.array_equal(a, b), f"{fmt} dequant in slabs of 7 rows differs"


def pin_mx_quant_chunks():
    """MX quantization in chunks of 3 blocks (the last one partial) gives
    the same codes and scales as one pass, on both axes and both element
    formats, with magnitudes spread over many binades."""
    g = W.rng(106, "x")
    mags = np.exp2(g.integers(-30, 30, size=(64, 1))).astype(np.float32)
    bits = W.bf16_bits(g.standard_normal((64, 160)).astype(np.float32) * mags)
    for axis in (-1, -2):
        for elem in ("e4m3", "e2m1"):
            q1, s1 = F.mx_quant(bits, axis, elem)
            q3, s3 = F.mx_quant(bits, axis, elem, chunk_blocks=3)
            assert np.array_equal(q1, q3) and np.array_equal(s1, s3), (axis, elem)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
