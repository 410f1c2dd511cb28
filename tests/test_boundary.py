"""The C-ABI library on the host: it loads, exports every function that
include/lp.h declares, and rejects bad arguments with the documented status
before touching the GPU (CPU only; no kernel is launched)."""
import ctypes

import pytest
import torch

import fp8_gemm_backward_amd as lp
from fp8_gemm_backward_amd import _QTensorC

OK, NULL, SHAPE, FORMAT, ALIGN = 0, 1, 2, 3, 4
FAKE = 0x10000          # 16-byte aligned stand-in pointer; never dereferenced here


def test_library_exports_every_header_function():
    names = lp.header_functions()
    assert set(names) == {"lp_dequant", "lp_mx_quant", "lp_linear_bwd", "lp_grouped_bwd", "lp_status_string",
                          "lp_linear_bwd_workspace", "lp_linear_bwd_ws", "lp_mx_quant_dual", "lp_tensor_amax",
                          "lp_tensor_quant", "lp_scale_from_history", "lp_linear_fwd", "lp_grouped_fwd",
                          "lp_tensor_quant_delayed", "lp_linear_bwd_noalloc", "lp_grouped_dx_deferred"}
    for n in names:
        assert hasattr(lp.lib, n), n


def test_status_strings():
    assert lp.lp_status_string(0) == "ok"
    for s in range(1, 6):
        assert lp.lp_status_string(s) not in ("ok", "unknown status")
    assert lp.lp_status_string(99) == "unknown status"


def q(fmt, rows, cols, batch=1, axis=-1, codes=FAKE, scales=FAKE, ts=FAKE):
    return _QTensorC(lp.FMT[fmt], axis, batch, rows, cols, codes, scales, ts)


def dq(t, dst=FAKE):
    return lp.lib.lp_dequant(ctypes.byref(t) if t is not None else None, dst, None)


@pytest.mark.parametrize("t,dst,expect", [
    (None, FAKE, NULL),
    (q("mxfp4", 4, 64, codes=None), FAKE, NULL),
    (q("mxfp4", 4, 64, scales=None), FAKE, NULL),
    (q("nvfp4", 4, 64, ts=None), FAKE, NULL),
    (q("mxfp4", 4, 64), None, NULL),
    (q("mxfp4", 4, 48), FAKE, SHAPE),            # MX blocks of 32 along cols
    (q("fp8_b128", 4, 40), FAKE, SHAPE),         # cols % 16
    (q("mxfp8", 40, 64, axis=-2), FAKE, SHAPE),  # rows % 32 along rows
    (q("mxfp8", -1, 64), FAKE, SHAPE),
    (q("bf16", 4, 64), FAKE, FORMAT),            # nothing to decode
    (q("mxfp4", 32, 64, axis=-2), FAKE, FORMAT),  # only MXFP8 scales along rows
    (_QTensorC(9, -1, 1, 4, 64, FAKE, FAKE, FAKE), FAKE, FORMAT),
    (q("mxfp4", 4, 64, codes=FAKE + 8), FAKE, ALIGN),
    (q("mxfp4", 4, 64, scales=FAKE + 4), FAKE, ALIGN),
    (q("mxfp4", 4, 64), FAKE + 2, ALIGN),
    (q("mxfp4", 0, 64, codes=None, scales=None), None, OK),   # empty: nothing to do
    (q("fp8t_e5m2", 4, 64, ts=None), FAKE, NULL),          # per-tensor: the tensor scale is required
    (q("fp8t_e4m3", 4, 40), FAKE, SHAPE),
    (q("fp8t_e4m3", 4, 64, ts=FAKE + 2), FAKE, ALIGN),
    (_QTensorC(7, -1, 1, 4, 64, FAKE, FAKE, FAKE), FAKE, FORMAT),
])
def test_dequant_rejects(t, dst, expect):
    assert dq(t, dst) == expect


@pytest.mark.parametrize("args,expect", [
    ((None, 1, 32, 32, -1, lp.FMT["mxfp8"], FAKE, FAKE), NULL),
    ((FAKE, 1, 32, 48, -1, lp.FMT["mxfp8"], FAKE, FAKE), SHAPE),
    ((FAKE, 1, 48, 32, -2, lp.FMT["mxfp8"], FAKE, FAKE), SHAPE),
    ((FAKE, 1, 32, 36, -2, lp.FMT["mxfp8"], FAKE, FAKE), SHAPE),
    ((FAKE, 1, 32, 32, 0, lp.FMT["mxfp8"], FAKE, FAKE), FORMAT),
    ((FAKE, 1, 32, 32, -1, lp.FMT["nvfp4"], FAKE, FAKE), FORMAT),
    ((FAKE + 8, 1, 32, 32, -1, lp.FMT["mxfp8"], FAKE, FAKE), ALIGN),
    ((None, 1, 0, 32, -1, lp.FMT["mxfp8"], None, None), OK),
])
def test_mx_quant_rejects(args, expect):
    assert lp.lib.lp_mx_quant(*args, None) == expect


@pytest.mark.parametrize("args,expect", [
    ((None, 1, 32, 32, lp.FMT["mxfp8"], FAKE, FAKE, FAKE, FAKE), NULL),
    ((FAKE, 1, 32, 32, lp.FMT["mxfp8"], FAKE, FAKE, None, FAKE), NULL),
    ((FAKE, 1, 32, 48, lp.FMT["mxfp8"], FAKE, FAKE, FAKE, FAKE), SHAPE),      # cols % 32
    ((FAKE, 1, 48, 32, lp.FMT["mxfp8"], FAKE, FAKE, FAKE, FAKE), SHAPE),      # rows % 32
    ((FAKE, 1, 32, 32, lp.FMT["fp8_b128"], FAKE, FAKE, FAKE, FAKE), FORMAT),
    ((FAKE, 1, 32, 32, lp.FMT["mxfp4"], FAKE, FAKE, FAKE, FAKE + 4), ALIGN),
    ((None, 3, 0, 64, lp.FMT["mxfp8"], None, None, None, None), OK),
])
def test_mx_quant_dual_rejects(args, expect):
    assert lp.lib.lp_mx_quant_dual(*args, None) == expect


E4M3T, E5M2T = lp.FMT["fp8t_e4m3"], lp.FMT["fp8t_e5m2"]


@pytest.mark.parametrize("args,expect", [
    ((FAKE, 64, lp.FMT["mxfp8"], FAKE, FAKE, FAKE), FORMAT),
    ((FAKE, 12, E4M3T, FAKE, FAKE, FAKE), SHAPE),          # n % 8
    ((FAKE, -8, E4M3T, FAKE, FAKE, FAKE), SHAPE),
    ((None, 64, E5M2T, FAKE, FAKE, FAKE), NULL),
    ((FAKE, 64, E5M2T, None, FAKE, None), NULL),           # the scale is required
    ((FAKE, 64, E5M2T, FAKE, FAKE, FAKE), SHAPE),          # amax would overwrite the scale
    ((FAKE, 64, E5M2T, FAKE, FAKE + 8, FAKE + 4), ALIGN),
    ((FAKE, 64, E5M2T, FAKE + 2, FAKE, FAKE + 4), ALIGN),
    ((FAKE + 8, 64, E4M3T, FAKE, FAKE, None), ALIGN),
])
def test_tensor_quant_rejects(args, expect):
    assert lp.lib.lp_tensor_quant(*args, None) == expect


def test_tensor_quant_delayed_rejects():
    f = lp.lib.lp_tensor_quant_delayed
    ring = 0x20000
    assert f(FAKE, 64, lp.FMT["mxfp8"], ring, 16, 0, 0, FAKE, FAKE, None) == FORMAT
    assert f(FAKE, 12, E5M2T, ring, 16, 0, 0, FAKE, FAKE, None) == SHAPE      # n % 8
    assert f(FAKE, 64, E5M2T, ring, 16, 16, 0, FAKE, FAKE, None) == SHAPE     # slot past the ring
    assert f(FAKE, 64, E5M2T, ring, 16, -1, 0, FAKE, FAKE, None) == SHAPE
    assert f(FAKE, 64, E5M2T, ring, 0, 0, 0, FAKE, FAKE, None) == SHAPE       # empty ring
    assert f(FAKE, 64, E5M2T, ring, 16, 0, 65, FAKE, FAKE, None) == SHAPE     # margin
    assert f(FAKE, 64, E5M2T, ring, 16, 0, 0, FAKE, ring + 8, None) == SHAPE  # scale inside the ring
    assert f(FAKE, 64, E5M2T, None, 16, 0, 0, FAKE, FAKE, None) == NULL
    assert f(FAKE, 64, E5M2T, ring, 16, 0, 0, FAKE, None, None) == NULL
    assert f(FAKE, 64, E5M2T, ring, 16, 0, 0, FAKE + 8, FAKE, None) == ALIGN


def test_tensor_amax_and_scale_reject():
    assert lp.lib.lp_tensor_amax(FAKE, 20, FAKE, None) == SHAPE
    assert lp.lib.lp_tensor_amax(FAKE, 64, None, None) == NULL
    assert lp.lib.lp_tensor_amax(None, 64, FAKE, None) == NULL
    assert lp.lib.lp_tensor_amax(FAKE + 8, 64, FAKE, None) == ALIGN
    sfh = lp.lib.lp_scale_from_history
    assert sfh(FAKE, 16, lp.FMT["mxfp8"], 0, FAKE, None) == FORMAT
    assert sfh(FAKE, 0, E4M3T, 0, FAKE, None) == SHAPE
    assert sfh(FAKE, 65537, E4M3T, 0, FAKE, None) == SHAPE
    assert sfh(FAKE, 16, E4M3T, 65, FAKE, None) == SHAPE
    assert sfh(FAKE, 16, E5M2T, -65, FAKE, None) == SHAPE
    assert sfh(None, 16, E5M2T, 0, FAKE, None) == NULL
    assert sfh(FAKE, 16, E5M2T, 0, FAKE + 1, None) == ALIGN


def fwd(x, w, y=FAKE):
    ref = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    return lp.lib.lp_linear_fwd(ref(x), ref(w), y, None)


@pytest.mark.parametrize("x,w,y,expect", [
    (None, q("mxfp4", 64, 128), FAKE, NULL),
    (q("mxfp4", 64, 128), q("mxfp4", 32, 128), None, NULL),
    (q("mxfp4", 64, 128), q("mxfp8", 32, 128), FAKE, FORMAT),       # formats must agree
    (q("bf16", 64, 128), q("mxfp4", 32, 128), FAKE, FORMAT),        # bf16 x: bf16, block-FP8 or NVFP4 weight
    (q("bf16", 64, 48), q("nvfp4", 32, 48), FAKE, SHAPE),           # NVFP4 weight: K % 32
    (q("fp8_b128", 64, 128), q("bf16", 32, 128), FAKE, FORMAT),     # the block-FP8 operand is the weight
    (q("nvfp4", 64, 128), q("bf16", 32, 128), FAKE, FORMAT),        # NVFP4 x: NVFP4 weight
    (q("nvfp4", 64, 48), q("nvfp4", 32, 48), FAKE, SHAPE),          # NVFP4: K % 32
    (q("bf16", 64, 128), q("fp8_b128", 40, 128), FAKE, SHAPE),      # N % 16
    (q("bf16", 0, 128, codes=None), q("fp8_b128", 32, 128), None, OK),
    (q("mxfp8", 64, 128, axis=-2), q("mxfp8", 32, 128), FAKE, FORMAT),
    (q("mxfp4", 64, 96), q("mxfp4", 32, 96), FAKE, SHAPE),          # MXFP4: K % 128
    (q("mxfp8", 64, 96), q("mxfp8", 32, 96), FAKE, SHAPE),          # MXFP8: K % 64
    (q("mxfp4", 64, 128), q("mxfp4", 40, 128), FAKE, SHAPE),        # N % 16
    (q("mxfp4", 64, 128), q("mxfp4", 32, 256), FAKE, SHAPE),        # K disagrees
    (q("mxfp4", 64, 128), q("mxfp4", 32, 128, batch=2), FAKE, SHAPE),
    (q("mxfp4", 64, 128), q("mxfp4", 32, 128), FAKE + 8, ALIGN),
    (q("mxfp4", 0, 128, codes=None, scales=None), q("mxfp4", 32, 128), None, OK),   # M = 0: nothing to do
])
def test_linear_fwd_rejects(x, w, y, expect):
    assert fwd(x, w, y) == expect


def test_grouped_fwd_rejects():
    x, w = q("mxfp4", 64, 128), q("mxfp4", 32, 128, batch=4)
    call = lambda off, G: lp.lib.lp_grouped_fwd(ctypes.byref(x), ctypes.byref(w), off, G, FAKE, None)  # noqa: E731
    assert call(FAKE, 0) == SHAPE
    assert call(FAKE, 3) == SHAPE            # w batch must equal groups
    assert call(None, 4) == NULL
    assert call(FAKE + 2, 4) == ALIGN


def test_grouped_rejects_row_scaled_grad():
    g, x = q("mxfp8", 64, 128, axis=-2), q("mxfp8", 64, 128, axis=-2)
    assert lp.lib.lp_grouped_bwd(ctypes.byref(g), ctypes.byref(x), None, FAKE, 2, None, FAKE, None) == FORMAT


def lin(g, x, w, dx=FAKE, dw=FAKE):
    ref = lambda t: ctypes.byref(t) if t is not None else None  # noqa: E731
    return lp.lib.lp_linear_bwd(ref(g), ref(x), ref(w), dx, dw, None)


@pytest.mark.parametrize("g,x,w,dx,dw,expect", [
    (q("bf16", 64, 128), q("mxfp4", 64, 128), q("mxfp4", 128, 128), None, None, OK),   # nothing asked
    (None, q("mxfp4", 64, 128), q("mxfp4", 128, 128), FAKE, FAKE, NULL),
    (q("bf16", 64, 128), None, q("mxfp4", 128, 128), FAKE, FAKE, NULL),        # dW needs x
    (q("bf16", 64, 128), q("mxfp4", 64, 128), None, FAKE, FAKE, NULL),         # dX needs w
    (q("bf16", 64, 128), q("mxfp4", 64, 128), q("mxfp4", 64, 128), FAKE, None, SHAPE),   # w rows != N
    (q("bf16", 64, 128), q("mxfp4", 32, 128), q("mxfp4", 128, 128), None, FAKE, SHAPE),  # x rows != M
    (q("bf16", 64, 128), q("mxfp4", 64, 96), q("mxfp4", 128, 128), FAKE, FAKE, SHAPE),   # K disagrees
    (q("bf16", 64, 120), q("mxfp4", 64, 128), q("mxfp4", 120, 128), FAKE, FAKE, SHAPE),  # N % 16
    (q("nvfp4", 64, 128), q("mxfp4", 64, 128), q("mxfp4", 128, 128), FAKE, None, FORMAT),  # grad format
    (q("mxfp8", 64, 128), q("mxfp4", 64, 128), q("mxfp4", 128, 128), None, FAKE, FORMAT),  # MXFP8 grad, dW
    (q("mxfp8", 64, 128, axis=-2), None, q("mxfp8", 128, 128, axis=-2), FAKE, None, FORMAT),  # row-scaled grad, dX
    (q("mxfp8", 64, 128, axis=-2), q("mxfp4", 64, 128), None, None, FAKE, FORMAT),   # row-scaled grad, X not MX rows
    (q("mxfp8", 64, 128, axis=-2), q("mxfp8", 64, 128, axis=-1), None, None, FAKE, FORMAT),
    (q("bf16", 64, 128), q("mxfp4", 64, 128), q("nvfp4", 128, 48), FAKE, None, SHAPE),   # FP4 K % 32
    (q("bf16", 64, 128), q("mxfp4", 64, 128), q("mxfp4", 128, 128, batch=2), FAKE, None, SHAPE),
    (q("bf16", 64, 128), q("mxfp4", 64, 128), q("mxfp4", 128, 128), FAKE + 8, None, ALIGN),
    # per-tensor FP8 operands pair only with each other
    (q("fp8t_e5m2", 64, 128), None, q("bf16", 128, 128), FAKE, None, FORMAT),
    (q("bf16", 64, 128), None, q("fp8t_e4m3", 128, 128), FAKE, None, FORMAT),
    (q("fp8t_e5m2", 64, 128), q("mxfp8", 64, 128, axis=-2), None, None, FAKE, FORMAT),
    (q("mxfp8", 64, 128, axis=-2), q("fp8t_e4m3", 64, 128), None, None, FAKE, FORMAT),
    (q("fp8t_e5m2", 64, 128), None, q("fp8t_e4m3", 128, 128, ts=None), FAKE, None, NULL),
    (q("fp8t_e5m2", 64, 128, ts=FAKE + 1), None, q("fp8t_e4m3", 128, 128), FAKE, None, ALIGN),
    (q("fp8t_e5m2", 64, 120), None, q("fp8t_e4m3", 120, 128), FAKE, None, SHAPE),
])
def test_linear_bwd_rejects(g, x, w, dx, dw, expect):
    assert lin(g, x, w, dx, dw) == expect


def test_grouped_bwd_rejects():
    g, x, w = q("bf16", 64, 128), q("mxfp4", 64, 128), q("mxfp4", 128, 128, batch=4)
    call = lambda off, G, w=w: lp.lib.lp_grouped_bwd(  # noqa: E731
        ctypes.byref(g), ctypes.byref(x), ctypes.byref(w), off, G, FAKE, FAKE, None)
    assert call(FAKE, 0) == SHAPE
    assert call(FAKE, 1025) == SHAPE
    assert call(None, 4) == NULL
    assert call(FAKE + 2, 4) == ALIGN
    assert call(FAKE, 3) == SHAPE          # w batch must equal groups


def ws_bytes(g, x, w, dx=True, dw=True):
    n = ctypes.c_size_t(123)
    st = lp.lib.lp_linear_bwd_workspace(ctypes.byref(g), ctypes.byref(x) if x else None,
                                        ctypes.byref(w) if w else None, 1 if dx else None, 1 if dw else None,
                                        ctypes.byref(n))
    return st, n.value


def test_workspace_size_rules():
    # dX of the frozen FP8 weight: 256 tiles of 256 x 128 fill the CUs -> no split
    g = q("bf16", 4096, 8192)
    st, n = ws_bytes(g, None, q("fp8_b128", 8192, 2048), dw=False)
    assert st == OK and n == 0
    # dX with 2 x 3 tiles of 256 x 256 over N = 4096: 64 slabs -> 4 splits of 16 slabs,
    # 6 per-tile counters (24 B, rounded to 256) + 6 x 4 fp32 tiles of 256 x 256
    st, n = ws_bytes(q("bf16", 300, 4096), None, q("fp8_b128", 4096, 544), dw=False)
    assert st == OK and n == 256 + 6 * 4 * 256 * 256 * 4
    # enough tiles already: no split
    st, n = ws_bytes(q("bf16", 8192, 4096), q("nvfp4", 8192, 4096), q("nvfp4", 4096, 4096))
    assert st == OK and n == 0
    # short contraction (2 slabs): no split
    st, n = ws_bytes(q("bf16", 64, 128), q("mxfp4", 64, 128), q("mxfp4", 128, 128))
    assert st == OK and n == 0
    # dW over a long token axis: 1 x 2 tiles, 4096 / 64 = 64 slabs -> 4 splits of 16 slabs
    st, n = ws_bytes(q("bf16", 4096, 256), q("bf16", 4096, 512), None, dx=False)
    assert st == OK and n == 256 + 2 * 4 * 256 * 256 * 4
    # per-tensor FP8 products never split
    st, n = ws_bytes(q("fp8t_e5m2", 300, 4096), None, q("fp8t_e4m3", 4096, 544), dw=False)
    assert st == OK and n == 0
    # argument errors as for lp_linear_bwd
    st, n = ws_bytes(q("bf16", 64, 128), q("mxfp4", 63, 128), None, dx=False)
    assert st == SHAPE and n == 0
    assert lp.lib.lp_linear_bwd_workspace(ctypes.byref(g), None, None, 1, None, None) == NULL


def test_linear_bwd_ws_rejects_misaligned_workspace():
    g = q("bf16", 4096, 8192)
    w = q("fp8_b128", 8192, 2048)
    assert lp.lib.lp_linear_bwd_ws(ctypes.byref(g), None, ctypes.byref(w), FAKE, None, FAKE + 16, 1 << 30,
                                   None) == ALIGN


def test_linear_bwd_noalloc_rejects_before_any_launch():
    """Argument errors of the no-allocation variant, reported as for
    lp_linear_bwd, before the library looks up its scratch array."""
    g = q("bf16", 4096, 8192)
    w = q("fp8_b128", 8192, 2048)
    f = lp.lib.lp_linear_bwd_noalloc
    assert f(ctypes.byref(g), None, None, FAKE, None, None) == NULL                 # dX without a weight
    assert f(ctypes.byref(g), None, ctypes.byref(w), FAKE + 8, None, None) == ALIGN
    bad = q("fp8_b128", 8000, 2048)
    assert f(ctypes.byref(g), None, ctypes.byref(bad), FAKE, None, None) == SHAPE
    assert f(ctypes.byref(g), None, ctypes.byref(w), None, None, None) == OK          # nothing asked for


BIG = (1 << 31) - 32        # below 2^31 and a multiple of 32


def test_element_counts_past_int64_are_rejected():
    """batch x rows x cols of three sizes just below 2^31 overflows 64 bits;
    the count is checked without forming the product."""
    assert dq(q("mxfp8", BIG, BIG, batch=BIG)) == SHAPE
    assert dq(q("mxfp8", 1 << 20, 1 << 14)) == SHAPE          # exactly 2^34 elements
    assert lp.lib.lp_mx_quant(FAKE, BIG, BIG, BIG, -1, lp.FMT["mxfp8"], FAKE, FAKE, None) == SHAPE
    assert lp.lib.lp_mx_quant_dual(FAKE, BIG, BIG, BIG, lp.FMT["mxfp8"], FAKE, FAKE, FAKE, FAKE, None) == SHAPE


def test_outputs_with_too_many_tiles_are_rejected():
    """Every operand fits its own limits, but the output has more tiles than
    a launch counts in 32 bits."""
    # grad_X of 2^29 tokens over a 2^21-wide input: about 2^36 tiles
    assert lin(q("bf16", 1 << 29, 16), None, q("fp8_b128", 16, 1 << 21), FAKE, None) == SHAPE
    # grad_W of 1024 groups of 2^21 x 2^21: about 2^38 tiles
    g, x = q("bf16", 16, 1 << 21), q("fp8_b128", 16, 1 << 21)
    assert lp.lib.lp_grouped_bwd(ctypes.byref(g), ctypes.byref(x), None, FAKE, 1024, None, FAKE, None) == SHAPE
    # forward of 2^24 tokens into 2^21 outputs
    xf, wf = q("mxfp4", 1 << 24, 128), q("mxfp4", 1 << 21, 128)
    assert lp.lib.lp_linear_fwd(ctypes.byref(xf), ctypes.byref(wf), FAKE, None) == SHAPE


def test_product_dimensions_beyond_the_kernels_addressing_are_rejected():
    """Rows of 2^22 or more elements, or 2^30 or more tokens."""
    assert lin(q("bf16", 16, 1 << 22), None, q("fp8_b128", 1 << 22, 16), FAKE, None) == SHAPE     # N
    assert lin(q("bf16", 16, 16), None, q("fp8_b128", 16, 1 << 22), FAKE, None) == SHAPE          # K
    assert lin(q("bf16", 1 << 30, 16), q("fp8_b128", 1 << 30, 16), None, None, FAKE) == SHAPE     # M
    xf, wf = q("mxfp4", 16, 1 << 22), q("mxfp4", 16, 1 << 22)
    assert lp.lib.lp_linear_fwd(ctypes.byref(xf), ctypes.byref(wf), FAKE, None) == SHAPE


def test_binding_rejects_host_tensors():
    """The binding passes bare pointers to kernels: a host tensor must be
    refused before any C call (CPU only)."""
    src = torch.zeros(64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        lp.lp_tensor_amax(src)
    with pytest.raises(ValueError, match="device tensor"):
        lp.lp_mx_quant(src.view(2, 32), -1)
    qt = lp.QTensor("mxfp8", torch.zeros((1, 4, 64), dtype=torch.uint8), torch.zeros((1, 4, 2), dtype=torch.uint8))
    with pytest.raises(ValueError, match="device tensor"):
        lp.lp_dequant(qt)
