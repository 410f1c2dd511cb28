"""lp_linear_bwd_noalloc (the split workspace held inside the library)
against lp_linear_bwd_ws with a caller-owned workspace, and against the
fp64 oracle (GPU).

Two calls in a row, the second on a smaller, ragged problem: both split
their contractions (few output tiles, long contractions), so both go
through the library's own scratch array, and the second must not be
disturbed by what the first left in it."""
import ctypes

import pytest
import torch

import workloads as W
from gpu_util import assert_bits_equal, assert_close, bf16_dev, bits_host, quantize
from oracle import gemm as O

pytestmark = pytest.mark.gpu


def _case(lp, number, M, N, K, xfmt, wfmt):
    gbits = W.bf16_bits(W.normal_f32(number, "grad", (M, N), 1.0))
    g = lp.QTensor("bf16", bf16_dev(gbits), shape=(1, M, N))
    x, xd = quantize(lp, xfmt, W.normal_f32(number, "x", (M, K), 1.0))
    w, wd = quantize(lp, wfmt, W.normal_f32(number, "w", (N, K), 0.02))
    return g, gbits, x, xd[0], w, wd[0]


def test_noalloc_matches_workspace_call_twice(lp):
    cases = [(60, 4096, 4096, 256, "mxfp4", "fp8_b128"),     # 16 output tiles each, 4 splits
             (61, 2100, 2048, 160, "nvfp4", "bf16")]         # smaller, ragged M, 2 splits
    for number, M, N, K, xfmt, wfmt in cases:
        print(f"case {number}: M={M} N={N} K={K} x={xfmt} w={wfmt}", flush=True)
        g, gbits, x, xd, w, wd = _case(lp, number, M, N, K, xfmt, wfmt)
        need = lp.lp_linear_bwd_workspace(g, x, w)
        assert need > 0, "the case is meant to split its contractions"
        dx, dw = lp.lp_linear_bwd_noalloc(g, x, w)
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        rx, rw = lp.lp_linear_bwd(g, x, w, workspace=ws)
        torch.cuda.synchronize()
        assert_bits_equal(bits_host(dx), bits_host(rx), f"case {number} dX vs the workspace call")
        assert_bits_equal(bits_host(dw), bits_host(rw), f"case {number} dW vs the workspace call")
        assert_close(dx, O.linear_dx(gbits, wd), f"case {number} dX")
        assert_close(dw, O.linear_dw(gbits, xd), f"case {number} dW")


def test_noalloc_without_split_and_rejects(lp):
    """A call whose tiles fill the GPU needs no scratch; argument errors
    are reported as for the other entry points."""
    M, N, K = 1024, 256, 4096
    g, gbits, x, xd, w, wd = _case(lp, 62, M, N, K, "mxfp4", "mxfp4")
    assert lp.lp_linear_bwd_workspace(g, x, w, need_dw=False) == 0
    dx, _ = lp.lp_linear_bwd_noalloc(g, None, w, need_dw=False)
    torch.cuda.synchronize()
    assert_close(dx, O.linear_dx(gbits, wd), "unsplit dX")
    gc = g.c()
    st = lp.lib.lp_linear_bwd_noalloc(ctypes.byref(gc), None, None, dx.data_ptr(), None, None)
    assert st == 1, lp.lib.lp_status_string(st)          # LP_ERR_NULL: dX asked for without a weight
