"""Maximum sizes: tensors past 2^31 elements (and bytes), and a gradient of
2^20 + 37 rows, through the same calls, checked on sampled rows (the first,
some in the middle, the last) against the oracle.  Inputs are drawn on the
device by torch's generator and the sampled rows copied to the host (GPU)."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import assert_bits_equal, assert_close, bits_host, dev
from oracle import formats as F
from oracle import gemm as O

pytestmark = pytest.mark.gpu

BIG_ROWS, BIG_COLS = 65536 + 8, 32768            # 2^31 + 2^18 elements


def _sample_rows(rows):
    return np.unique(np.concatenate([[0, 1], np.arange(0, rows, rows // 7), [rows - 2, rows - 1]]))


def test_dequant_past_2g_elements(lp):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(51)
    codes = torch.randint(0, 256, (1, BIG_ROWS, BIG_COLS), generator=gen, dtype=torch.uint8, device="cuda")
    scales = torch.randint(112, 142, (1, BIG_ROWS, BIG_COLS // 32), generator=gen, dtype=torch.uint8, device="cuda")
    q = lp.QTensor("mxfp8", codes, scales, shape=(1, BIG_ROWS, BIG_COLS), axis=-1)
    out = lp.lp_dequant(q)
    torch.cuda.synchronize()
    rows = _sample_rows(BIG_ROWS)
    ridx = torch.from_numpy(rows).cuda()
    want = F.dequant("mxfp8", codes[0, ridx].cpu().numpy()[None], scales[0, ridx].cpu().numpy()[None], axis=-1)[0]
    assert_bits_equal(bits_host(out[0, ridx]), want, "dequant rows past 2^31 elements")
    del out, codes, scales
    torch.cuda.empty_cache()


def test_mx_quant_past_2g_elements(lp):
    src = W.torch_normal_bf16((BIG_ROWS, BIG_COLS), 1.0, 52, "cuda")
    q = lp.lp_mx_quant(src, -1, "mxfp8")
    torch.cuda.synchronize()
    rows = _sample_rows(BIG_ROWS)
    ridx = torch.from_numpy(rows).cuda()
    bits = bits_host(src[ridx])
    rc, rs = F.mx_quant(bits[None], -1, "e4m3")
    assert_bits_equal(q.scales[0, ridx].cpu().numpy(), rs[0], "scales of rows past 2^31 elements")
    assert_bits_equal(q.codes[0, ridx].cpu().numpy(), rc[0], "codes of rows past 2^31 elements")
    del q, src
    torch.cuda.empty_cache()


def test_linear_dx_tall_gradient(lp):
    """2^20 + 37 token rows (4097 row tiles, a ragged last one)."""
    M, N, K = (1 << 20) + 37, 512, 256
    g = W.torch_normal_bf16((M, N), 1.0, 53, "cuda")
    w = W.normal_f32(53, "w", (N, K), 0.02)
    wc, ws = F.quant_mxfp4_f32(w[None])
    wq = lp.QTensor("mxfp4", dev(wc), dev(ws), shape=(1, N, K))
    gq = lp.QTensor("bf16", g, shape=(1, M, N))
    dx, _ = lp.lp_linear_bwd(gq, None, wq, need_dw=False)
    torch.cuda.synchronize()
    rows = _sample_rows(M)
    ridx = torch.from_numpy(rows).cuda()
    wd = F.dequant("mxfp4", wc, ws)[0]
    assert_close(dx[ridx], O.linear_dx(bits_host(g[ridx]), wd), "dX rows of a 2^20-row gradient")
