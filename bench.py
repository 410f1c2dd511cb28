"""Benchmark of the block-scaled backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu]

A step is one pass of the workload's whole backward path over one batch of
synthetic input already resident in HBM:
  mxfp8_deferred  lp_mx_quant(grad, -1) + lp_grouped_dx_deferred: grouped dX over 64 experts
                  against the bf16 weight quantized to MXFP8 along its reduction axis, inside
                  the product for experts of at most 1536 tokens (default: the largest
                  workload, 962 GFLOP per step; --unfused: lp_mx_quant(W, -2) then
                  lp_grouped_bwd)
  fp8_frozen      lp_dequant of a frozen FP8 128x128-block weight to bf16, then
                  lp_linear_bwd: dX against the bf16 copy
  nvfp4_linear    lp_linear_bwd: dX and dW, NVFP4 X and W
  mxfp4_grouped   lp_grouped_bwd: dX and dW over 8 experts, MXFP4 X and W
  mxfp8_dense     lp_mx_quant_dual(grad) + lp_mx_quant(W, -2) + lp_mx_quant(X, -2) + lp_linear_bwd dX, dW
  fp8_hybrid      lp_tensor_quant_delayed(grad -> E5M2 with the ring's scale, amax into the ring)
                  + lp_linear_bwd dX, dW against E4M3 X and W (per-tensor scales)
  mxfp4_forward   lp_linear_fwd: y = X @ W^T, MXFP4 X 8192x4096 and W 4096x4096 (the forward
                  the FP4 backward pairs with, on the block-scaled FP4 MFMA)
  nvfp4_forward   lp_dequant of NVFP4 X 8192x4096 to bf16, then lp_linear_fwd: y = X @ W^T
                  against the NVFP4 W 4096x4096, decoded inside the contraction
  fp8_grouped_forward  lp_grouped_fwd: bf16 X 16384x4096 against 8 block-FP8 experts
                  8x2048x4096 (the FP8-adapter page's grouped forward)
  mxfp4_tiny      lp_linear_bwd: dX and dW, 64 x 128 x 128
Input sets are rotated through about 1 GB so that the 256 MiB Infinity Cache
cannot serve a repeated step.  Prints one JSON line (rank 0).

The default warmup is long (1000 steps): the GPU reaches its sustained
clock only after some hundreds of milliseconds of load, and a training step
runs in that steady state.  Measured on the FP8 frozen-weight workload, its
GEMM's launch time was 160 us after 5 warmup steps, 148 us after 100 and
139-143 us after 1000 to 10000; the deferred MXFP8 step, about 1.2 ms long,
moves by about 1%.

The CPU-baseline leg times the oracle kernel by kernel (decode, quantize,
products) on bounded samples, on one thread and on all of BLAS's threads,
and scales each to the whole step.

Inputs are drawn on the GPU by torch and quantized there: FP8 blocks and
NVFP4 with plain torch ops (input preparation only), MXFP4 with the
library's own lp_mx_quant.  The CPU-baseline leg runs the CPU oracle on a
bounded sample of the same workload (its inputs drawn with numpy).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "backward TFLOP/s (dX+dW) and % BF16 MFMA peak; dequant/quant GB/s vs HBM"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA (the block-scaled MXFP8 contraction)
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense fp4 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
ROTATE_BYTES = 1 << 30
UNFUSED = False                # mxfp8_deferred: the three-call step instead of lp_grouped_dx_deferred
# mxfp8_deferred: experts of at most this many tokens (six 256-row tiles)
# quantize their weight inside the product.  Interleaved steady-state sweeps
# of the whole call, with each weight column's row tiles listed together:
# 512 836-839 us, 768 827, 1024 831-835, 1536 805-809, 2048 811-820, every
# expert 845 (with row tiles listed row by row: 0 1046, 256 897-901, 512
# 873-879, every expert 896).
FUSE_ROWS = 1536


# ------------------------------------------------------------------ input preparation (torch, GPU)

def _randn(shape, sigma, seed):
    return W.torch_normal_bf16(shape, sigma, seed, "cuda").float()


def fp8_b128_quant_torch(w: torch.Tensor):
    """FP8 block inputs: s = amax/448 per 128x128 block, codes = E4M3(w / s)."""
    R, C = w.shape[-2:]
    lead = w.shape[:-2]
    wb = w.reshape(*lead, R // 128, 128, C // 128, 128)
    amax = wb.abs().amax(dim=(-3, -1))
    s = (amax / 448.0).clamp_min(1e-30)
    t = wb / s[..., :, None, :, None]
    codes = t.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, R, C)
    return codes.contiguous(), s.float().contiguous()


_E2M1 = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def nvfp4_quant_torch(x: torch.Tensor):
    """NVFP4 inputs (two-level recipe): tensor scale amax/(6*448), E4M3 block
    scale per 16, E2M1 codes by nearest magnitude."""
    st = (x.abs().amax() / (6.0 * 448.0)).clamp_min(1e-30).float()
    R, C = x.shape[-2:]
    xb = x.reshape(R, C // 16, 16)
    sb = (xb.abs().amax(-1) / 6.0 / st).to(torch.float8_e4m3fn)
    S = sb.float() * st
    t = (xb / S.clamp_min(1e-30)[..., None]).reshape(R, C)
    grid = _E2M1.to(x.device)
    mag = (t.abs()[..., None] - grid).abs().argmin(-1).to(torch.uint8)
    code = mag | ((t < 0).to(torch.uint8) << 3)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return packed, sb.view(torch.uint8).contiguous(), st.reshape(1).contiguous()


# ------------------------------------------------------------------ workload runners

class Phase:
    """One library call of a step, timed with HIP events on the launch stream."""

    def __init__(self, name, kernel, flops=0.0, nbytes=0.0, peak=PEAK_BF16_TFLOPS):
        self.name, self.kernel, self.flops, self.nbytes, self.peak = name, kernel, flops, nbytes, peak
        self.ms = []


def build(lp, name: str):
    w = W.WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    sets = []
    phases = []
    if name in ("fp8_frozen", "nvfp4_linear", "mxfp4_tiny"):
        per_set = M * N * 2 + N * K * (1 if w.fmt == "fp8_b128" else 0.5) * (1 if name == "fp8_frozen" else 2)
        nsets = max(1, min(16, math.ceil(ROTATE_BYTES / per_set)))
        for i in range(nsets):
            g = W.torch_normal_bf16((M, N), 1.0, 7000 + i, "cuda")
            wt = _randn((N, K), w.w_sigma, 7100 + i)
            gq = lp.QTensor("bf16", g, shape=(1, M, N))
            if w.fmt == "fp8_b128":
                c, s = fp8_b128_quant_torch(wt)
                wq, xq = lp.QTensor("fp8_b128", c, s, shape=(1, N, K)), None
            elif w.fmt == "nvfp4":
                xt = _randn((M, K), 1.0, 7200 + i)
                c, s, ts = nvfp4_quant_torch(wt)
                wq = lp.QTensor("nvfp4", c, s, ts, shape=(1, N, K))
                c, s, ts = nvfp4_quant_torch(xt)
                xq = lp.QTensor("nvfp4", c, s, ts, shape=(1, M, K))
            else:
                xt = _randn((M, K), 1.0, 7200 + i).to(torch.bfloat16)
                wq = lp.lp_mx_quant(wt.to(torch.bfloat16), -1, "mxfp4")
                xq = lp.lp_mx_quant(xt, -1, "mxfp4")
            dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
            dw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda") if w.need_dw else None
            sets.append((gq, xq, wq, dx, dw))
        flops = 2.0 * M * N * K * (2 if w.need_dw else 1)
        if name == "fp8_frozen":
            # The weight is decoded once per step into a bf16 copy (lp_dequant), then dX
            # contracts bf16 with bf16, both operands loaded straight into LDS: the
            # order of "Train adapters on top of FP8 weights", FP8LinearFunction.backward
            # (dequantize the weight, then matmul).  At this shape it is faster than
            # decoding inside the GEMM, where each of the 16 row tiles decodes the
            # weight again; the results are bit-identical.
            wbf = torch.empty((1, N, K), dtype=torch.bfloat16, device="cuda")
            wbq = lp.QTensor("bf16", wbf, shape=(1, N, K))
            scale_bytes = ((N + 127) // 128) * ((K + 127) // 128) * 4
            phases.append(Phase("dequant W", "dequant_fp8_b128", nbytes=N * K * 3 + scale_bytes))
            phases.append(Phase("linear_bwd dX (bf16 W)", "gemm_kernel", flops=flops))

            def step(i, stream):
                gq, xq, wq, dx, dw = sets[i % len(sets)]
                ev = _events(stream)
                lp.lp_dequant(wq, wbf, stream=stream)
                t0 = ev.stop(stream)
                ev = _events(stream)
                lp.lp_linear_bwd(gq, None, wbq, need_dw=False, grad_x=dx, stream=stream)
                return [t0, ev.stop(stream)]
        else:
            phases.append(Phase("linear_bwd", "gemm_kernel", flops=flops))
            # One workspace serves every input set: steps run in order on one stream.
            gq, xq, wq = sets[0][:3]
            nws = lp.lp_linear_bwd_workspace(gq, xq, wq, True, w.need_dw)
            ws = torch.zeros(nws, dtype=torch.uint8, device="cuda") if nws else None

            def step(i, stream):
                gq, xq, wq, dx, dw = sets[i % len(sets)]
                ev = _events(stream)
                lp.lp_linear_bwd(gq, xq, wq, need_dw=w.need_dw, grad_x=dx, grad_w=dw, stream=stream, workspace=ws)
                return [ev.stop(stream)]
        standalone = [("W", sets[0][2])] + ([("X", sets[0][1])] if sets[0][1] is not None else [])
    elif name == "mxfp4_grouped":
        offsets = torch.from_numpy(W.cumulative_ends(W.group_sizes(w))).cuda()
        per_set = M * N * 2 + (M * K + w.groups * N * K) * 0.53125
        nsets = max(1, min(8, math.ceil(ROTATE_BYTES / per_set)))
        for i in range(nsets):
            g = W.torch_normal_bf16((M, N), 1.0, 7300 + i, "cuda")
            xq = lp.lp_mx_quant(W.torch_normal_bf16((M, K), 1.0, 7400 + i, "cuda"), -1, "mxfp4")
            wq = lp.lp_mx_quant(W.torch_normal_bf16((w.groups, N, K), 1.0, 7500 + i, "cuda"), -1, "mxfp4")
            dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
            dw = torch.empty((w.groups, N, K), dtype=torch.bfloat16, device="cuda")
            sets.append((lp.QTensor("bf16", g, shape=(1, M, N)), xq, wq, dx, dw))
        # dX and dW in one launch (grad_X tiles first)
        phases.append(Phase("grouped_bwd", "gemm_pair_kernel", flops=4.0 * M * N * K))

        def step(i, stream):
            gq, xq, wq, dx, dw = sets[i % len(sets)]
            ev = _events(stream)
            lp.lp_grouped_bwd(gq, xq, wq, offsets, grad_x=dx, grad_w=dw, stream=stream)
            return [ev.stop(stream)]
        standalone = [("X", sets[0][1]), ("W", sets[0][2])]
    elif name == "mxfp8_deferred":
        offsets = torch.from_numpy(W.cumulative_ends(W.group_sizes(w))).cuda()
        g = W.torch_normal_bf16((M, N), 1.0, 7600, "cuda")
        wt = W.torch_normal_bf16((w.groups, N, K), w.w_sigma, 7601, "cuda")
        gq = lp.lp_mx_quant(g, -1, "mxfp8")
        wq = lp.lp_mx_quant(wt, -2, "mxfp8")
        gq.shape = (1, M, N)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        sets.append((g, wt, gq, wq, dx))
        phases.append(Phase("mx_quant grad", "mx_quant_cols", nbytes=M * N * (2 + 1 + 1 / 32)))
        if UNFUSED:
            phases.append(Phase("mx_quant W", "mx_quant_tile", nbytes=w.groups * N * K * (2 + 1 + 1 / 32)))
            # MXFP8 x MXFP8 with both scales along the contraction: block-scaled FP8 MFMA
            phases.append(Phase("grouped_bwd dX", "fp8_mfma_paired", flops=2.0 * M * N * K,
                                peak=PEAK_FP8_TFLOPS))

            def step(i, stream):
                g, wt, gq, wq, dx = sets[0]
                ev = _events(stream)
                lp.lp_mx_quant(g, -1, "mxfp8", codes=gq.codes, scales=gq.scales, stream=stream)
                t0 = ev.stop(stream)
                ev = _events(stream)
                lp.lp_mx_quant(wt, -2, "mxfp8", codes=wq.codes, scales=wq.scales, stream=stream)
                t1 = ev.stop(stream)
                ev = _events(stream)
                lp.lp_grouped_bwd(gq, None, wq, offsets, need_dw=False, grad_x=dx, stream=stream)
                return [t0, t1, ev.stop(stream)]
        else:
            # One call: the weight is quantized inside the product for experts
            # of at most FUSE_ROWS tokens, first (into wq) for the others.
            # Algorithmic bytes: the bf16 weight, the gradient's codes and
            # scales, the bf16 result.
            phases.append(Phase("grouped_dx_deferred (W quant + dX)",
                                "mx_quant_rows_groups + fp8_mfma_paired + fp8_mfma_wquant_kernel",
                                flops=2.0 * M * N * K, peak=PEAK_FP8_TFLOPS,
                                nbytes=w.groups * N * K * 2 + M * N * (1 + 1 / 32) + M * K * 2))

            def step(i, stream):
                g, wt, gq, wq, dx = sets[0]
                ev = _events(stream)
                lp.lp_mx_quant(g, -1, "mxfp8", codes=gq.codes, scales=gq.scales, stream=stream)
                t0 = ev.stop(stream)
                ev = _events(stream)
                lp.lp_grouped_dx_deferred(gq, wt, offsets, fuse_rows=FUSE_ROWS, grad_x=dx, w_codes=wq.codes,
                                          w_scales=wq.scales, stream=stream)
                return [t0, ev.stop(stream)]
        standalone = []
    elif name == "mxfp8_dense":
        g = W.torch_normal_bf16((M, N), 1.0, 7700, "cuda")
        wt = W.torch_normal_bf16((N, K), w.w_sigma, 7701, "cuda")
        xt = W.torch_normal_bf16((M, K), w.x_sigma, 7702, "cuda")
        gc, gr = lp.lp_mx_quant_dual(g, "mxfp8")
        wq = lp.lp_mx_quant(wt, -2, "mxfp8")
        xq = lp.lp_mx_quant(xt, -2, "mxfp8")
        dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
        dw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
        phases.append(Phase("mx_quant_dual grad", "mx_quant_tile<dual>", nbytes=M * N * (2 + 2 * (1 + 1 / 32))))
        phases.append(Phase("mx_quant W", "mx_quant_tile", nbytes=N * K * (2 + 1 + 1 / 32)))
        phases.append(Phase("mx_quant X", "mx_quant_tile", nbytes=M * K * (2 + 1 + 1 / 32)))
        phases.append(Phase("linear_bwd dX", "fp8_mfma_paired", flops=2.0 * M * N * K, peak=PEAK_FP8_TFLOPS))
        phases.append(Phase("linear_bwd dW", "fp8_mfma_kernel", flops=2.0 * M * N * K, peak=PEAK_FP8_TFLOPS))

        def step(i, stream):
            ts = []
            ev = _events(stream)
            lp.lib.lp_mx_quant_dual(g.data_ptr(), 1, M, N, lp.FMT["mxfp8"], gc.codes.data_ptr(), gc.scales.data_ptr(),
                                    gr.codes.data_ptr(), gr.scales.data_ptr(), stream.cuda_stream)
            ts.append(ev.stop(stream))
            ev = _events(stream)
            lp.lp_mx_quant(wt, -2, "mxfp8", codes=wq.codes, scales=wq.scales, stream=stream)
            ts.append(ev.stop(stream))
            ev = _events(stream)
            lp.lp_mx_quant(xt, -2, "mxfp8", codes=xq.codes, scales=xq.scales, stream=stream)
            ts.append(ev.stop(stream))
            ev = _events(stream)
            lp.lp_linear_bwd(gc, None, wq, need_dw=False, grad_x=dx, stream=stream)
            ts.append(ev.stop(stream))
            ev = _events(stream)
            lp.lp_linear_bwd(gr, xq, None, need_dx=False, grad_w=dw, stream=stream)
            ts.append(ev.stop(stream))
            return ts
        standalone = []
    elif name == "fp8_hybrid":
        # Saved forward operands: E4M3 codes with their dynamic scales (set-up).
        # Per step: the gradient's delayed scale from its amax ring, E5M2
        # quantization recording the gradient's amax into the ring's next slot,
        # then dX and dW.
        per_set = M * N * 3 + (M * K + N * K) * 3
        nsets = max(1, min(16, math.ceil(ROTATE_BYTES / per_set)))
        for i in range(nsets):
            g = W.torch_normal_bf16((M, N), 1.0, 7800 + i, "cuda")
            saved = []
            for shape, sigma, seed in (((M, K), w.x_sigma, 7900 + i), ((N, K), w.w_sigma, 8000 + i)):
                t = W.torch_normal_bf16(shape, sigma, seed, "cuda")
                sc = lp.lp_scale_from_history(lp.lp_tensor_amax(t), "fp8t_e4m3")
                saved.append(lp.lp_tensor_quant(t, "fp8t_e4m3", sc))
            ring = torch.empty(W.AMAX_RING, dtype=torch.float32, device="cuda")
            ring.copy_(lp.lp_tensor_amax(g).expand(W.AMAX_RING))    # a first use fills the ring
            gq = lp.QTensor("fp8t_e5m2", torch.empty((1, M, N), dtype=torch.uint8, device="cuda"), None,
                            torch.empty(1, dtype=torch.float32, device="cuda"), shape=(1, M, N))
            dx = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
            dw = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
            sets.append((g, ring, gq, saved[0], saved[1], dx, dw))
        phases.append(Phase("tensor_quant_delayed grad E5M2", "tensor_quant", nbytes=M * N * 3))
        # dX and dW of the one E5M2 gradient in one call: one launch of both
        phases.append(Phase("linear_bwd dX+dW", "pt_pair_kernel", flops=4.0 * M * N * K, peak=PEAK_FP8_TFLOPS))

        def step(i, stream):
            g, ring, gq, xq, wq, dx, dw = sets[i % len(sets)]
            slot = (i // len(sets)) % W.AMAX_RING
            ts = []
            ev = _events(stream)
            lp.lp_tensor_quant_delayed(g, "fp8t_e5m2", ring, slot, codes=gq.codes, scale=gq.tensor_scale,
                                       stream=stream)
            ts.append(ev.stop(stream))
            ev = _events(stream)
            lp.lp_linear_bwd(gq, xq, wq, grad_x=dx, grad_w=dw, stream=stream)
            ts.append(ev.stop(stream))
            return ts
        standalone = []
    elif name == "mxfp4_forward":
        per_set = (M * K + N * K) * (0.5 + 1 / 16) + M * N * 2
        nsets = max(1, min(16, math.ceil(ROTATE_BYTES / per_set)))
        for i in range(nsets):
            xq = lp.lp_mx_quant(W.torch_normal_bf16((M, K), w.x_sigma, 8100 + i, "cuda"), -1, "mxfp4")
            wq = lp.lp_mx_quant(W.torch_normal_bf16((N, K), w.w_sigma, 8200 + i, "cuda"), -1, "mxfp4")
            sets.append((xq, wq, torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        phases.append(Phase("linear_fwd", "mx_fwd_kernel", flops=2.0 * M * N * K, peak=PEAK_FP4_TFLOPS))

        def step(i, stream):
            xq, wq, y = sets[i % len(sets)]
            ev = _events(stream)
            lp.lp_linear_fwd(xq, wq, y=y, stream=stream)
            return [ev.stop(stream)]
        standalone = []
    elif name == "nvfp4_forward":
        per_set = (M * K + N * K) * (0.5 + 1 / 16) + M * N * 2
        nsets = max(1, min(16, math.ceil(ROTATE_BYTES / per_set)))
        for i in range(nsets):
            c, s, ts = nvfp4_quant_torch(_randn((M, K), w.x_sigma, 8300 + i))
            xq = lp.QTensor("nvfp4", c, s, ts, shape=(1, M, K))
            c, s, ts = nvfp4_quant_torch(_randn((N, K), w.w_sigma, 8400 + i))
            wq = lp.QTensor("nvfp4", c, s, ts, shape=(1, N, K))
            sets.append((xq, wq, torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        # X is decoded once per step into a bf16 copy (lp_dequant), then the
        # forward contracts it with the NVFP4 weight, decoded inside the tiles.
        # Decoding X inside the contraction instead repeats it in each of the
        # 16 column tiles that read it; the results are bit-identical.
        xbf = torch.empty((1, M, K), dtype=torch.bfloat16, device="cuda")
        xbq = lp.QTensor("bf16", xbf, shape=(1, M, K))
        phases.append(Phase("dequant X", "dequant_nvfp4", nbytes=M * K * (0.5 + 1 / 16 + 2)))
        phases.append(Phase("linear_fwd (bf16 X)", "gemm_kernel", flops=2.0 * M * N * K))

        def step(i, stream):
            xq, wq, y = sets[i % len(sets)]
            ev = _events(stream)
            lp.lp_dequant(xq, xbf, stream=stream)
            t0 = ev.stop(stream)
            ev = _events(stream)
            lp.lp_linear_fwd(xbq, wq, y=y, stream=stream)
            return [t0, ev.stop(stream)]
        standalone = []
    elif name == "fp8_grouped_forward":
        offsets = torch.from_numpy(W.cumulative_ends(W.group_sizes(w))).cuda()
        per_set = M * K * 2 + w.groups * N * K + M * N * 2
        nsets = max(1, min(8, math.ceil(ROTATE_BYTES / per_set)))
        for i in range(nsets):
            x = W.torch_normal_bf16((M, K), w.x_sigma, 8500 + i, "cuda")
            c, s = fp8_b128_quant_torch(_randn((w.groups, N, K), w.w_sigma, 8600 + i))
            sets.append((lp.QTensor("bf16", x, shape=(1, M, K)), lp.QTensor("fp8_b128", c, s, shape=(w.groups, N, K)),
                         torch.empty((M, N), dtype=torch.bfloat16, device="cuda")))
        phases.append(Phase("grouped_fwd", "gemm_kernel", flops=2.0 * M * N * K))

        def step(i, stream):
            xq, wq, y = sets[i % len(sets)]
            ev = _events(stream)
            lp.lp_grouped_fwd(xq, wq, offsets, y=y, stream=stream)
            return [ev.stop(stream)]
        standalone = []
    else:
        raise SystemExit(f"unknown workload {name}")
    return w, phases, step, standalone


# Which phase of a step gets its HIP event pair: all of them (None), or only
# the one with this index.  Each event pair costs queue time on the stream,
# so the timed steps bracket only the dominant phase; the others are timed in
# an untimed pass before them.  `ctr` counts the pairs opened in the step.
_SEL = {"only": None, "ctr": 0}


class _events:
    def __init__(self, stream):
        k = _SEL["ctr"]
        _SEL["ctr"] += 1
        self.on = _SEL["only"] is None or _SEL["only"] == k
        if self.on:
            self.a = torch.cuda.Event(enable_timing=True)
            self.b = torch.cuda.Event(enable_timing=True)
            self.a.record(stream)

    def stop(self, stream):
        if not self.on:
            return None
        self.b.record(stream)
        return (self.a, self.b)


def _run(step, i, stream):
    _SEL["ctr"] = 0
    return step(i, stream)


def dequant_bytes(q) -> float:
    n = q.shape[0] * q.shape[1] * q.shape[2]
    per = {"mxfp4": 0.5 + 1 / 32, "nvfp4": 0.5 + 1 / 16, "fp8_b128": 1.0 + 4 / (128 * 128), "mxfp8": 1 + 1 / 32}
    return n * (per[q.fmt] + 2.0)


def time_standalone(lp, stream, q, reps=50):
    """Median time of lp_dequant of `q` (5 warmups, `reps` timed calls), with
    copies of the operand and of the output rotated through more than 1 GB
    so that no call finds its input or output in the 256 MiB Infinity Cache."""
    per = dequant_bytes(q)
    n = max(2, math.ceil(ROTATE_BYTES / per) + 1)
    copies = [q] + [lp.QTensor(q.fmt, q.codes.clone(), None if q.scales is None else q.scales.clone(),
                               q.tensor_scale, shape=q.shape, axis=q.axis) for _ in range(n - 1)]
    outs = [torch.empty(q.shape, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
    for i in range(5):
        lp.lp_dequant(copies[i % n], outs[i % n], stream=stream)
    evs = []
    for i in range(reps):
        ev = _events(stream)
        lp.lp_dequant(copies[(i + 5) % n], outs[(i + 5) % n], stream=stream)
        evs.append(ev.stop(stream))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    med = float(np.median(ms))
    gbs = per / (med * 1e-3) / 1e9
    return {"ms": round(med, 5), "p10_ms": round(float(np.percentile(ms, 10)), 5),
            "p90_ms": round(float(np.percentile(ms, 90)), 5), "GB/s": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "rotated_copies": n}


# ------------------------------------------------------------------ HBM traffic from committed counters

def kernel_source_digest() -> str:
    """Digest of every kernel source (the library's .hip, .hpp and .inc files)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_gemm_backward_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".hpp", ".inc")):
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM bytes per launch of the dominant kernel from profiles/, or None if
    absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sources") != kernel_source_digest():
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------ CPU baseline (oracle)

def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [os.cpu_count() or 1])
    except Exception:  # noqa: BLE001
        return os.cpu_count() or 1


class _Part:
    """One oracle kernel of the step on a sample: `fn` runs the sample, the
    whole step's share is `scale` times its time.  `blas` parts (the fp64
    contractions) are timed on one thread and on all of BLAS's threads; the
    others are numpy element-wise code, which runs on one thread either way,
    and are timed once."""

    def __init__(self, name, fn, scale, blas, sample):
        self.name, self.fn, self.scale, self.blas, self.sample = name, fn, scale, blas, sample


def _oracle_parts(name: str):
    """The step of workload `name` as oracle kernels on bounded samples."""
    from oracle import formats as F
    from oracle import gemm as O
    w = W.WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    rows = min(M, 256)
    parts = []
    if name == "mxfp8_deferred":
        gb = W.bf16_bits(W.normal_f32(w.number, "grad", (rows, N), 1.0))
        wb = W.bf16_bits(W.normal_f32(w.number, "w", (N, K), w.w_sigma))
        st = {}

        def qg():
            st["g"] = F.mx_quant(gb[None], -1, "e4m3")

        def qw():
            st["w"] = F.mx_quant(wb[None], -2, "e4m3")

        def dec_w():
            st["wd"] = F.dequant("mxfp8", *st["w"], axis=-2)[0]

        def dx():
            O.linear_dx(F.dequant("mxfp8", *st["g"], axis=-1)[0], st["wd"])
        parts += [_Part("mx_quant grad", qg, M / rows, False, f"{rows} of {M} gradient rows"),
                  _Part("mx_quant W", qw, w.groups, False, f"1 of {w.groups} experts' weights"),
                  _Part("decode W", dec_w, w.groups, False, f"1 of {w.groups} experts' weights"),
                  _Part("grouped dX (gradient decode + fp64 product)", dx, M / rows, True,
                        f"{rows} token rows against one expert's weight")]
        return parts, 2.0 * M * N * K
    if name == "mxfp8_dense":
        gb = W.bf16_bits(W.normal_f32(w.number, "grad", (rows, N), 1.0))
        xb = W.bf16_bits(W.normal_f32(w.number, "x", (rows, K), w.x_sigma))
        wb = W.bf16_bits(W.normal_f32(w.number, "w", (N, K), w.w_sigma))
        st = {}

        def qg():
            st["g1"] = F.mx_quant(gb[None], -1, "e4m3")
            st["g2"] = F.mx_quant(gb[None], -2, "e4m3")

        def qw():
            st["w"] = F.mx_quant(wb[None], -2, "e4m3")

        def qx():
            st["x"] = F.mx_quant(xb[None], -2, "e4m3")

        def dec_w():
            st["wd"] = F.dequant("mxfp8", *st["w"], axis=-2)[0]

        def dx():
            O.linear_dx(F.dequant("mxfp8", *st["g1"], axis=-1)[0], st["wd"])

        def dw():
            O.linear_dw(F.dequant("mxfp8", *st["g2"], axis=-2)[0], F.dequant("mxfp8", *st["x"], axis=-2)[0])
        parts += [_Part("mx_quant grad, both axes", qg, M / rows, False, f"{rows} of {M} gradient rows"),
                  _Part("mx_quant W", qw, 1, False, "whole weight"),
                  _Part("mx_quant X", qx, M / rows, False, f"{rows} of {M} input rows"),
                  _Part("decode W", dec_w, 1, False, "whole weight"),
                  _Part("dX (decode + fp64 product)", dx, M / rows, True, f"{rows} token rows"),
                  _Part("dW (decode + fp64 product)", dw, M / rows, True, f"{rows} token rows of the contraction")]
        return parts, 4.0 * M * N * K
    if name == "fp8_hybrid":
        from oracle import pertensor as PT
        gb = W.bf16_bits(W.normal_f32(w.number, "grad", (rows, N), 1.0))
        xb = W.bf16_bits(W.normal_f32(w.number, "x", (rows, K), w.x_sigma))
        wb = W.bf16_bits(W.normal_f32(w.number, "w", (N, K), w.w_sigma))
        ws_ = PT.scale_from_history([PT.amax(wb)], "e4m3")
        wc = PT.quantize(wb, "e4m3", ws_)
        xs = PT.scale_from_history([PT.amax(xb)], "e4m3")
        xc = PT.quantize(xb, "e4m3", xs)
        st = {}

        def q():
            hist = np.full(W.AMAX_RING, PT.amax(gb), np.float32)
            gs = PT.scale_from_history(hist, "e5m2")
            st["g"] = (PT.quantize(gb, "e5m2", gs), gs)
            PT.record(hist, 0, PT.amax(gb))

        def prod():
            gc, gs = st["g"]
            PT.linear_dx(gc, "e5m2", gs, wc, "e4m3", ws_)
            PT.linear_dw(gc, "e5m2", gs, xc, "e4m3", xs)
        parts += [_Part("tensor_quant_delayed grad E5M2", q, M / rows, False, f"{rows} of {M} gradient rows"),
                  _Part("dX + dW (fp64 products)", prod, M / rows, True, f"{rows} token rows")]
        return parts, 4.0 * M * N * K
    if name == "mxfp4_forward":
        x = W.normal_f32(w.number, "x", (rows, K), w.x_sigma)
        wt = W.normal_f32(w.number, "w", (N, K), w.w_sigma)
        xq, wq = F.quant_mxfp4_f32(x[None]), F.quant_mxfp4_f32(wt[None])
        st = {}

        def dec_w():
            st["w"] = F.dequant("mxfp4", *wq)[0]

        def dec_x():
            st["x"] = F.dequant("mxfp4", *xq)[0]

        def fwd():
            O.linear_fwd(st["x"], st["w"])
        parts += [_Part("dequant W", dec_w, 1, False, "whole weight"),
                  _Part("dequant X", dec_x, M / rows, False, f"{rows} of {M} input rows"),
                  _Part("forward (fp64 product)", fwd, M / rows, True, f"{rows} token rows")]
        return parts, 2.0 * M * N * K
    if name == "nvfp4_forward":
        xq = F.quant_nvfp4(W.with_outliers(W.normal_f32(w.number, "x", (rows, K), w.x_sigma), w.number, "x")[None])
        wq = F.quant_nvfp4(W.with_outliers(W.normal_f32(w.number, "w", (N, K), w.w_sigma), w.number, "w")[None])
        st = {}

        def dec_w():
            st["w"] = F.dequant("nvfp4", *wq)[0]

        def dec_x():
            st["x"] = F.dequant("nvfp4", *xq)[0]

        def fwd():
            O.linear_fwd(st["x"], st["w"])
        parts += [_Part("dequant W", dec_w, 1, False, "whole weight"),
                  _Part("dequant X", dec_x, M / rows, False, f"{rows} of {M} input rows"),
                  _Part("forward (fp64 product)", fwd, M / rows, True, f"{rows} token rows")]
        return parts, 2.0 * M * N * K
    if name == "fp8_grouped_forward":
        xb = W.bf16_bits(W.normal_f32(w.number, "x", (rows, K), w.x_sigma))
        wc, ws = F.quant_fp8_b128(W.normal_f32(w.number, "w", (1, N, K), w.w_sigma))
        st = {}

        def dec_w():
            st["w"] = F.dequant("fp8_b128", wc, ws)[0]

        def fwd():
            O.linear_fwd(xb, st["w"])
        # Every token row meets exactly one expert's weight: the cost per row
        # is that of one dense row, whatever the group sizes.
        parts += [_Part("dequant W", dec_w, w.groups, False, f"one of {w.groups} expert weights"),
                  _Part("grouped forward (fp64 product)", fwd, M / rows, True, f"{rows} token rows, one expert")]
        return parts, 2.0 * M * N * K
    # Saved packed operands (fp8_frozen, nvfp4_linear, mxfp4_grouped, mxfp4_tiny):
    # decode, then the fp64 products over sampled token rows.
    X, Wt, G = W.dense_inputs(w, M=rows)
    fmt = w.fmt
    quant = {"fp8_b128": F.quant_fp8_b128, "nvfp4": F.quant_nvfp4, "mxfp4": F.quant_mxfp4_f32}[fmt]
    wq = quant(Wt)
    xq = quant(X) if X is not None else None
    st = {}

    def deq(q):
        return F.dequant(fmt, q[0], q[1], q[2]) if fmt == "nvfp4" else F.dequant(fmt, q[0], q[1])

    def dw_dec():
        st["w"] = deq(wq)

    parts.append(_Part("dequant W", dw_dec, 1, False, "whole weight" + (f"s of {w.groups} experts" if w.grouped else "")))
    if xq is not None:
        def dx_dec():
            st["x"] = deq(xq)[0]
        parts.append(_Part("dequant X", dx_dec, M / rows, False, f"{rows} of {M} input rows"))

    def dx():
        O.rows_dx(G, st["w"][0], np.arange(rows))
    parts.append(_Part("dX (fp64 product)", dx, M / rows, True, f"{rows} token rows"))
    if w.need_dw:
        def dw():
            O.rows_dw(G, st["x"], np.arange(N))
        parts.append(_Part("dW (fp64 product)", dw, M / rows, True, f"{rows} token rows of the contraction"))
    return parts, 2.0 * M * N * K * (2 if w.need_dw else 1)


def cpu_baseline(name: str):
    """The oracle on a bounded sample of the workload's step, kernel by
    kernel: each kernel's sample time is scaled linearly to the whole step
    (token rows, or experts' weights).  The contractions run on one thread
    and on all of BLAS's threads; `value` is the whole step at all threads."""
    from threadpoolctl import threadpool_limits
    parts, flops = _oracle_parts(name)
    cores = _blas_threads()
    per = {}
    tot1 = totn = 0.0
    for part in parts:
        times = {}
        for nthreads in ((1, cores) if part.blas else (1,)):
            with threadpool_limits(limits=nthreads):
                t0 = time.perf_counter()
                part.fn()
                times[nthreads] = (time.perf_counter() - t0) * part.scale
        s1, sn = times[1], times.get(cores, times[1])
        tot1 += s1
        totn += sn
        per[part.name] = {"s_1_thread": round(s1, 3), f"s_{cores}_threads": round(sn, 3), "sample": part.sample,
                          "threads": "1 and all (BLAS)" if part.blas else "1 (numpy element-wise)"}
    return {"value": round(flops / totn / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": "; ".join(f"{p.name}: {p.sample}" for p in parts) + "; each scaled to the whole step",
            "seconds": round(totn, 3), "seconds_1_thread": round(tot1, 3),
            "value_1_thread": round(flops / tot1 / 1e12, 6), "cpu_model": _cpu_model(), "per_kernel": per}


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="mxfp8_deferred", choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-baseline leg")
    ap.add_argument("--unfused", action="store_true",
                    help="mxfp8_deferred: quantize the whole weight first (three calls) instead of lp_grouped_dx_deferred")
    a = ap.parse_args()
    global UNFUSED
    UNFUSED = a.unfused
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import fp8_gemm_backward_amd as lp
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        w, phases, step, standalone = build(lp, a.workload)
    torch.cuda.synchronize()

    for i in range(a.warmup):
        _run(step, i, stream)
    # Untimed pass with every phase bracketed: the per-phase times, and which
    # phase dominates.
    diag = [_run(step, a.warmup + i, stream) for i in range(min(a.steps, 50))]
    torch.cuda.synchronize()
    for r in diag:
        for ph, (e0, e1) in zip(phases, r):
            ph.ms.append(e0.elapsed_time(e1))
    di = int(np.argmax([np.mean(p.ms) for p in phases]))
    dom = phases[di]
    dom.ms = []
    _SEL["only"] = di
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = []
    for i in range(a.steps):
        recs.append(_run(step, a.warmup + i, stream)[di])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _SEL["only"] = None
    for e0, e1 in recs:
        dom.ms.append(e0.elapsed_time(e1))

    ms_step = elapsed / a.steps * 1e3
    flops = sum(p.flops for p in phases)
    value = flops / (ms_step * 1e-3) / 1e12
    dom_ms = float(np.mean(dom.ms))
    # The binding roof is the one that allows the longer time: MFMA
    # (flops / peak) or HBM (algorithmic bytes / 8 TB/s).
    hbm_bound = dom.nbytes and (not dom.flops or dom.nbytes / PEAK_HBM_GBS / 1e9 > dom.flops / dom.peak / 1e12)
    if not hbm_bound:
        achieved = dom.flops / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": dom.peak, "unit": "TFLOP/s",
                "frac": round(achieved / dom.peak, 4)}
    else:
        achieved = dom.nbytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    # The recorded traffic is that of the default step's dominant launch;
    # the three-call variant of the deferred step times another launch.
    roof["traffic"] = None if UNFUSED else committed_traffic(a.workload)
    roof["kernel"] = dom.kernel
    roof["launch_ms"] = round(dom_ms, 5)

    phase_rec = {}
    for p in phases:
        m = float(np.mean(p.ms))
        rec = {"ms": round(m, 5)}
        if p.flops:
            rec["TFLOP/s"] = round(p.flops / (m * 1e-3) / 1e12, 2)
            rec["frac_mfma"] = round(p.flops / (m * 1e-3) / 1e12 / p.peak, 4)
            rec["mfma_peak"] = p.peak
        if p.nbytes:
            rec["GB/s"] = round(p.nbytes / (m * 1e-3) / 1e9, 1)
            rec["frac_hbm"] = round(p.nbytes / (m * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        phase_rec[p.name] = rec
    hbm = {f"dequant {n}": time_standalone(lp, stream, q) for n, q in standalone}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "data": "synthetic",
        "dtype": "fp4" if w.name == "mxfp4_forward" else ("fp8" if w.fmt in ("mxfp8", "fp8t") else "bf16"),
        "config": {"workload": w.name, "format": w.fmt, "M": w.M, "N": w.N, "K": w.K, "groups": w.groups,
                   "grad_x": w.need_dx, "grad_w": w.need_dw, "global_batch": w.M, "parallelism": "none (1 GPU)",
                   **({"weight_quant": "three calls" if UNFUSED else f"inside the product for experts <= {FUSE_ROWS} tokens"}
                      if w.name == "mxfp8_deferred" else {})},
        "roofline": roof, "phases": phase_rec, "standalone_hbm": hbm,
    }
    if not a.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w.name)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
