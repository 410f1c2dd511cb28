"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This module draws random numbers and describes workload shapes.  It holds
none of the method's arithmetic: no format decoding, no quantization, no
products.  Values that the method consumes in bf16 are rounded from fp32 by
torch's CPU cast (a library conversion, neither the oracle nor the HIP path).

Workloads (the shapes and value distributions of the backward passes that
the source documents describe: a frozen FP8-E4M3 128x128-block linear as in "Train
adapters on top of FP8 weights", FP4 linear / grouped backward as in "Add
Autograd Backward Support for FP4 GEMM Custom Ops", and the deferred MXFP8
grouped backward of "perf: defer mxfp8 backward quantization"):

  mxfp4_tiny     X 64x128, W 128x128 N(0,1) -> MXFP4 along K; grad_out 64x128
  fp8_frozen     W 8192x2048 N(0,0.02) -> E4M3, fp32 scale per 128x128 block;
                 grad_out 4096x8192 N(0,1); dX only
  nvfp4_linear   X 8192x4096, W 4096x4096 N(0,1) with 1% outliers x10 ->
                 NVFP4 along K; grad_out 8192x4096 N(0,1); dX and dW
  mxfp4_grouped  8 experts, W 8x2048x4096, X 16384x4096 N(0,1) -> MXFP4;
                 group sizes ~ Multinomial(16384, Dirichlet(1)); dX and dW
  mxfp8_deferred 64 experts, W bf16 64x2048x7168 N(0,0.02), grad_out bf16
                 32768x2048 N(0,1); group sizes ~ Multinomial(32768, Zipf 1.1)
  mxfp8_dense    the dense form of the deferred MXFP8 backward (the page's
                 MXFP8MatMul.backward): X 8192x4096 N(0,1), W 4096x4096
                 N(0,0.02), grad_out 8192x4096 N(0,1), all bf16, quantized in
                 the backward; dX and dW
  fp8_hybrid     the per-tensor FP8 hybrid backward of "AstrAI fp8.py"
                 (_LinearFp8.backward): X 4096x1536 N(0,1) and W 6144x1536
                 N(0,0.02) saved as E4M3 with their dynamic scales; grad_out
                 4096x6144 N(0,1) bf16, quantized to E5M2 in the backward with
                 the delayed scale of a 16-entry amax ring; dX and dW.  The page
                 times a 0.67B model at batch 4x1024 without giving its layer
                 sizes: 4096 tokens and the FFN up-projection (1536 -> 6144) of
                 a GPT-style block with d = 1536 (12 * 24 * 1536^2 = 0.68B over
                 24 blocks) stand in for it.
  mxfp4_forward  the forward the FP4 backward pairs with ("Add Autograd Backward
                 Support for FP4 GEMM Custom Ops"): X 8192x4096 N(0,1) and W
                 4096x4096 N(0,1), both MXFP4 along K; y = X @ W^T
  nvfp4_forward  the same forward with NVFP4 operands and nvfp4_linear's
                 inputs (1% outliers x10); y = X @ W^T
  fp8_grouped_forward  the block-FP8 grouped forward of "Train adapters on top
                 of FP8 weights" (FP8GroupedMatmulFunction.forward): X bf16
                 16384x4096 N(0,1), W 8x2048x4096 N(0,0.02) -> E4M3 with an
                 fp32 scale per 128x128 block, group sizes as mxfp4_grouped
                 (Multinomial(16384, Dirichlet(1)))

Every tensor has its own PCG64 stream: SeedSequence(entropy=1000 + config
number, spawn_key=(tensor id,)), so a tensor's values do not depend on which
other tensors were drawn first.
"""
from __future__ import annotations

import dataclasses

import numpy as np

# Tensor ids for the per-tensor random streams.
_STREAM = {"x": 0, "w": 1, "grad": 2, "route": 3, "x_outlier": 4, "w_outlier": 5,
           "perm": 6, "grad_outlier": 7}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    number: int              # 1-based config number, also the seed offset
    fmt: str                 # saved-operand format: mxfp4 | nvfp4 | fp8_b128 | mxfp8
    M: int                   # tokens (rows of grad_out and X)
    N: int                   # layer output dim (cols of grad_out, rows of W)
    K: int                   # layer input dim
    groups: int = 0          # 0 = dense linear, else number of experts
    w_sigma: float = 1.0
    x_sigma: float = 1.0
    outliers: bool = False   # 1% of elements scaled by 10
    need_dx: bool = True
    need_dw: bool = True
    routing: str = ""        # dirichlet | zipf (grouped only)

    @property
    def grouped(self) -> bool:
        return self.groups > 0


WORKLOADS = {
    "mxfp4_tiny": Workload("mxfp4_tiny", 1, "mxfp4", M=64, N=128, K=128),
    "fp8_frozen": Workload("fp8_frozen", 2, "fp8_b128", M=4096, N=8192, K=2048,
                           w_sigma=0.02, need_dw=False),
    "nvfp4_linear": Workload("nvfp4_linear", 3, "nvfp4", M=8192, N=4096, K=4096,
                             outliers=True),
    "mxfp4_grouped": Workload("mxfp4_grouped", 4, "mxfp4", M=16384, N=2048, K=4096,
                              groups=8, routing="dirichlet"),
    "mxfp8_deferred": Workload("mxfp8_deferred", 5, "mxfp8", M=32768, N=2048, K=7168,
                               groups=64, w_sigma=0.02, need_dw=False, routing="zipf"),
    "mxfp8_dense": Workload("mxfp8_dense", 6, "mxfp8", M=8192, N=4096, K=4096, w_sigma=0.02),
    "fp8_hybrid": Workload("fp8_hybrid", 7, "fp8t", M=4096, N=6144, K=1536, w_sigma=0.02),
    "mxfp4_forward": Workload("mxfp4_forward", 8, "mxfp4", M=8192, N=4096, K=4096, need_dx=False, need_dw=False),
    "nvfp4_forward": Workload("nvfp4_forward", 9, "nvfp4", M=8192, N=4096, K=4096, outliers=True,
                              need_dx=False, need_dw=False),
    "fp8_grouped_forward": Workload("fp8_grouped_forward", 10, "fp8_b128", M=16384, N=2048, K=4096, groups=8,
                                    w_sigma=0.02, need_dx=False, need_dw=False, routing="dirichlet"),
}

AMAX_RING = 16               # amax history length of the delayed-scaling recipe


def rng(number: int, tensor: str) -> np.random.Generator:
    """The independent PCG64 stream of one tensor of workload `number`."""
    seq = np.random.SeedSequence(entropy=1000 + number, spawn_key=(_STREAM[tensor],))
    return np.random.Generator(np.random.PCG64(seq))


def normal_f32(number: int, tensor: str, shape, sigma: float) -> np.ndarray:
    """N(0, sigma) draws in fp32."""
    g = rng(number, tensor)
    return (g.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma))


def with_outliers(values: np.ndarray, number: int, tensor: str,
                  frac: float = 0.01, factor: float = 10.0) -> np.ndarray:
    """Scale a Bernoulli(frac) subset of the elements by `factor`."""
    g = rng(number, tensor + "_outlier")
    mask = g.random(size=values.shape, dtype=np.float32) < np.float32(frac)
    out = values.copy()
    out[mask] *= np.float32(factor)
    return out


def bf16_bits(values_f32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) through torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(values_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def dirichlet_sizes(number: int, total: int, groups: int) -> np.ndarray:
    """Expert sizes ~ Multinomial(total, Dirichlet(1,...,1))."""
    g = rng(number, "route")
    p = g.dirichlet(np.ones(groups))
    return g.multinomial(total, p).astype(np.int64)


def zipf_sizes(number: int, total: int, groups: int, s: float = 1.1) -> np.ndarray:
    """Expert sizes ~ Multinomial(total, pmf proportional to r^-s), expert ids
    shuffled by a seeded permutation."""
    g = rng(number, "route")
    r = np.arange(1, groups + 1, dtype=np.float64)
    p = r ** (-s)
    p /= p.sum()
    sizes = g.multinomial(total, p).astype(np.int64)
    perm = rng(number, "perm").permutation(groups)
    return sizes[perm]


def group_sizes(w: Workload, M: int | None = None) -> np.ndarray:
    M = w.M if M is None else M
    if w.routing == "dirichlet":
        return dirichlet_sizes(w.number, M, w.groups)
    if w.routing == "zipf":
        return zipf_sizes(w.number, M, w.groups)
    raise ValueError(f"workload {w.name} is not grouped")


def cumulative_ends(sizes) -> np.ndarray:
    """int32 cumulative end offsets, one per group (the first group starts at 0)."""
    return np.cumsum(np.asarray(sizes, dtype=np.int64)).astype(np.int32)


def force_empty(sizes: np.ndarray, group: int) -> np.ndarray:
    """Move every token of `group` to the largest group, leaving `group` empty."""
    s = sizes.copy()
    big = int(np.argmax(np.where(np.arange(len(s)) == group, -1, s)))
    s[big] += s[group]
    s[group] = 0
    return s


def dense_inputs(w: Workload, M: int | None = None, N: int | None = None,
                 K: int | None = None):
    """fp32 X [M,K], fp32 W [N,K] (or [G,N,K]) and bf16-bit grad_out [M,N].

    Sizes default to the workload's own; smaller overrides keep its
    distributions for cases the oracle finishes quickly.
    """
    M = w.M if M is None else M
    N = w.N if N is None else N
    K = w.K if K is None else K
    wshape = (w.groups, N, K) if w.grouped else (N, K)
    W = normal_f32(w.number, "w", wshape, w.w_sigma)
    X = normal_f32(w.number, "x", (M, K), w.x_sigma) if w.need_dw else None
    if w.outliers:
        W = with_outliers(W, w.number, "w")
        if X is not None:
            X = with_outliers(X, w.number, "x")
    G = bf16_bits(normal_f32(w.number, "grad", (M, N), 1.0))
    return X, W, G


def torch_normal_bf16(shape, sigma: float, seed: int, device):
    """N(0, sigma) bf16 tensor drawn by torch's generator on `device` (used
    where a full-size tensor is too large to draw on the host quickly)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return (t * sigma).to(torch.bfloat16)
