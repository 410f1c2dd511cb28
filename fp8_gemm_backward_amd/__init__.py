"""Backward of block-scaled low-precision linear and grouped matmuls on MI355X.

A thin Python binding over the C-ABI library `liblp.so` (declared in
`include/lp.h`).  The functions below keep the C names; they only marshal
torch tensors (device memory) and the current HIP stream into the C calls.
Every step of the computation runs in the library's HIP kernels; there is no
fallback, and importing this package fails if the library is not built
(`python fp8_gemm_backward_amd/build.py`).

Formats (see include/lp.h): "bf16", "mxfp4", "nvfp4", "fp8_b128", "mxfp8",
and the per-tensor scaled "fp8t_e4m3", "fp8t_e5m2".
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import re
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblp.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "lp.h")

FMT = {"bf16": 0, "mxfp4": 1, "nvfp4": 2, "fp8_b128": 3, "mxfp8": 4, "fp8t_e4m3": 5, "fp8t_e5m2": 6}
STATUS = {0: "LP_OK", 1: "LP_ERR_NULL", 2: "LP_ERR_SHAPE", 3: "LP_ERR_FORMAT", 4: "LP_ERR_ALIGN",
          5: "LP_ERR_HIP"}


class LpError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class _QTensorC(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("scale_axis", ctypes.c_int32), ("batch", ctypes.c_int64),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("codes", ctypes.c_void_p),
                ("scales", ctypes.c_void_p), ("tensor_scale", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python fp8_gemm_backward_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(_QTensorC)
    v = ctypes.c_void_p
    i64, i32 = ctypes.c_int64, ctypes.c_int32
    lib.lp_dequant.argtypes = [P, v, v]
    lib.lp_mx_quant.argtypes = [v, i64, i64, i64, i32, i32, v, v, v]
    lib.lp_mx_quant_dual.argtypes = [v, i64, i64, i64, i32, v, v, v, v, v]
    lib.lp_linear_bwd.argtypes = [P, P, P, v, v, v]
    lib.lp_grouped_bwd.argtypes = [P, P, P, v, i64, v, v, v]
    lib.lp_linear_bwd_workspace.argtypes = [P, P, P, v, v, ctypes.POINTER(ctypes.c_size_t)]
    lib.lp_linear_bwd_ws.argtypes = [P, P, P, v, v, v, ctypes.c_size_t, v]
    lib.lp_linear_bwd_noalloc.argtypes = [P, P, P, v, v, v]
    lib.lp_grouped_dx_deferred.argtypes = [P, v, i64, v, i64, i64, v, v, v, v]
    lib.lp_tensor_amax.argtypes = [v, i64, v, v]
    lib.lp_tensor_quant.argtypes = [v, i64, i32, v, v, v, v]
    lib.lp_scale_from_history.argtypes = [v, i32, i32, i32, v, v]
    lib.lp_tensor_quant_delayed.argtypes = [v, i64, i32, v, i32, i32, i32, v, v, v]
    lib.lp_linear_fwd.argtypes = [P, P, v, v]
    lib.lp_grouped_fwd.argtypes = [P, P, v, i64, v, v]
    lib.lp_status_string.argtypes = [i32]
    lib.lp_status_string.restype = ctypes.c_char_p
    for f in ("lp_dequant", "lp_mx_quant", "lp_mx_quant_dual", "lp_linear_bwd", "lp_grouped_bwd",
              "lp_linear_bwd_workspace", "lp_linear_bwd_ws", "lp_linear_bwd_noalloc", "lp_grouped_dx_deferred", "lp_tensor_amax", "lp_tensor_quant",
              "lp_scale_from_history", "lp_linear_fwd", "lp_grouped_fwd", "lp_tensor_quant_delayed"):
        getattr(lib, f).restype = ctypes.c_int32
    return lib


lib = _load()


_CODE_BITS = {"bf16": 16, "mxfp4": 4, "nvfp4": 4, "fp8_b128": 8, "mxfp8": 8, "fp8t_e4m3": 8, "fp8t_e5m2": 8}


def _scale_bytes(fmt: str, axis: int, b: int, r: int, c: int) -> int:
    """Bytes of a tensor's block scales (include/lp.h, formats)."""
    if fmt == "mxfp4" or (fmt == "mxfp8" and axis == -1):
        return b * r * (c // 32)
    if fmt == "mxfp8":
        return b * (r // 32) * c
    if fmt == "nvfp4":
        return b * r * (c // 16)
    if fmt == "fp8_b128":
        return b * (-(-r // 128)) * (-(-c // 128)) * 4
    return 0


def _device(t: Optional[torch.Tensor], name: str, nbytes: int, dtype=None) -> None:
    """A tensor the library reads or writes `nbytes` of: on the GPU,
    contiguous, large enough (and of `dtype` where its element count is what
    the call passes).  Checked here because the C calls take bare pointers:
    a host pointer or a short buffer would reach a kernel as it is."""
    if nbytes <= 0:
        return
    if t is None:
        raise ValueError(f"{name}: a device tensor of {nbytes} bytes is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor, not on {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, the call needs {nbytes}")


def header_functions() -> list[str]:
    """Names of the functions declared in include/lp.h."""
    text = open(HEADER_PATH).read()
    return re.findall(r"^\s*(?:lp_status|const char\*)\s+(lp_\w+)\s*\(", text, re.M)


@dataclasses.dataclass
class QTensor:
    """A (possibly block-scaled) tensor of logical shape [batch, rows, cols].

    codes: bf16 values (fmt "bf16"), uint8 E4M3 codes, or uint8 packed E2M1
    pairs; scales: uint8 E8M0 / E4M3 bytes or float32 block scales; for
    NVFP4 and the per-tensor FP8 formats `tensor_scale` is a one-element
    float32 device tensor.
    """
    fmt: str
    codes: torch.Tensor
    scales: Optional[torch.Tensor] = None
    tensor_scale: Optional[torch.Tensor] = None
    shape: tuple = ()
    axis: int = -1

    def __post_init__(self):
        if not self.shape:
            s = tuple(self.codes.shape)
            cols = s[-1] * (2 if self.fmt in ("mxfp4", "nvfp4") else 1)
            self.shape = (s[0] if len(s) == 3 else 1, s[-2], cols)
        if len(self.shape) == 2:
            self.shape = (1,) + tuple(self.shape)

    @property
    def rows(self) -> int:
        return self.shape[1]

    @property
    def cols(self) -> int:
        return self.shape[2]

    def c(self) -> _QTensorC:
        b, r, c = self.shape
        n = b * r * c
        _device(self.codes, f"{self.fmt} codes", n * _CODE_BITS[self.fmt] // 8)
        _device(self.scales, f"{self.fmt} scales", _scale_bytes(self.fmt, self.axis, b, r, c))
        if self.fmt in ("nvfp4", "fp8t_e4m3", "fp8t_e5m2"):
            _device(self.tensor_scale, f"{self.fmt} tensor scale", 4 if n else 0, torch.float32)

        def ptr(t):
            return None if t is None else t.data_ptr()
        return _QTensorC(FMT[self.fmt], self.axis, self.shape[0], self.shape[1], self.shape[2],
                         ptr(self.codes), ptr(self.scales), ptr(self.tensor_scale))


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(st: int, where: str):
    if st != 0:
        raise LpError(st, where)


def lp_dequant(src: QTensor, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode `src` to bf16 [batch, rows, cols] (bit-exact)."""
    if out is None:
        out = torch.empty(src.shape, dtype=torch.bfloat16, device=src.codes.device)
    q = src.c()
    _device(out, "out", 2 * src.shape[0] * src.shape[1] * src.shape[2])
    _check(lib.lp_dequant(ctypes.byref(q), out.data_ptr(), _stream(stream)), "lp_dequant")
    return out


def lp_mx_quant(src: torch.Tensor, axis: int, fmt: str = "mxfp8", codes: Optional[torch.Tensor] = None,
                scales: Optional[torch.Tensor] = None, stream=None) -> QTensor:
    """MX-quantize a bf16 tensor [batch, rows, cols] (or [rows, cols]) along
    `axis` (-1 or -2) to "mxfp8" or "mxfp4"."""
    shape = tuple(src.shape) if src.dim() == 3 else (1,) + tuple(src.shape)
    b, r, c = shape
    dev = src.device
    if codes is None:
        codes = torch.empty((b, r, c if fmt == "mxfp8" else c // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        sshape = (b, r, c // 32) if axis == -1 else (b, r // 32, c)
        scales = torch.empty(sshape, dtype=torch.uint8, device=dev)
    n = b * r * c
    _device(src, "src", 2 * n, torch.bfloat16)
    _device(codes, "codes", n if fmt == "mxfp8" else n // 2)
    _device(scales, "scales", _scale_bytes(fmt, axis, b, r, c))
    _check(lib.lp_mx_quant(src.data_ptr(), b, r, c, axis, FMT[fmt], codes.data_ptr(), scales.data_ptr(),
                           _stream(stream)), "lp_mx_quant")
    return QTensor(fmt, codes, scales, None, shape, axis)


def lp_mx_quant_dual(src: torch.Tensor, fmt: str = "mxfp8", stream=None) -> tuple:
    """MX-quantize a bf16 tensor [batch, rows, cols] (or [rows, cols]) along
    both axes in one pass: (copy scaled along -1, copy scaled along -2)."""
    shape = tuple(src.shape) if src.dim() == 3 else (1,) + tuple(src.shape)
    b, r, c = shape
    dev = src.device
    cb = c if fmt == "mxfp8" else c // 2
    _device(src, "src", 2 * b * r * c, torch.bfloat16)
    codes_c = torch.empty((b, r, cb), dtype=torch.uint8, device=dev)
    scales_c = torch.empty((b, r, c // 32), dtype=torch.uint8, device=dev)
    codes_r = torch.empty((b, r, cb), dtype=torch.uint8, device=dev)
    scales_r = torch.empty((b, r // 32, c), dtype=torch.uint8, device=dev)
    _check(lib.lp_mx_quant_dual(src.data_ptr(), b, r, c, FMT[fmt], codes_c.data_ptr(), scales_c.data_ptr(),
                                codes_r.data_ptr(), scales_r.data_ptr(), _stream(stream)), "lp_mx_quant_dual")
    return QTensor(fmt, codes_c, scales_c, None, shape, -1), QTensor(fmt, codes_r, scales_r, None, shape, -2)


def lp_tensor_amax(src: torch.Tensor, amax: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """max |x| of a bf16 tensor into a float32 device scalar (`amax` may be a
    one-element view into an amax history)."""
    if amax is None:
        amax = torch.empty(1, dtype=torch.float32, device=src.device)
    _device(src, "src", 2 * src.numel(), torch.bfloat16)
    _device(amax, "amax", 4, torch.float32)
    _check(lib.lp_tensor_amax(src.data_ptr(), src.numel(), amax.data_ptr(), _stream(stream)), "lp_tensor_amax")
    return amax


def lp_tensor_quant(src: torch.Tensor, fmt: str, scale: torch.Tensor, amax: Optional[torch.Tensor] = None,
                    codes: Optional[torch.Tensor] = None, stream=None) -> QTensor:
    """Per-tensor FP8 quantization ("fp8t_e4m3" / "fp8t_e5m2") of a bf16
    tensor [batch, rows, cols] (or [rows, cols]) with the float32 device
    scalar `scale`; the input's amax goes to `amax` when given."""
    shape = tuple(src.shape) if src.dim() == 3 else (1,) + tuple(src.shape)
    if codes is None:
        codes = torch.empty(shape, dtype=torch.uint8, device=src.device)
    _device(src, "src", 2 * src.numel(), torch.bfloat16)
    _device(codes, "codes", src.numel())
    _device(scale, "scale", 4, torch.float32)
    if amax is not None:
        _device(amax, "amax", 4, torch.float32)
    _check(lib.lp_tensor_quant(src.data_ptr(), src.numel(), FMT[fmt], scale.data_ptr(), codes.data_ptr(),
                               None if amax is None else amax.data_ptr(), _stream(stream)), "lp_tensor_quant")
    return QTensor(fmt, codes, None, scale, shape, -1)


def lp_tensor_quant_delayed(src: torch.Tensor, fmt: str, history: torch.Tensor, slot: int, margin: int = 0,
                            codes: Optional[torch.Tensor] = None, scale: Optional[torch.Tensor] = None,
                            stream=None) -> QTensor:
    """Delayed scaling in one call: scale from `history` (float32 device
    ring), quantization with it, the input's amax into history[slot]."""
    shape = tuple(src.shape) if src.dim() == 3 else (1,) + tuple(src.shape)
    if codes is None:
        codes = torch.empty(shape, dtype=torch.uint8, device=src.device)
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=src.device)
    _device(src, "src", 2 * src.numel(), torch.bfloat16)
    _device(codes, "codes", src.numel())
    _device(history, "history", 4 * max(history.numel(), 1), torch.float32)
    _device(scale, "scale", 4, torch.float32)
    _check(lib.lp_tensor_quant_delayed(src.data_ptr(), src.numel(), FMT[fmt], history.data_ptr(), history.numel(),
                                       slot, margin, codes.data_ptr(), scale.data_ptr(), _stream(stream)),
           "lp_tensor_quant_delayed")
    return QTensor(fmt, codes, None, scale, shape, -1)


def lp_scale_from_history(history: torch.Tensor, fmt: str, margin: int = 0, scale: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """Per-tensor scale (float32 device scalar) from a float32 amax history."""
    if scale is None:
        scale = torch.empty(1, dtype=torch.float32, device=history.device)
    _device(history, "history", 4 * max(history.numel(), 1), torch.float32)
    _device(scale, "scale", 4, torch.float32)
    _check(lib.lp_scale_from_history(history.data_ptr(), history.numel(), FMT[fmt], margin, scale.data_ptr(),
                                     _stream(stream)), "lp_scale_from_history")
    return scale


def lp_linear_bwd(grad_out: QTensor, x: Optional[QTensor], w: Optional[QTensor], need_dx: bool = True,
                  need_dw: bool = True, grad_x: Optional[torch.Tensor] = None,
                  grad_w: Optional[torch.Tensor] = None, stream=None, workspace: Optional[torch.Tensor] = None):
    """(grad_X [M,K] or None, grad_W [N,K] or None) of a linear layer.
    `workspace`: a zero-filled uint8 device tensor of at least
    lp_linear_bwd_workspace(...) bytes lets the call split its contraction
    (lp_linear_bwd_ws); None calls lp_linear_bwd."""
    M, N = grad_out.rows, grad_out.cols
    K = (w if need_dx else x).cols
    dev = grad_out.codes.device
    if need_dx and grad_x is None:
        grad_x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if need_dw and grad_w is None:
        grad_w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    if need_dx:
        _device(grad_x, "grad_x", 2 * M * K)
    if need_dw:
        _device(grad_w, "grad_w", 2 * N * K)
    if workspace is not None:
        _device(workspace, "workspace", 1)
    g = grad_out.c()
    xc = x.c() if x is not None else None
    wc = w.c() if w is not None else None
    args = (ctypes.byref(g), ctypes.byref(xc) if xc else None, ctypes.byref(wc) if wc else None,
            grad_x.data_ptr() if need_dx else None, grad_w.data_ptr() if need_dw else None)
    if workspace is None:
        st = lib.lp_linear_bwd(*args, _stream(stream))
        _check(st, "lp_linear_bwd")
    else:
        st = lib.lp_linear_bwd_ws(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  _stream(stream))
        _check(st, "lp_linear_bwd_ws")
    return (grad_x if need_dx else None), (grad_w if need_dw else None)


def lp_linear_bwd_noalloc(grad_out: QTensor, x: Optional[QTensor], w: Optional[QTensor], need_dx: bool = True,
                          need_dw: bool = True, grad_x: Optional[torch.Tensor] = None,
                          grad_w: Optional[torch.Tensor] = None, stream=None):
    """lp_linear_bwd with the split workspace held inside the library (no
    device allocation by the call; outputs are allocated here only when not
    given)."""
    M, N = grad_out.rows, grad_out.cols
    K = (w if need_dx else x).cols
    dev = grad_out.codes.device
    if need_dx and grad_x is None:
        grad_x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if need_dw and grad_w is None:
        grad_w = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    if need_dx:
        _device(grad_x, "grad_x", 2 * M * K)
    if need_dw:
        _device(grad_w, "grad_w", 2 * N * K)
    g = grad_out.c()
    xc = x.c() if x is not None else None
    wc = w.c() if w is not None else None
    st = lib.lp_linear_bwd_noalloc(ctypes.byref(g), ctypes.byref(xc) if xc else None,
                                   ctypes.byref(wc) if wc else None, grad_x.data_ptr() if need_dx else None,
                                   grad_w.data_ptr() if need_dw else None, _stream(stream))
    _check(st, "lp_linear_bwd_noalloc")
    return (grad_x if need_dx else None), (grad_w if need_dw else None)


def lp_grouped_dx_deferred(grad_out: QTensor, w: torch.Tensor, offsets: torch.Tensor, fuse_rows: int = 1536,
                           grad_x: Optional[torch.Tensor] = None, w_codes: Optional[torch.Tensor] = None,
                           w_scales: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """grad_X of the deferred MXFP8 recipe: grad_out (MXFP8 along -1) times
    the bf16 weight w [G, N, K] quantized to MXFP8 along N; groups of at most
    fuse_rows rows quantize their weight inside the product.  w_codes /
    w_scales (the weight's MXFP8 copy for the larger groups) are allocated
    here when not given and fuse_rows < M."""
    G, N, K = w.shape
    M = grad_out.rows
    dev = grad_out.codes.device
    if grad_x is None:
        grad_x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if fuse_rows < M or N % 512 or K % 32:
        if w_codes is None:
            w_codes = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
        if w_scales is None:
            w_scales = torch.empty((G, N // 32, K), dtype=torch.uint8, device=dev)
        _device(w_codes, "w_codes", G * N * K)
        _device(w_scales, "w_scales", G * (N // 32) * K)
    _device(w, "w", 2 * G * N * K, torch.bfloat16)
    _device(offsets, "offsets", 4 * G, torch.int32)
    _device(grad_x, "grad_x", 2 * M * K)
    g = grad_out.c()
    st = lib.lp_grouped_dx_deferred(ctypes.byref(g), w.data_ptr(), K, offsets.data_ptr(), G, fuse_rows,
                                    grad_x.data_ptr(), None if w_codes is None else w_codes.data_ptr(),
                                    None if w_scales is None else w_scales.data_ptr(), _stream(stream))
    _check(st, "lp_grouped_dx_deferred")
    return grad_x


def lp_linear_bwd_workspace(grad_out: QTensor, x: Optional[QTensor], w: Optional[QTensor], need_dx: bool = True,
                            need_dw: bool = True) -> int:
    """Workspace bytes lp_linear_bwd_ws can use for this call (0: it does not split)."""
    g = grad_out.c()
    xc = x.c() if x is not None else None
    wc = w.c() if w is not None else None
    n = ctypes.c_size_t(0)
    st = lib.lp_linear_bwd_workspace(ctypes.byref(g), ctypes.byref(xc) if xc else None,
                                     ctypes.byref(wc) if wc else None, 1 if need_dx else None,
                                     1 if need_dw else None, ctypes.byref(n))
    _check(st, "lp_linear_bwd_workspace")
    return n.value


def lp_grouped_bwd(grad_out: QTensor, x: Optional[QTensor], w: Optional[QTensor], offsets: torch.Tensor,
                   need_dx: bool = True, need_dw: bool = True, grad_x: Optional[torch.Tensor] = None,
                   grad_w: Optional[torch.Tensor] = None, stream=None):
    """(grad_X [M,K] or None, grad_W [G,N,K] or None) of a grouped matmul.
    Rows of grad_X at or past offsets[-1] are left as they were in `grad_x`."""
    M, N = grad_out.rows, grad_out.cols
    G = offsets.numel()
    K = (w if need_dx else x).cols
    dev = grad_out.codes.device
    if need_dx and grad_x is None:
        grad_x = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    if need_dw and grad_w is None:
        grad_w = torch.empty((G, N, K), dtype=torch.bfloat16, device=dev)
    if need_dx:
        _device(grad_x, "grad_x", 2 * M * K)
    if need_dw:
        _device(grad_w, "grad_w", 2 * G * N * K)
    _device(offsets, "offsets", 4 * G, torch.int32)
    g = grad_out.c()
    xc = x.c() if x is not None else None
    wc = w.c() if w is not None else None
    st = lib.lp_grouped_bwd(ctypes.byref(g), ctypes.byref(xc) if xc else None, ctypes.byref(wc) if wc else None,
                            offsets.data_ptr(), G, grad_x.data_ptr() if need_dx else None,
                            grad_w.data_ptr() if need_dw else None, _stream(stream))
    _check(st, "lp_grouped_bwd")
    return (grad_x if need_dx else None), (grad_w if need_dw else None)


def lp_linear_fwd(x: QTensor, w: QTensor, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y [M, N] = x @ w^T: both "mxfp4" or both "mxfp8" (scaled along k),
    both "nvfp4", or a "bf16" x with a "bf16", "fp8_b128" or "nvfp4" weight."""
    if y is None:
        y = torch.empty((x.rows, w.rows), dtype=torch.bfloat16, device=x.codes.device)
    _device(y, "y", 2 * x.rows * w.rows)
    xc, wc = x.c(), w.c()
    _check(lib.lp_linear_fwd(ctypes.byref(xc), ctypes.byref(wc), y.data_ptr(), _stream(stream)), "lp_linear_fwd")
    return y


def lp_grouped_fwd(x: QTensor, w: QTensor, offsets: torch.Tensor, y: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """y [M, N]: rows of group g are x[rows] @ w[g]^T; rows at or past
    offsets[-1] are left as they were in `y`."""
    if y is None:
        y = torch.empty((x.rows, w.rows), dtype=torch.bfloat16, device=x.codes.device)
    _device(y, "y", 2 * x.rows * w.rows)
    _device(offsets, "offsets", 4 * offsets.numel(), torch.int32)
    xc, wc = x.c(), w.c()
    _check(lib.lp_grouped_fwd(ctypes.byref(xc), ctypes.byref(wc), offsets.data_ptr(), offsets.numel(), y.data_ptr(),
                              _stream(stream)), "lp_grouped_fwd")
    return y


def lp_status_string(status: int) -> str:
    return lib.lp_status_string(status).decode()
