"""MI355X-native 4-bit block-quantized linear layer.

    y = linear(x, wq, scales)        # y[M, N] = x[M, K] . dequant(Wq[N, K])^T

A thin binding over libq4.so (include/q4.h): every step runs in the HIP
kernels; this module only checks tensors and passes device pointers and the
current HIP stream.  PyTorch supplies device memory and streams.

Format: blocks of 32 weights along K with one fp16 scale d each, 4-bit codes
q in 0..15, weight (q - 8) * d; ``wq`` is uint8 [N, K/2] (low nibble = even
k), ``scales`` is float16 [N, K/32], ``x`` is bfloat16 or float16 [M, K],
``y`` is float32 [M, N].
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import KERNELS, Q4Error

__all__ = ["linear", "pack", "workspace_bytes", "get_crossover", "set_crossover",
           "segments", "Q4Error", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtypes, ndim: int, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor (got %s)" % (name, t.device))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if t.dim() != ndim:
        raise ValueError("%s must be %d-D, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def workspace_bytes(M: int, N: int, K: int, kernel: str = "auto") -> int:
    return int(_lib.load().q4_workspace_bytes(M, N, K, KERNELS[kernel]))


def linear(x: torch.Tensor, wq: torch.Tensor, scales: torch.Tensor, out: torch.Tensor | None = None,
           kernel: str = "auto", workspace: torch.Tensor | bool | None = True) -> torch.Tensor:
    """y = x . dequant(wq, scales)^T on the current stream of x's device.

    kernel: "auto" (crossover rule), "gemv" or "gemm" (forced).  The result
    bits do not depend on this choice.
    workspace: True (default) allocates the workspace the matrix-matrix
    kernel can use; False/None runs without one; a uint8 tensor is used as
    given.
    """
    lib = _lib.load()
    _need(x, "x", (torch.bfloat16, torch.float16), 2)
    dev = x.device
    _need(wq, "wq", (torch.uint8,), 2, dev)
    _need(scales, "scales", (torch.float16,), 2, dev)
    M, K = x.shape
    N = wq.shape[0]
    if tuple(wq.shape) != (N, K // 2) or tuple(scales.shape) != (N, K // 32):
        raise ValueError("shape mismatch: x %s, wq %s, scales %s"
                         % (tuple(x.shape), tuple(wq.shape), tuple(scales.shape)))
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", (torch.float32,), 2, dev)
        if tuple(out.shape) != (M, N):
            raise ValueError("out must be [%d, %d]" % (M, N))
    if kernel not in KERNELS:
        raise ValueError("kernel must be one of %s" % sorted(KERNELS))
    ws_ptr, ws_len = None, 0
    if isinstance(workspace, torch.Tensor):
        _need(workspace, "workspace", (torch.uint8,), 1, dev)
        ws_ptr, ws_len = workspace.data_ptr(), workspace.numel()
    elif workspace:
        need = lib.q4_workspace_bytes(M, N, K, KERNELS[kernel])
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            ws_ptr, ws_len = ws.data_ptr(), need
    dtype = _lib.Q4_BF16 if x.dtype == torch.bfloat16 else _lib.Q4_F16
    with torch.cuda.device(dev):
        st = lib.q4_linear_ex(x.data_ptr(), dtype, wq.data_ptr(), scales.data_ptr(), out.data_ptr(),
                              M, N, K, KERNELS[kernel], ws_ptr, ws_len, _stream(dev))
    _lib.check(st, "q4_linear_ex")
    return out


def pack(codes: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """codes uint8 [N, K] (low 4 bits used) -> packed uint8 [N, K/2]."""
    lib = _lib.load()
    _need(codes, "codes", (torch.uint8,), 2)
    N, K = codes.shape
    dev = codes.device
    if out is None:
        out = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    else:
        _need(out, "out", (torch.uint8,), 2, dev)
        if tuple(out.shape) != (N, K // 2):
            raise ValueError("out must be [%d, %d]" % (N, K // 2))
    with torch.cuda.device(dev):
        st = lib.q4_pack(codes.data_ptr(), out.data_ptr(), N, K, _stream(dev))
    _lib.check(st, "q4_pack")
    return out


def get_crossover() -> int:
    return int(_lib.load().q4_get_crossover())


def set_crossover(T: int) -> None:
    _lib.check(_lib.load().q4_set_crossover(int(T)), "q4_set_crossover")


def segments(K: int) -> int:
    return int(_lib.load().q4_segments(int(K)))
