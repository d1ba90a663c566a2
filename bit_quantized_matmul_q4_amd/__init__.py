"""MI355X-native 4-bit block-quantized linear layer.

    w = pack(codes, scales)           # canonical -> the library's packed form
    y = linear(x, w)                  # y[M, N] = x[M, K] . dequant(W[N, K])^T

A thin binding over libq4.so (include/q4.h): every step runs in the HIP
kernels; this module only checks tensors and passes device pointers and the
current HIP stream.  PyTorch supplies device memory and streams.

Format: blocks of 32 weights along K with one fp16 scale d each, 4-bit codes
q in 0..15, weight (q - 8) * d.  ``quantize`` makes codes and scales from
dense weights (absmax / 7 scaling, include/q4.h).  Canonical inputs: ``codes`` uint8 [N, K]
(one code per byte), ``scales`` float16 [N, K/32].  ``pack`` turns them into
the packed (tiled) form held by a ``Q4Weight``; ``x`` is bfloat16 or float16
[M, K], ``y`` is float32 [M, N].
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import KERNELS, Q4Error

__all__ = ["Q4Weight", "linear", "linear_noalloc", "linear_grouped", "pack", "pack_nibbles", "quantize", "quantize_pack", "concat_n", "split_n", "packed_sizes", "workspace_bytes", "get_crossover",
           "set_crossover", "segments", "Q4Error", "library_path"]


def library_path() -> str:
    return _lib.LIB_PATH


@dataclass
class Q4Weight:
    """A packed N x K weight: ``codes`` uint8 [q4_packed_code_bytes],
    ``scales`` float16 [q4_packed_scale_bytes / 2], both on one GPU."""
    codes: torch.Tensor
    scales: torch.Tensor
    N: int
    K: int

    @property
    def device(self) -> torch.device:
        return self.codes.device


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
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must be %d-D, got shape %s" % (name, ndim, tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def packed_sizes(N: int, K: int):
    """(packed code bytes, packed scale bytes) of an N x K matrix."""
    lib = _lib.load()
    cb, sb = int(lib.q4_packed_code_bytes(N, K)), int(lib.q4_packed_scale_bytes(N, K))
    if cb == 0:
        raise ValueError("bad shape N=%d K=%d (K must be a positive multiple of 32)" % (N, K))
    return cb, sb


def pack(codes: torch.Tensor, scales: torch.Tensor) -> Q4Weight:
    """codes uint8 [N, K] (low 4 bits used), scales float16 [N, K/32] -> Q4Weight."""
    lib = _lib.load()
    _need(codes, "codes", (torch.uint8,), 2)
    dev = codes.device
    _need(scales, "scales", (torch.float16,), 2, dev)
    N, K = codes.shape
    if tuple(scales.shape) != (N, K // 32):
        raise ValueError("scales must be [%d, %d]" % (N, K // 32))
    cb, sb = packed_sizes(N, K)
    wq = torch.empty(cb, dtype=torch.uint8, device=dev)
    ws = torch.empty(sb // 2, dtype=torch.float16, device=dev)
    with torch.cuda.device(dev):
        st = lib.q4_pack(codes.data_ptr(), scales.data_ptr(), wq.data_ptr(), ws.data_ptr(), N, K, _stream(dev))
    _lib.check(st, "q4_pack")
    return Q4Weight(wq, ws, N, K)


def pack_nibbles(rows: torch.Tensor, scales: torch.Tensor) -> Q4Weight:
    """Nibble rows uint8 [N, K/2] (byte j: k = 2j low nibble, 2j + 1 high),
    scales float16 [N, K/32] -> Q4Weight (q4_pack_nibbles)."""
    lib = _lib.load()
    _need(rows, "rows", (torch.uint8,), 2)
    dev = rows.device
    _need(scales, "scales", (torch.float16,), 2, dev)
    N, K = rows.shape[0], rows.shape[1] * 2
    if tuple(scales.shape) != (N, K // 32):
        raise ValueError("scales must be [%d, %d]" % (N, K // 32))
    cb, sb = packed_sizes(N, K)
    wq = torch.empty(cb, dtype=torch.uint8, device=dev)
    ws = torch.empty(sb // 2, dtype=torch.float16, device=dev)
    with torch.cuda.device(dev):
        st = lib.q4_pack_nibbles(rows.data_ptr(), scales.data_ptr(), wq.data_ptr(), ws.data_ptr(), N, K,
                                 _stream(dev))
    _lib.check(st, "q4_pack_nibbles")
    return Q4Weight(wq, ws, N, K)


def quantize(w: torch.Tensor):
    """Dense weights [N, K] (float32, bfloat16 or float16, on a GPU) ->
    canonical (codes uint8 [N, K], scales float16 [N, K/32]) for ``pack``.
    Per block of 32 weights of a row: d = absmax / 7 rounded once to fp16,
    code = clamp(round_half_even(w / d), -8, 7) + 8 (include/q4.h)."""
    lib = _lib.load()
    _need(w, "w", (torch.float32, torch.bfloat16, torch.float16), 2)
    N, K = w.shape
    kind = {torch.float32: _lib.Q4_F32, torch.bfloat16: _lib.Q4_BF16, torch.float16: _lib.Q4_F16}[w.dtype]
    codes = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    scales = torch.empty((N, max(K // 32, 0)), dtype=torch.float16, device=w.device)
    with torch.cuda.device(w.device):
        st = lib.q4_quantize(w.data_ptr(), kind, codes.data_ptr(), scales.data_ptr(), N, K, _stream(w.device))
    _lib.check(st, "q4_quantize")
    return codes, scales


def quantize_pack(w: torch.Tensor) -> Q4Weight:
    """quantize() then pack(): dense weights [N, K] -> Q4Weight."""
    return pack(*quantize(w))


def workspace_bytes(M: int, N: int, K: int, kernel: str = "auto") -> int:
    return int(_lib.load().q4_workspace_bytes(M, N, K, KERNELS[kernel]))


def linear(x: torch.Tensor, w: Q4Weight, out: torch.Tensor | None = None, kernel: str = "auto",
           workspace: torch.Tensor | bool | None = True) -> torch.Tensor:
    """y = x . dequant(w)^T on the current stream of x's device.

    kernel: "auto" (crossover rule), "gemv" or "gemm" (forced).  The result
    bits do not depend on this choice.
    workspace: True (default) allocates the workspace the matrix-matrix
    kernel can use; False/None runs without one; a uint8 tensor is used as
    given.
    """
    lib = _lib.load()
    _need(x, "x", (torch.bfloat16, torch.float16), 2)
    dev = x.device
    if not isinstance(w, Q4Weight):
        raise TypeError("w must be a Q4Weight (see pack)")
    _need(w.codes, "w.codes", (torch.uint8,), 1, dev)
    _need(w.scales, "w.scales", (torch.float16,), 1, dev)
    M, K = x.shape
    N = w.N
    if K != w.K:
        raise ValueError("x has K=%d, weight has K=%d" % (K, w.K))
    cb, sb = packed_sizes(N, K)
    if w.codes.numel() != cb or w.scales.numel() * 2 != sb:
        raise ValueError("packed weight sizes do not match N=%d K=%d" % (N, K))
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
        st = lib.q4_linear_ex(x.data_ptr(), dtype, w.codes.data_ptr(), w.scales.data_ptr(), out.data_ptr(),
                              M, N, K, KERNELS[kernel], ws_ptr, ws_len, _stream(dev))
    _lib.check(st, "q4_linear_ex")
    return out


def linear_noalloc(x: torch.Tensor, w: Q4Weight, out: torch.Tensor, kernel: str = "auto") -> torch.Tensor:
    """q4_linear_noalloc: like ``linear`` with the library's fixed scratch
    buffer as the workspace, so the call allocates nothing (``out`` must be
    given).  Calls that overlap in time on one GPU share that buffer and
    race."""
    lib = _lib.load()
    _need(x, "x", (torch.bfloat16, torch.float16), 2)
    dev = x.device
    if not isinstance(w, Q4Weight):
        raise TypeError("w must be a Q4Weight (see pack)")
    _need(w.codes, "w.codes", (torch.uint8,), 1, dev)
    _need(w.scales, "w.scales", (torch.float16,), 1, dev)
    M, K = x.shape
    if K != w.K:
        raise ValueError("x has K=%d, weight has K=%d" % (K, w.K))
    _need(out, "out", (torch.float32,), 2, dev)
    if tuple(out.shape) != (M, w.N):
        raise ValueError("out must be [%d, %d]" % (M, w.N))
    if kernel not in KERNELS:
        raise ValueError("kernel must be one of %s" % sorted(KERNELS))
    dtype = _lib.Q4_BF16 if x.dtype == torch.bfloat16 else _lib.Q4_F16
    with torch.cuda.device(dev):
        st = lib.q4_linear_noalloc(x.data_ptr(), dtype, w.codes.data_ptr(), w.scales.data_ptr(), out.data_ptr(),
                                   M, w.N, K, KERNELS[kernel], _stream(dev))
    _lib.check(st, "q4_linear_noalloc")
    return out


def linear_grouped(x: torch.Tensor, weights, outs=None, workspace: torch.Tensor | bool | None = True) -> list:
    """q4_linear_grouped: y_i = x . dequant(w_i)^T for 1..8 weights sharing
    x's K, in one launch of the matrix-vector kernel where the crossover rule
    picks it (else one call per weight, with ``workspace`` as in ``linear``:
    True allocates the largest one the calls can use).  Returns the outputs
    (allocated unless ``outs`` is given)."""
    lib = _lib.load()
    _need(x, "x", (torch.bfloat16, torch.float16), 2)
    dev = x.device
    weights = list(weights)
    if not 1 <= len(weights) <= _lib.GROUP_MAX:
        raise ValueError("linear_grouped takes 1..%d weights" % _lib.GROUP_MAX)
    M, K = x.shape
    if outs is None:
        outs = [torch.empty((M, w.N), dtype=torch.float32, device=dev) for w in weights]
    outs = list(outs)
    if len(outs) != len(weights):
        raise ValueError("one output per weight")
    items = (_lib.GroupItem * len(weights))()
    for i, (w, y) in enumerate(zip(weights, outs)):
        if not isinstance(w, Q4Weight):
            raise TypeError("weights must be Q4Weight objects")
        if w.K != K:
            raise ValueError("weight %d has K=%d, x has K=%d" % (i, w.K, K))
        _need(w.codes, "w.codes", (torch.uint8,), 1, dev)
        _need(w.scales, "w.scales", (torch.float16,), 1, dev)
        cb, sb = packed_sizes(w.N, K)
        if w.codes.numel() != cb or w.scales.numel() * 2 != sb:
            raise ValueError("packed weight %d sizes do not match N=%d K=%d" % (i, w.N, K))
        _need(y, "out", (torch.float32,), 2, dev)
        if tuple(y.shape) != (M, w.N):
            raise ValueError("out %d must be [%d, %d]" % (i, M, w.N))
        items[i] = _lib.GroupItem(w.codes.data_ptr(), w.scales.data_ptr(), y.data_ptr(), w.N)
    ws_ptr, ws_len = None, 0
    if isinstance(workspace, torch.Tensor):
        _need(workspace, "workspace", (torch.uint8,), 1, dev)
        ws_ptr, ws_len = workspace.data_ptr(), workspace.numel()
    elif workspace:
        need = max(lib.q4_workspace_bytes(M, w.N, K, _lib.Q4_AUTO) for w in weights)
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)
            ws_ptr, ws_len = ws.data_ptr(), need
    dtype = _lib.Q4_BF16 if x.dtype == torch.bfloat16 else _lib.Q4_F16
    with torch.cuda.device(dev):
        st = lib.q4_linear_grouped(x.data_ptr(), dtype, items, len(weights), M, K, ws_ptr, ws_len, _stream(dev))
    _lib.check(st, "q4_linear_grouped")
    return outs


def get_crossover() -> int:
    return int(_lib.load().q4_get_crossover())


def set_crossover(T: int) -> None:
    _lib.check(_lib.load().q4_set_crossover(int(T)), "q4_set_crossover")


def segments(K: int) -> int:
    return int(_lib.load().q4_segments(int(K)))


def concat_n(weights) -> Q4Weight:
    """Packed weights of one K stacked along N, for fused launches (q|k|v,
    gate|up): one call then computes all of them.  The packed form is
    tile-major along N, so concatenating the packed buffers packs the
    concatenated rows; every part but the last must have N a multiple of
    16 (no padding rows inside).  Each output column keeps its bits: the
    reduction order depends on K only."""
    weights = list(weights)
    if not weights:
        raise ValueError("concat_n needs at least one weight")
    K = weights[0].K
    for i, w in enumerate(weights):
        if not isinstance(w, Q4Weight):
            raise TypeError("concat_n takes Q4Weight objects")
        if w.K != K:
            raise ValueError("all weights must share K (%d != %d)" % (w.K, K))
        if i + 1 < len(weights) and w.N % 16:
            raise ValueError("every part but the last needs N % 16 == 0 (part %d has N=%d)" % (i, w.N))
    codes = torch.cat([w.codes for w in weights])
    scales = torch.cat([w.scales for w in weights])
    return Q4Weight(codes, scales, sum(w.N for w in weights), K)


def split_n(w: Q4Weight, Ns) -> list:
    """Views of a packed weight as consecutive row blocks of Ns[i] rows
    (all but the last a multiple of 16; sum(Ns) == w.N): the inverse of
    concat_n, sharing w's memory."""
    Ns = [int(n) for n in Ns]
    if sum(Ns) != w.N or any(n < 1 for n in Ns) or any(n % 16 for n in Ns[:-1]):
        raise ValueError("row blocks %s do not split N=%d on 16-row tiles" % (Ns, w.N))
    out, c0, s0 = [], 0, 0
    for n in Ns:
        cb, sb = packed_sizes(n, w.K)
        out.append(Q4Weight(w.codes[c0:c0 + cb], w.scales[s0:s0 + sb // 2], n, w.K))
        c0 += cb
        s0 += sb // 2
    return out
