"""ctypes loader for libq4.so (the C ABI in include/q4.h).

The library must have been built in-tree (``python -m
bit_quantized_matmul_q4_amd.build``); there is no fallback: if it is
missing or does not load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libq4.so")

Q4_OK = 0
Q4_ERR_NULL = -1
Q4_ERR_SHAPE = -2
Q4_ERR_ALIGN = -3
Q4_ERR_ENUM = -4
Q4_ERR_HIP = -5
Q4_ERR_WORKSPACE = -6
Q4_ERR_SCRATCH = -7

Q4_F16 = 0
Q4_BF16 = 1
Q4_F32 = 2

Q4_AUTO = 0
Q4_GEMV = 1
Q4_GEMM = 2

KERNELS = {"auto": Q4_AUTO, "gemv": Q4_GEMV, "gemm": Q4_GEMM}

EXPORTS = (
    "q4_linear", "q4_linear_f16", "q4_linear_ex", "q4_linear_noalloc", "q4_linear_grouped", "q4_workspace_bytes",
    "q4_pack", "q4_pack_nibbles", "q4_quantize",
    "q4_packed_code_bytes", "q4_packed_scale_bytes",
    "q4_get_crossover", "q4_set_crossover", "q4_segments", "q4_strerror",
    "q4_last_hip_error", "q4_abi_version",
)

ABI_VERSION = 6
GROUP_MAX = 8


class GroupItem(ctypes.Structure):
    """q4_group_item (include/q4.h)."""
    _fields_ = [("Wq", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("y", ctypes.c_void_p), ("N", ctypes.c_int)]


class Q4Error(RuntimeError):
    def __init__(self, status: int, what: str, lib=None):
        text = lib.q4_strerror(status).decode() if lib is not None else str(status)
        extra = ""
        if lib is not None and status == Q4_ERR_HIP:
            extra = " (hip error %d)" % lib.q4_last_hip_error()
        super().__init__("%s: %s%s" % (what, text, extra))
        self.status = status


_lock = threading.Lock()
_lib = None


def _declare(lib):
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.q4_linear.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.q4_linear.restype = i
    lib.q4_linear_f16.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.q4_linear_f16.restype = i
    lib.q4_linear_ex.argtypes = [vp, i, vp, vp, vp, i, i, i, i, vp, sz, vp]
    lib.q4_linear_ex.restype = i
    lib.q4_linear_noalloc.argtypes = [vp, i, vp, vp, vp, i, i, i, i, vp]
    lib.q4_linear_noalloc.restype = i
    lib.q4_linear_grouped.argtypes = [vp, i, ctypes.POINTER(GroupItem), i, i, i, vp, sz, vp]
    lib.q4_linear_grouped.restype = i
    lib.q4_pack_nibbles.argtypes = [vp, vp, vp, vp, i, i, vp]
    lib.q4_pack_nibbles.restype = i
    lib.q4_workspace_bytes.argtypes = [i, i, i, i]
    lib.q4_workspace_bytes.restype = sz
    lib.q4_pack.argtypes = [vp, vp, vp, vp, i, i, vp]
    lib.q4_pack.restype = i
    lib.q4_quantize.argtypes = [vp, i, vp, vp, i, i, vp]
    lib.q4_quantize.restype = i
    lib.q4_packed_code_bytes.argtypes = [i, i]
    lib.q4_packed_code_bytes.restype = sz
    lib.q4_packed_scale_bytes.argtypes = [i, i]
    lib.q4_packed_scale_bytes.restype = sz
    lib.q4_get_crossover.argtypes = []
    lib.q4_get_crossover.restype = i
    lib.q4_set_crossover.argtypes = [i]
    lib.q4_set_crossover.restype = i
    lib.q4_segments.argtypes = [i]
    lib.q4_segments.restype = i
    lib.q4_strerror.argtypes = [i]
    lib.q4_strerror.restype = ctypes.c_char_p
    lib.q4_last_hip_error.argtypes = []
    lib.q4_last_hip_error.restype = i
    lib.q4_abi_version.argtypes = []
    lib.q4_abi_version.restype = i
    return lib


def load(path: str | None = None):
    """Load libq4.so (default: the in-tree build).  Raises if it is missing."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(
                    "libq4.so is not built (%s); run `python -m bit_quantized_matmul_q4_amd.build`"
                    % LIB_PATH)
            lib = _declare(ctypes.CDLL(LIB_PATH))
            if lib.q4_abi_version() != ABI_VERSION:
                raise ImportError("libq4.so ABI %d, binding expects %d"
                                  % (lib.q4_abi_version(), ABI_VERSION))
            _lib = lib
    return _lib


def check(status: int, what: str) -> None:
    if status != Q4_OK:
        raise Q4Error(status, what, load())
