"""CPU fp64 oracle for the Q4 linear layer -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library in
``bit_quantized_matmul_q4_amd``) shares no code with it and never calls it.

The arithmetic lives in ``q4_oracle.c`` (plain C, fp64, ascending-k sums);
this module only builds and loads that library and moves numpy arrays in and
out.  What it computes, per "Why Continuous Batching Slowed Down My LLM
Inference Engine: A Metal Kernel Investigation", section "Two Rows of Input,
Two Different Kernels" (each weight row is dot-producted with each input row):

    y[m][n] = sum_k x[m][k] * (q[n][k] - 8) * d[n][k // 32]
    A[m][n] = sum_k |x[m][k] * (q[n][k] - 8) * d[n][k // 32]|

with the block format stated in ``q4_oracle.c``.  Inputs are raw bit
patterns: x as uint16 (fp16 or bf16 bits), scales as uint16 (fp16 bits),
packed codes as uint8.  Weights come in the canonical row-major layout
(``linear``) or in the library's tiled layout (``linear_tiled``); both are
defined in ``q4_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "q4_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lock = threading.Lock()
_lib = None


def compile_library(src: str = _SRC, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the C oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", *extra_flags, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _declare(lib):
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.q4o_abi_version.restype = ctypes.c_int
    lib.q4o_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.q4o_f16_to_f64.restype = ctypes.c_double
    lib.q4o_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.q4o_bf16_to_f64.restype = ctypes.c_double
    lib.q4o_pack.argtypes = [u8p, u8p, i64, i64]
    lib.q4o_pack.restype = None
    lib.q4o_unpack.argtypes = [u8p, u8p, i64, i64]
    lib.q4o_unpack.restype = None
    lib.q4o_linear.argtypes = [u16p, ctypes.c_int, u8p, u16p, i64, i64, i64, f64p, f64p]
    lib.q4o_linear.restype = ctypes.c_int
    lib.q4o_linear_fmt.argtypes = [u16p, ctypes.c_int, u8p, u16p, i64, i64, i64, ctypes.c_int,
                                   f64p, f64p]
    lib.q4o_linear_fmt.restype = ctypes.c_int
    lib.q4o_linear_sampled.argtypes = [u16p, ctypes.c_int, u8p, u16p, i64, i64, i64, ctypes.c_int,
                                       i64p, i64p, i64, f64p, f64p]
    lib.q4o_linear_sampled.restype = ctypes.c_int
    lib.q4o_tiled_code_bytes.argtypes = [i64, i64]
    lib.q4o_tiled_code_bytes.restype = i64
    lib.q4o_tiled_scale_count.argtypes = [i64, i64]
    lib.q4o_tiled_scale_count.restype = i64
    lib.q4o_pack_tiled.argtypes = [u8p, u16p, u8p, u16p, i64, i64]
    lib.q4o_pack_tiled.restype = None
    lib.q4o_unpack_tiled.argtypes = [u8p, u16p, u8p, u16p, i64, i64]
    lib.q4o_unpack_tiled.restype = None
    lib.q4o_f64_to_f16.argtypes = [ctypes.c_double]
    lib.q4o_f64_to_f16.restype = ctypes.c_uint16
    lib.q4o_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int, u8p, u16p, i64, i64]
    lib.q4o_quantize.restype = ctypes.c_int
    return lib


def load_library(path: str | None = None):
    """Load (building first if absent) the oracle library.  A path loads a
    separately compiled copy, e.g. one a test built from altered source."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH) or (
                    os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC)):
                compile_library()
            _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def f16_to_f64(bits: int, lib=None) -> float:
    return (lib or load_library()).q4o_f16_to_f64(int(bits))


def bf16_to_f64(bits: int, lib=None) -> float:
    return (lib or load_library()).q4o_bf16_to_f64(int(bits))


def pack(codes: np.ndarray, lib=None) -> np.ndarray:
    """codes uint8 [N, K] -> packed uint8 [N, K/2] (low nibble = even k)."""
    codes = _c(codes, np.uint8)
    n, k = codes.shape
    if k % 2:
        raise ValueError("K must be even")
    out = np.empty((n, k // 2), np.uint8)
    (lib or load_library()).q4o_pack(_ptr(codes, ctypes.c_uint8), _ptr(out, ctypes.c_uint8), n, k)
    return out


def unpack(wq: np.ndarray, K: int, lib=None) -> np.ndarray:
    """packed uint8 [N, K/2] -> codes uint8 [N, K]."""
    wq = _c(wq, np.uint8)
    n = wq.shape[0]
    if wq.shape[1] * 2 != K:
        raise ValueError("packed row length must be K/2")
    out = np.empty((n, K), np.uint8)
    (lib or load_library()).q4o_unpack(_ptr(wq, ctypes.c_uint8), _ptr(out, ctypes.c_uint8), n, K)
    return out


def tiled_sizes(N: int, K: int, lib=None):
    """(code bytes, scale entries) of the tiled layout for an N x K matrix."""
    lib = lib or load_library()
    return int(lib.q4o_tiled_code_bytes(N, K)), int(lib.q4o_tiled_scale_count(N, K))


def pack_tiled(codes: np.ndarray, scales: np.ndarray, lib=None):
    """codes uint8 [N, K] (low 4 bits used), scales fp16 bits [N, K/32] ->
    (tiled codes uint8 [bytes], tiled scales uint16 [entries])."""
    lib = lib or load_library()
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    N, K = codes.shape
    if K % 32 or scales.shape != (N, K // 32):
        raise ValueError("need K % 32 == 0 and scales [N, K/32]")
    nb, ns = tiled_sizes(N, K, lib)
    wq = np.empty(nb, np.uint8)
    sc = np.empty(ns, np.uint16)
    lib.q4o_pack_tiled(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint16),
                       _ptr(wq, ctypes.c_uint8), _ptr(sc, ctypes.c_uint16), N, K)
    return wq, sc


def unpack_tiled(wq_t: np.ndarray, sc_t: np.ndarray, N: int, K: int, lib=None):
    """Inverse of pack_tiled -> (codes uint8 [N, K], scales uint16 [N, K/32])."""
    lib = lib or load_library()
    nb, ns = tiled_sizes(N, K, lib)
    wq_t = _c(wq_t, np.uint8).reshape(-1)
    sc_t = _c(sc_t, np.uint16).reshape(-1)
    if wq_t.size != nb or sc_t.size != ns:
        raise ValueError("tiled sizes for (%d, %d) are %d code bytes and %d scales" % (N, K, nb, ns))
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, K // 32), np.uint16)
    lib.q4o_unpack_tiled(_ptr(wq_t, ctypes.c_uint8), _ptr(sc_t, ctypes.c_uint16),
                         _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint16), N, K)
    return codes, scales


def _check(x_bits, wq, scales):
    x_bits = _c(x_bits, np.uint16)
    wq = _c(wq, np.uint8)
    scales = _c(scales, np.uint16)
    M, K = x_bits.shape
    N = wq.shape[0]
    if K % 32 or K <= 0:
        raise ValueError("K must be a positive multiple of 32")
    if wq.shape != (N, K // 2) or scales.shape != (N, K // 32):
        raise ValueError("shape mismatch: x %s, wq %s, scales %s" % (x_bits.shape, wq.shape, scales.shape))
    return x_bits, wq, scales, M, N, K


def linear(x_bits: np.ndarray, x_is_bf16: bool, wq: np.ndarray, scales: np.ndarray, lib=None):
    """Full fp64 product, canonical layout.  Returns (y, A), both float64 [M, N]."""
    x_bits, wq, scales, M, N, K = _check(x_bits, wq, scales)
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    rc = (lib or load_library()).q4o_linear(
        _ptr(x_bits, ctypes.c_uint16), int(bool(x_is_bf16)), _ptr(wq, ctypes.c_uint8),
        _ptr(scales, ctypes.c_uint16), M, N, K, _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("oracle q4o_linear failed (%d)" % rc)
    return y, a


def _check_tiled(x_bits, wq_t, sc_t, N, K, lib):
    x_bits = _c(x_bits, np.uint16)
    M = x_bits.shape[0]
    if x_bits.shape[1] != K or K % 32 or K <= 0:
        raise ValueError("x must be [M, K] with K a positive multiple of 32")
    nb, ns = tiled_sizes(N, K, lib)
    wq_t = _c(wq_t, np.uint8).reshape(-1)
    sc_t = _c(sc_t, np.uint16).reshape(-1)
    if wq_t.size != nb or sc_t.size != ns:
        raise ValueError("tiled sizes for (%d, %d) are %d code bytes and %d scales" % (N, K, nb, ns))
    return x_bits, wq_t, sc_t, M


def linear_tiled(x_bits, x_is_bf16, wq_t, sc_t, N: int, K: int, lib=None):
    """Full fp64 product from the tiled layout.  Returns (y, A) [M, N]."""
    lib = lib or load_library()
    x_bits, wq_t, sc_t, M = _check_tiled(x_bits, wq_t, sc_t, N, K, lib)
    y = np.empty((M, N), np.float64)
    a = np.empty((M, N), np.float64)
    rc = lib.q4o_linear_fmt(_ptr(x_bits, ctypes.c_uint16), int(bool(x_is_bf16)), _ptr(wq_t, ctypes.c_uint8),
                            _ptr(sc_t, ctypes.c_uint16), M, N, K, 1, _ptr(y, ctypes.c_double),
                            _ptr(a, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("oracle q4o_linear_fmt failed (%d)" % rc)
    return y, a


def linear_sampled(x_bits, x_is_bf16, wq, scales, ms, ns, lib=None, tiled_nk=None):
    """Outputs (ms[i], ns[i]) only.  Returns (y, A), float64 [count].
    tiled_nk=(N, K) reads wq/scales in the tiled layout."""
    lib = lib or load_library()
    if tiled_nk is not None:
        N, K = tiled_nk
        x_bits, wq, scales, M = _check_tiled(x_bits, wq, scales, N, K, lib)
    else:
        x_bits, wq, scales, M, N, K = _check(x_bits, wq, scales)
    ms = _c(ms, np.int64)
    ns = _c(ns, np.int64)
    if ms.shape != ns.shape or ms.ndim != 1:
        raise ValueError("ms and ns must be 1-D of equal length")
    y = np.empty(ms.shape[0], np.float64)
    a = np.empty(ms.shape[0], np.float64)
    rc = lib.q4o_linear_sampled(
        _ptr(x_bits, ctypes.c_uint16), int(bool(x_is_bf16)), _ptr(wq, ctypes.c_uint8),
        _ptr(scales, ctypes.c_uint16), M, N, K, int(tiled_nk is not None),
        _ptr(ms, ctypes.c_int64), _ptr(ns, ctypes.c_int64),
        ms.shape[0], _ptr(y, ctypes.c_double), _ptr(a, ctypes.c_double))
    if rc != 0:
        raise RuntimeError("oracle q4o_linear_sampled failed (%d)" % rc)
    return y, a


def max_normalised_error(y_test: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray) -> float:
    """max over outputs of |y_test - y_ref| / A, with A = 0 requiring y_test = 0
    (reported as inf otherwise)."""
    y_test = np.asarray(y_test, np.float64)
    diff = np.abs(y_test - y_ref)
    zero = a_ref == 0
    if np.any(zero & (y_test != 0)):
        return float("inf")
    rel = np.where(zero, 0.0, diff / np.where(zero, 1.0, a_ref))
    return float(rel.max()) if rel.size else 0.0


def f64_to_f16(v: float, lib=None) -> int:
    """binary16 bits of v, nearest, ties to even."""
    return int((lib or load_library()).q4o_f64_to_f16(float(v)))


QUANT_KINDS = {"f16": 0, "bf16": 1, "f32": 2}


def quantize(w, kind: str, lib=None):
    """Dense weights [N, K] -> (codes uint8 [N, K], scales fp16 bits uint16
    [N, K/32]) by the block rule stated in q4_oracle.c.  w: uint16 bit
    patterns for kind "f16" / "bf16", float32 values for "f32"."""
    k = QUANT_KINDS[kind]
    w = _c(w, np.float32 if k == 2 else np.uint16)
    N, K = w.shape
    if K % 32 or K <= 0:
        raise ValueError("K must be a positive multiple of 32")
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, K // 32), np.uint16)
    rc = (lib or load_library()).q4o_quantize(w.ctypes.data_as(ctypes.c_void_p), k, _ptr(codes, ctypes.c_uint8),
                                              _ptr(scales, ctypes.c_uint16), N, K)
    if rc != 0:
        raise RuntimeError("oracle q4o_quantize failed (%d)" % rc)
    return codes, scales
