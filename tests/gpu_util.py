"""Helpers shared by the GPU tests: build-if-missing, host<->device moves of
raw bit patterns, and the oracle comparison."""
from __future__ import annotations

import ctypes
import os
import sys

import numpy as np
import torch

import bit_quantized_matmul_q4_amd as q4
from bit_quantized_matmul_q4_amd import _lib, build

DEV = torch.device("cuda:0")

# max |y_gpu - y_ref| / sum|x w| allowed against the fp64 oracle
TOL = 2e-3


def ensure_built() -> None:
    """Tests call the in-tree build; they build only when nothing is built."""
    if not os.path.exists(build.LIB):
        build.build_library()
    if not os.path.exists(build.PROBE_LIB):
        build.build_probe()


def require_gpu() -> None:
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X (torch.cuda.is_available() is False)")
    ensure_built()
    _lib.load()


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    sys.stdout.write("[gpu] %s\n" % msg)
    sys.stdout.flush()


def x_to_dev(bits: np.ndarray, bf16: bool) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16 if bf16 else torch.float16)


def scales_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(DEV).view(torch.float16)


def u8_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def y_bits(y: torch.Tensor) -> np.ndarray:
    return y.detach().cpu().numpy().view(np.uint32)


def pack_dev(codes: np.ndarray, s_bits: np.ndarray) -> "q4.Q4Weight":
    """Canonical codes [N, K] and scale bits [N, K/32] -> packed on the GPU."""
    return q4.pack(u8_to_dev(codes), scales_to_dev(s_bits))


def weight_from_tiled(wq_t: np.ndarray, sc_t: np.ndarray, N: int, K: int) -> "q4.Q4Weight":
    """Packed (tiled) bytes built on the host -> a Q4Weight on the GPU."""
    return q4.Q4Weight(u8_to_dev(wq_t.reshape(-1)), scales_to_dev(sc_t.reshape(-1)), N, K)


def run_linear(x_bits, bf16, codes, s_bits, kernel="auto", workspace=True) -> torch.Tensor:
    """Canonical inputs -> GPU pack -> GPU linear (synchronized)."""
    out = q4.linear(x_to_dev(x_bits, bf16), pack_dev(codes, s_bits), kernel=kernel, workspace=workspace)
    torch.cuda.synchronize()
    return out


class Probe:
    """libq4probe.so: raw-lane probes of the library's device primitives."""

    def __init__(self):
        ensure_built()
        self.lib = ctypes.CDLL(build.PROBE_LIB)
        vp, i = ctypes.c_void_p, ctypes.c_int
        self.lib.q4probe_mfma.argtypes = [vp, vp, vp, i, i, vp]
        self.lib.q4probe_mfma_acc.argtypes = [vp, vp, vp, vp, i, i, vp]
        self.lib.q4probe_dequant.argtypes = [vp, vp, i, i, vp]
        self.lib.q4probe_fma0.argtypes = [vp, vp, vp, i, vp]
        self.lib.q4probe_q4dot.argtypes = [vp, vp, vp, vp, i, i, vp]

    def mfma(self, a_lanes: np.ndarray, b_lanes: np.ndarray, bf16: bool) -> np.ndarray:
        """a_lanes, b_lanes: uint16 [waves, 64, 8] -> float32 [waves, 64, 4]."""
        waves = a_lanes.shape[0]
        a = torch.from_numpy(np.ascontiguousarray(a_lanes, np.uint16).view(np.int16)).to(DEV)
        b = torch.from_numpy(np.ascontiguousarray(b_lanes, np.uint16).view(np.int16)).to(DEV)
        d = torch.empty((waves, 64, 4), dtype=torch.float32, device=DEV)
        rc = self.lib.q4probe_mfma(a.data_ptr(), b.data_ptr(), d.data_ptr(), waves, int(bf16),
                                   torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        return d.cpu().numpy()

    def mfma_acc(self, a_lanes: np.ndarray, b_lanes: np.ndarray, c_lanes: np.ndarray, bf16: bool) -> np.ndarray:
        """The same with the accumulator input c_lanes (float32 [waves, 64, 4])."""
        waves = a_lanes.shape[0]
        a = torch.from_numpy(np.ascontiguousarray(a_lanes, np.uint16).view(np.int16)).to(DEV)
        b = torch.from_numpy(np.ascontiguousarray(b_lanes, np.uint16).view(np.int16)).to(DEV)
        c = torch.from_numpy(np.ascontiguousarray(c_lanes, np.float32)).to(DEV)
        d = torch.empty((waves, 64, 4), dtype=torch.float32, device=DEV)
        rc = self.lib.q4probe_mfma_acc(a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(), waves, int(bf16),
                                       torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        return d.cpu().numpy()

    def dequant(self, words: np.ndarray, bf16: bool) -> np.ndarray:
        """uint32 [n] -> uint16 [n, 8] operand values."""
        n = words.shape[0]
        w = torch.from_numpy(np.ascontiguousarray(words, np.uint32).view(np.int32)).to(DEV)
        out = torch.empty((n, 4), dtype=torch.int32, device=DEV)
        rc = self.lib.q4probe_dequant(w.data_ptr(), out.data_ptr(), n, int(bf16),
                                      torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        return out.cpu().numpy().view(np.uint16).reshape(n, 8)

    def q4dot(self, a_lanes: np.ndarray, words: np.ndarray, bf16: bool):
        """a_lanes uint16 [waves, 64, 8], words uint32 [waves, 64] -> (D, C)
        float32 [waves, 64, 4] each: the block dot and its correction input."""
        waves = a_lanes.shape[0]
        a = torch.from_numpy(np.ascontiguousarray(a_lanes, np.uint16).view(np.int16)).to(DEV)
        w = torch.from_numpy(np.ascontiguousarray(words, np.uint32).view(np.int32)).to(DEV)
        d = torch.empty((waves, 64, 4), dtype=torch.float32, device=DEV)
        e = torch.empty((waves, 64, 4), dtype=torch.float32, device=DEV)
        rc = self.lib.q4probe_q4dot(a.data_ptr(), w.data_ptr(), d.data_ptr(), e.data_ptr(), waves, int(bf16),
                                    torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        return d.cpu().numpy(), e.cpu().numpy()

    def fma0(self, d: np.ndarray, s: np.ndarray) -> np.ndarray:
        n = d.shape[0]
        dt = torch.from_numpy(np.ascontiguousarray(d, np.float32)).to(DEV)
        st = torch.from_numpy(np.ascontiguousarray(s, np.float32)).to(DEV)
        out = torch.empty(n, dtype=torch.float32, device=DEV)
        rc = self.lib.q4probe_fma0(dt.data_ptr(), st.data_ptr(), out.data_ptr(), n,
                                   torch.cuda.current_stream().cuda_stream)
        assert rc == 0
        torch.cuda.synchronize()
        return out.cpu().numpy()


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)
