"""Seeded synthetic inputs for the Q4 linear layer.

This module is shared by the tests, the benchmark and the smoke check, and
serves both the HIP path and the CPU oracle.  It holds none of the method's
arithmetic: it only draws random numbers and rounds them to the storage
types (fp16 via numpy's round-to-nearest-even cast; bf16 by rounding the
fp32 value to nearest-even on its top 16 bits).  Inputs are handed around as
raw bit patterns (uint16 for fp16/bf16, uint8 for codes and packed codes),
so the stored bits define each input.

Workload shapes stand in for the trained models named on the pages
("Why Continuous Batching Slowed Down My LLM Inference Engine", intro: a
4-bit Qwen2.5-7B and a Qwen2.5-0.5B draft model).  No weights, prompts or
datasets are used: codes are i.i.d. uniform on 0..15, block scales are
|N(0, 0.02)| rounded to fp16 (subnormal results are kept), and activations
are N(0, 1) rounded to the activation type.  Streams are numpy PCG64 seeded
from SeedSequence([0, workload, matrix, tensor]) so that every (workload,
matrix, tensor) triple is reproducible and independent.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# tensor ids inside a seed
T_CODES, T_SCALES, T_X = 0, 1, 2


@dataclass(frozen=True)
class Matrix:
    name: str
    N: int  # output features (rows of W)
    K: int  # input features


# Qwen2.5-0.5B-shaped projections (hidden 896, MLP 4864, 2 KV heads x 64).
SET_05B = (
    Matrix("q_proj", 896, 896),
    Matrix("k_proj", 128, 896),
    Matrix("v_proj", 128, 896),
    Matrix("gate_proj", 4864, 896),
    Matrix("up_proj", 4864, 896),
    Matrix("down_proj", 896, 4864),
)

# Qwen2.5-7B-shaped projections (hidden 3584, MLP 18944, 4 KV heads x 128).
SET_7B = (
    Matrix("q_proj", 3584, 3584),
    Matrix("k_proj", 512, 3584),
    Matrix("v_proj", 512, 3584),
    Matrix("gate_proj", 18944, 3584),
    Matrix("up_proj", 18944, 3584),
    Matrix("down_proj", 3584, 18944),
)

LM_HEAD_7B = Matrix("lm_head", 152064, 3584)
N_LAYERS_7B = 28

# GPT-2-small-shaped attention projections ("Why LLM Decoding Is Slow, and
# Why Batching Is (Almost) Free", section "The Catch: Every User Brings Their
# Own Cache": 12 heads of 64, d_model 768).  The MLP and vocabulary widths
# are not on the pages, so only the 768-wide projections are built.
SET_GPT2 = (
    Matrix("q_proj", 768, 768),
    Matrix("k_proj", 768, 768),
    Matrix("v_proj", 768, 768),
    Matrix("o_proj", 768, 768),
)

# The workloads.  x dtype: "f16" or "bf16".
WORKLOADS = {
    1: dict(name="q4_matvec_896", matrices=(Matrix("w", 896, 896),), Ms=(1,), x="f16"),
    2: dict(name="qwen2.5-0.5b_layer_set", matrices=SET_05B, Ms=(1, 2, 4), x="f16"),
    3: dict(name="qwen2.5-7b_layer_set", matrices=SET_7B, Ms=tuple(range(1, 9)), x="bf16"),
    4: dict(name="qwen2.5-7b_layer_set_mixed_124", matrices=SET_7B, Ms=(124,), x="bf16"),
    5: dict(name="qwen2.5-7b_decode_weight_stream", matrices=SET_7B + (LM_HEAD_7B,),
            Ms=(1, 4, 16, 64), x="bf16"),
    6: dict(name="gpt2-small_attention_set", matrices=SET_GPT2, Ms=tuple(range(1, 17)), x="bf16"),
}


def generator(workload: int, matrix: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, workload, matrix, tensor])))


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16, nearest-even; returns uint16 bits.
    (Finite inputs only: the generators never produce inf or nan.)"""
    u = np.ascontiguousarray(v, np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(v, np.float64).astype(np.float16).view(np.uint16)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(np.asarray(v, np.float64).astype(np.float32))


def codes(N: int, K: int, workload: int = 0, matrix: int = 0) -> np.ndarray:
    """uint8 [N, K], i.i.d. uniform on 0..15."""
    return generator(workload, matrix, T_CODES).integers(0, 16, size=(N, K), dtype=np.uint8)


def packed_weight(N: int, K: int, workload: int = 0, matrix: int = 0, sigma: float = 0.02):
    """A weight already in the library's packed (tiled) form, drawn directly:
    code bytes are i.i.d. uniform (two independent uniform nibbles per byte,
    the packed form of i.i.d. uniform codes) and scales |N(0, sigma)| in
    fp16, over the whole tiled extent (16-row by 4-block tiles).  Padding
    positions, if the shape has any, hold random values too: the kernels never
    use them.  For benchmark pools and very large matrices, where the
    canonical codes are never needed."""
    tiles = -(-N // 16) * -(-(K // 32) // 4)
    g = generator(workload, matrix, T_CODES)
    wq = g.integers(0, 256, size=tiles * 1024, dtype=np.uint8)
    gs = generator(workload, matrix, T_SCALES)
    sc = f64_to_f16_bits(np.abs(gs.normal(0.0, sigma, size=tiles * 64)))
    return wq, sc


def scales(N: int, K: int, workload: int = 0, matrix: int = 0, sigma: float = 0.02) -> np.ndarray:
    """fp16 bits [N, K/32] of |N(0, sigma)|."""
    g = generator(workload, matrix, T_SCALES)
    return f64_to_f16_bits(np.abs(g.normal(0.0, sigma, size=(N, K // 32))))


def activations(M: int, K: int, dtype: str, workload: int = 0, matrix: int = 0) -> np.ndarray:
    """uint16 bits [M, K] of N(0, 1) rounded to fp16 or bf16.  Row m does not
    depend on M, so smaller batches are prefixes of larger ones."""
    g = generator(workload, matrix, T_X)
    rows = []
    # draw row by row so that row m is the same for every M
    for _ in range(M):
        rows.append(g.normal(0.0, 1.0, size=K))
    v = np.stack(rows) if rows else np.zeros((0, K))
    if dtype == "f16":
        return f64_to_f16_bits(v)
    if dtype == "bf16":
        return f64_to_bf16_bits(v)
    raise ValueError("dtype must be 'f16' or 'bf16'")


def problem(N: int, K: int, M: int, dtype: str, workload: int = 0, matrix: int = 0):
    """(x_bits [M,K], codes [N,K], scales_bits [N,K/32]) for one matrix."""
    return (activations(M, K, dtype, workload, matrix), codes(N, K, workload, matrix),
            scales(N, K, workload, matrix))


def algorithmic_bytes(M: int, N: int, K: int) -> int:
    """Bytes one call must move at least: packed codes, fp16 scales,
    16-bit activations and fp32 outputs."""
    return N * K // 2 + N * K // 16 + 2 * M * K + 4 * M * N
