"""Batch-composition invariance where it matters downstream: near-tied
greedy choices and persistent cache writes.

"Why Continuous Batching Slowed Down My LLM Inference Engine: A Metal Kernel
Investigation" (sections "Same Prompt, Different Story" and "The Other
Request Already Finished") traces diverging output to two kernels that sum
in different orders: the same row computed alone (matrix-vector) or inside
a 124-row batch (matrix-matrix) gets slightly different values, a near-tied
greedy choice flips, and values written to the KV cache keep the
difference.  No trained weights are needed to show the mechanism: candidate
pairs are built whose two logits are exactly equal in real arithmetic (the
second row swaps codes between positions where x holds equal values), so
which one wins is decided by rounding order alone.

The library computes the row alone (matrix-vector kernel) and inside a
124-row batch (matrix-matrix kernel) with identical bits, so no pair flips
and every cached value is the same.  Two plain PyTorch kernels with
different summation orders (an elementwise product summed per row, and a
dense matrix product over the batch) stand in for the pages' pair of
kernels; between them some pairs flip and many cached values differ."""
import numpy as np
import pytest
import torch

import bit_quantized_matmul_q4_amd as q4
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    gu.require_gpu()


def tied_problem(seed=0, pairs=1024, K=3584, M=124):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, size=(M, K)).astype(np.float32)
    x[0, 1::2] = x[0, 0::2]  # row 0: equal values at positions 2j, 2j + 1
    x = torch.from_numpy(x).to(torch.bfloat16)
    x[0, 1::2] = x[0, 0::2]  # (exactly equal after rounding too)
    codes = rng.integers(0, 16, size=(2 * pairs, K), dtype=np.uint8)
    swapped = codes[0::2].copy()
    flip = rng.random((pairs, K // 2)) < 0.5
    ev, od = swapped[:, 0::2].copy(), swapped[:, 1::2].copy()
    swapped[:, 0::2] = np.where(flip, od, ev)
    swapped[:, 1::2] = np.where(flip, ev, od)
    codes[1::2] = swapped  # row 2p + 1: row 2p with codes swapped inside position pairs
    scales = np.abs(rng.normal(0, 0.02, size=(pairs, K // 32))).astype(np.float16)
    scales = np.repeat(scales, 2, axis=0)  # both rows of a pair share their scales
    return x, codes, scales


def winners(logits: torch.Tensor) -> torch.Tensor:
    """Per pair, 1 if the second logit is strictly greater, else 0 (greedy
    argmax keeps the first of equal values)."""
    return (logits[1::2] > logits[0::2]).to(torch.int8)


def test_tied_pairs_exact_and_library_invariant():
    x, codes, scales = tied_problem()
    gu.note("invariance demo: %d tied pairs, K=%d" % (codes.shape[0] // 2, codes.shape[1]))
    # the ties are exact in real arithmetic: both rows of a pair have the
    # same multiset of products x_k w_k (each exact in fp64: 8 x 15 bits)
    d = np.repeat(scales.astype(np.float64), 32, axis=1)
    wd = (codes.astype(np.float64) - 8) * d
    x0 = x[0].float().numpy().astype(np.float64)
    terms = np.sort(wd * x0[None, :], axis=1)
    assert np.array_equal(terms[0::2], terms[1::2])

    w = q4.pack(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda())
    xd = x.cuda()
    alone = q4.linear(xd[:1], w, kernel="auto")[0]      # one row: matrix-vector kernel
    batched = q4.linear(xd, w, kernel="auto")[0]        # 124 rows: matrix-matrix kernel
    assert q4.get_crossover() < 124
    assert torch.equal(alone.view(torch.int32), batched.view(torch.int32)), "cache write differs"
    assert torch.equal(winners(alone), winners(batched))

    # the contrast: two plain kernels with different summation orders
    wdev = torch.from_numpy(wd.astype(np.float32)).cuda()  # dequantized weights, exact in fp32
    xf = xd.float()
    gemv_like = (xf[0:1] * wdev).sum(dim=1)                 # per-row reduction
    gemm_like = torch.mm(xf, wdev.t().contiguous())[0]      # dense product over the batch
    differ = int((gemv_like.view(torch.int32) != gemm_like.view(torch.int32)).sum())
    flips = int((winners(gemv_like) != winners(gemm_like)).sum())
    gu.note("contrast kernels: %d of %d cached values differ, %d of %d tied choices flip"
            % (differ, gemv_like.numel(), flips, gemv_like.numel() // 2))
    assert differ > 0 and flips > 0, "the contrast kernels happened to agree; the demonstration needs a new seed"
