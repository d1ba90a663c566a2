"""Full-size 7B-shaped matrices, in the launch configuration the benchmark
times: outputs sampled against the oracle (which computes them one by one
from the canonical codes, never from the GPU's packed bytes), the whole
GPU-packed buffer against the oracle's packing, and the bit contract
between the kernels at full size."""
import numpy as np
import pytest
import torch

import bit_quantized_matmul_q4_amd as q4
import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SAMPLES = 1500


def sampled_check(x_bits, wq, sc, K, y, rng, bf16=True, tiled=False):
    """wq, sc: the weight as host arrays -- canonical nibble rows [N, K/2]
    and scale bits [N, K/32], or (tiled=True) a packed weight drawn directly
    in the library layout by the seeded generator."""
    M, N = y.shape
    ms = rng.integers(0, M, SAMPLES)
    ns = rng.integers(0, N, SAMPLES)
    # always include the corners (tails of both dimensions)
    ms = np.concatenate([ms, [0, M - 1, 0, M - 1]])
    ns = np.concatenate([ns, [0, 0, N - 1, N - 1]])
    y_ref, a_ref = oracle.linear_sampled(x_bits, bf16, wq, sc, ms, ns, tiled_nk=(N, K) if tiled else None)
    err = oracle.max_normalised_error(y[ms, ns], y_ref, a_ref)
    assert err <= gu.TOL, err


@pytest.fixture(scope="module", autouse=True)
def gpu():
    gu.require_gpu()


@pytest.mark.parametrize("mi", range(6))
def test_7b_layer_set(mi):
    mat = synth.SET_7B[mi]
    rng = np.random.default_rng(40 + mi)
    x, codes, s = synth.problem(mat.N, mat.K, 124, "bf16", workload=3, matrix=mi)
    gu.note("7B %s pack" % mat.name)
    xd, w = gu.x_to_dev(x, True), gu.pack_dev(codes, s)
    # the whole packed buffer the GPU made is the oracle's packing of the codes
    wq_o, sc_o = oracle.pack_tiled(codes, s)
    assert np.array_equal(w.codes.cpu().numpy(), wq_o)
    assert np.array_equal(w.scales.view(torch.int16).cpu().numpy().view(np.uint16), sc_o)
    del wq_o, sc_o
    canon = oracle.pack(codes)  # canonical nibble rows: the oracle's own input
    gu.note("7B %s M=8 gemv" % mat.name)
    y8 = q4.linear(xd[:8], w, kernel="gemv")
    torch.cuda.synchronize()
    y8h = y8.cpu().numpy()
    sampled_check(x[:8], canon, s, mat.K, y8h, rng)
    for M in (1, 3, 8, 16, 124):
        for kernel in ("auto", "gemv", "gemm"):
            gu.note("7B %s M=%d %s" % (mat.name, M, kernel))
            y = q4.linear(xd[:M], w, kernel=kernel).cpu().numpy()
            assert np.array_equal(y[: min(M, 8)].view(np.uint32), y8h[: min(M, 8)].view(np.uint32))
            if M == 124:
                sampled_check(x[:124], canon, s, mat.K, y, rng)


def test_lm_head_sampled():
    mat = synth.LM_HEAD_7B
    rng = np.random.default_rng(50)
    x = synth.activations(64, mat.K, "bf16", workload=5, matrix=6)
    wq_t, sc_t = synth.packed_weight(mat.N, mat.K, workload=5, matrix=6)
    xd, w = gu.x_to_dev(x, True), gu.weight_from_tiled(wq_t, sc_t, mat.N, mat.K)
    ys = {}
    for M in (1, 4, 16, 64):
        gu.note("lm_head M=%d" % M)
        ys[M] = q4.linear(xd[:M], w).cpu().numpy()
        sampled_check(x[:M], wq_t, sc_t, mat.K, ys[M], rng, tiled=True)
    for M in (1, 4, 16):
        assert np.array_equal(ys[64][:M].view(np.uint32), ys[M].view(np.uint32))


def test_gemm_large_grid_repeatable():
    """The matrix-matrix kernel on the LM head (thousands of workgroups),
    repeated: every call's rows are bit-identical to the matrix-vector
    kernel's.  (An activation stage once raced its loads: a few workgroups
    per call read stale chunks, different ones each time.)"""
    mat = synth.LM_HEAD_7B
    x = synth.activations(64, mat.K, "bf16", workload=5, matrix=7)
    wq_t, sc_t = synth.packed_weight(mat.N, mat.K, workload=5, matrix=7)
    xd, w = gu.x_to_dev(x, True), gu.weight_from_tiled(wq_t, sc_t, mat.N, mat.K)
    ref = q4.linear(xd[:16], w, kernel="gemv").cpu().numpy().view(np.uint32)
    for M in (17, 20, 33, 64, 17, 20, 33, 64):
        gu.note("lm_head gemm repeat M=%d" % M)
        y = q4.linear(xd[:M], w, kernel="gemm").cpu().numpy().view(np.uint32)
        assert np.array_equal(y[:16], ref), (M, int((y[:16] != ref).sum()))
