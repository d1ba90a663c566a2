"""q4_linear_grouped -- several matrices that share x in one launch -- and
q4_pack_nibbles, through the C ABI.

The group's outputs must be bit-identical to one q4_linear_ex call per
matrix (the reduction order depends on K only) and within the oracle's
tolerance: the 7B layer's q, k, v, gate and up projections (one launch of
the matrix-vector kernel's segment form) at 1..16 rows, past the crossover
(one call per matrix), ragged and tiny matrices in one group, K the segment
form does not take (one launch of the split form: the 0.5B layer's five
projections that share x, GPT-2's q, k and v, K = 896, 6176 and 18944), and
a group too wide for one launch (one call per matrix)."""
import numpy as np
import pytest
import torch

import bit_quantized_matmul_q4_amd as q4
import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    gu.require_gpu()


def check_group(x, bf16, mats, Ms, workload, sample_rng=None, workspace=True):
    """mats: list of (N, K); all share x [Mmax, K]."""
    K = mats[0][1]
    probs = [synth.problem(N, K, 1, "bf16", workload=workload, matrix=i)[1:] for i, (N, _) in enumerate(mats)]
    ws = [gu.pack_dev(c, s) for c, s in probs]
    xd = gu.x_to_dev(x, bf16)
    for M in Ms:
        gu.note("grouped %d matrices K=%d M=%d" % (len(mats), K, M))
        ys = q4.linear_grouped(xd[:M], ws, workspace=workspace)
        torch.cuda.synchronize()
        for i, (w, y) in enumerate(zip(ws, ys)):
            ref = q4.linear(xd[:M], w).cpu().numpy().view(np.uint32)
            assert np.array_equal(y.cpu().numpy().view(np.uint32), ref), (i, M)
        if sample_rng is not None:
            for i, (w, y) in enumerate(zip(ws, ys)):
                c, s = probs[i]
                ms = sample_rng.integers(0, M, 300)
                ns = sample_rng.integers(0, w.N, 300)
                y_ref, a_ref = oracle.linear_sampled(x[:M], bf16, oracle.pack(c), s, ms, ns)
                err = oracle.max_normalised_error(y.cpu().numpy()[ms, ns], y_ref, a_ref)
                assert err <= gu.TOL, (i, M, err)


def test_grouped_7b_qkv_gate_up():
    mats = [(m.N, m.K) for m in synth.SET_7B[:5]]
    x = synth.activations(24, 3584, "bf16", workload=8, matrix=0)
    check_group(x, True, mats, [1, 2, 3, 4, 5, 8, 9, 16, 17, 24], workload=8, sample_rng=np.random.default_rng(60))


@pytest.mark.parametrize("bf16", [True, False])
def test_grouped_ragged(bf16):
    """Column counts that are not multiples of 16 anywhere in the group, a
    one-tile matrix, and the maximum group size (8)."""
    mats = [(100, 2048), (17, 2048), (300, 2048), (1, 2048), (4100, 2048), (16, 2048), (33, 2048), (2000, 2048)]
    x = synth.activations(12, 2048, "bf16" if bf16 else "f16", workload=9, matrix=0)
    check_group(x, bf16, mats, [1, 3, 7, 12], workload=9, sample_rng=np.random.default_rng(61))


def test_grouped_other_k():
    """K = 896 (4 segments) and K = 6176 (the segment form's limit passed):
    one launch of the split form, same bits."""
    for K in (896, 6176):
        mats = [(128, K), (896, K), (40, K)]
        x = synth.activations(6, K, "f16", workload=10, matrix=K)
        check_group(x, False, mats, [1, 4, 6], workload=10, sample_rng=np.random.default_rng(62))


def test_grouped_05b_layer():
    """The 0.5B layer's q, k, v, gate and up (K = 896, fp16 x) in one launch."""
    mats = [(m.N, m.K) for m in synth.SET_05B[:5]]
    x = synth.activations(16, 896, "f16", workload=2, matrix=0)
    check_group(x, False, mats, [1, 2, 3, 4, 8, 16], workload=2, sample_rng=np.random.default_rng(63))


def test_grouped_gpt2_qkv():
    """GPT-2-small's q, k and v (768 x 768, bf16 x) in one launch at 1..16 rows."""
    mats = [(m.N, m.K) for m in synth.SET_GPT2[:3]]
    x = synth.activations(16, 768, "bf16", workload=6, matrix=0)
    check_group(x, True, mats, list(range(1, 17)), workload=6, sample_rng=np.random.default_rng(64))


@pytest.mark.parametrize("workspace", [True, False])
def test_grouped_long_k(workspace):
    """K = 18944: one launch up to 8 rows; at 9..16 rows one launch without a
    workspace, one matrix-matrix call per matrix with one."""
    mats = [(3584, 18944), (512, 18944), (100, 18944)]
    x = synth.activations(12, 18944, "bf16", workload=12, matrix=0)
    check_group(x, True, mats, [1, 5, 8, 12], workload=12, sample_rng=np.random.default_rng(65),
                workspace=workspace)


def test_grouped_too_wide():
    """70000 columns in all with K = 256: too wide for one launch, one call
    per matrix."""
    mats = [(30000, 256), (30000, 256), (10000, 256)]
    x = synth.activations(3, 256, "bf16", workload=13, matrix=0)
    check_group(x, True, mats, [1, 3], workload=13, sample_rng=np.random.default_rng(66))


@pytest.mark.parametrize("N,K", [(16, 32), (17, 96), (300, 3584), (18944, 3584), (3584, 18944)])
def test_pack_nibbles_bit_exact(N, K):
    """q4_pack_nibbles on the canonical nibble rows gives the oracle's packing
    byte for byte (and the same bytes as q4_pack on one code per byte)."""
    gu.note("pack_nibbles N=%d K=%d" % (N, K))
    codes = synth.codes(N, K, workload=11, matrix=N)
    s = synth.scales(N, K, workload=11, matrix=N)
    rows = oracle.pack(codes)
    w = q4.pack_nibbles(gu.u8_to_dev(rows), gu.scales_to_dev(s))
    wq_o, sc_o = oracle.pack_tiled(codes, s)
    assert np.array_equal(w.codes.cpu().numpy(), wq_o)
    assert np.array_equal(w.scales.view(torch.int16).cpu().numpy().view(np.uint16), sc_o)
