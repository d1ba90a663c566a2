"""Bitwise invariance of every output row.

A row's bits depend only on its own x row, the weights and K: not on M, on
the row's position, on the other rows, on which kernel ran, on the
workspace split, on repetition, or on slicing N.  This is the property whose
absence "Why Continuous Batching Slowed Down My LLM Inference Engine: A Metal
Kernel Investigation" traces (sections "Same Prompt, Different Story" and
"The Other Request Already Finished"): forcing every input through one
kernel made the serial and batched runs agree again."""
import numpy as np
import pytest
import torch

import bit_quantized_matmul_q4_amd as q4
import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

K = 3584
N = 160


@pytest.fixture(scope="module")
def prob():
    gu.require_gpu()
    x, codes, s = synth.problem(N, K, 128, "bf16", workload=93, matrix=0)
    xd, w = gu.x_to_dev(x, True), gu.pack_dev(codes, s)
    rows = []
    for m in range(128):
        rows.append(q4.linear(xd[m:m + 1].contiguous(), w, kernel="gemv"))
    torch.cuda.synchronize()
    ref = torch.cat(rows).cpu().numpy().view(np.uint32)
    y_or, a_or = oracle.linear(x, True, oracle.pack(codes), s)
    err = oracle.max_normalised_error(ref.view(np.float32), y_or, a_or)
    assert err <= gu.TOL
    return x, xd, w, codes, s, ref


MS = list(range(1, 18)) + [31, 32, 33, 64, 100, 124, 128]


@pytest.mark.parametrize("kernel", ["gemv", "gemm", "auto"])
def test_rows_independent_of_m(prob, kernel):
    x, xd, w, codes, s, ref = prob
    for M in MS:
        gu.note("invariance over M=%d kernel=%s" % (M, kernel))
        y = q4.linear(xd[:M], w, kernel=kernel)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref[:M]), (M, kernel)


def test_workspace_split_same_bits(prob):
    x, xd, w, codes, s, ref = prob
    for M in (9, 64, 124):
        gu.note("workspace split M=%d" % M)
        a = q4.linear(xd[:M], w, kernel="gemm", workspace=True)
        b = q4.linear(xd[:M], w, kernel="gemm", workspace=None)
        assert np.array_equal(a.cpu().numpy().view(np.uint32), ref[:M])
        assert np.array_equal(b.cpu().numpy().view(np.uint32), ref[:M])


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
def test_permutation_and_companions(prob, kernel):
    x, xd, w, codes, s, ref = prob
    rng = np.random.default_rng(31)
    gu.note("permutation kernel=%s" % kernel)
    perm = rng.permutation(128)
    y = q4.linear(xd[torch.from_numpy(perm).to(gu.DEV)].contiguous(), w, kernel=kernel)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), ref[perm])
    gu.note("companion rows kernel=%s" % kernel)
    other = synth.f64_to_bf16_bits(rng.normal(0, 30, size=(40, K)))
    xm = np.concatenate([other[:17], x[5:6], other[17:]])
    y = q4.linear(gu.x_to_dev(xm, True), w, kernel=kernel)
    assert np.array_equal(y.cpu().numpy().view(np.uint32)[17], ref[5])


def test_repeat_runs_identical(prob):
    x, xd, w, codes, s, ref = prob
    for kernel in ("gemv", "gemm"):
        gu.note("repeat kernel=%s" % kernel)
        outs = [q4.linear(xd[:37], w, kernel=kernel).cpu().numpy().view(np.uint32) for _ in range(4)]
        for o in outs:
            assert np.array_equal(o, ref[:37])


def test_mixed_124_rows(prob):
    """120 prefill + 4 verify rows: each verify row equals its M=4 and M=1
    results, whichever kernel ran the 124-row batch."""
    x, xd, w, codes, s, ref = prob
    for kernel in ("auto", "gemv", "gemm"):
        gu.note("mixed 124 kernel=%s" % kernel)
        y124 = q4.linear(xd[:124], w, kernel=kernel).cpu().numpy().view(np.uint32)
        y4 = q4.linear(xd[120:124].contiguous(), w, kernel="auto").cpu().numpy().view(np.uint32)
        assert np.array_equal(y124[120:124], y4)
        assert np.array_equal(y124, ref[:124])


def test_n_sharding(prob):
    """Row slices of W give the column slices of y, bit for bit (the segment
    count depends on K only): slices packed on their own, and tile-aligned
    slices cut straight out of the packed weight."""
    x, xd, w, codes, s, ref = prob
    for (n0, n1) in ((0, 16), (16, 80), (80, 160), (37, 121)):
        for kernel in ("gemv", "gemm"):
            gu.note("shard %d:%d kernel=%s" % (n0, n1, kernel))
            ws = gu.pack_dev(np.ascontiguousarray(codes[n0:n1]), np.ascontiguousarray(s[n0:n1]))
            y = q4.linear(xd[:20], ws, kernel=kernel)
            assert np.array_equal(y.cpu().numpy().view(np.uint32), ref[:20, n0:n1])
    G = (K // 32 + 3) // 4
    for (t0, t1) in ((0, 1), (1, 5), (5, 10)):
        sl = q4.Q4Weight(w.codes[t0 * G * 1024:t1 * G * 1024], w.scales[t0 * G * 64:t1 * G * 64],
                         16 * (t1 - t0), K)
        y = q4.linear(xd[:20], sl, kernel="gemv")
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref[:20, 16 * t0:16 * t1])


def test_fused_n_concat(prob):
    """Weights sharing K, concatenated along N (one fused launch, as for
    q|k|v or gate|up), give every part's columns bit for bit; split_n views
    of the fused buffers give each part back."""
    x, xd, w, codes, s, ref = prob
    parts = [(0, 48), (48, 80), (80, 117)]
    ws = [gu.pack_dev(np.ascontiguousarray(codes[a:b]), np.ascontiguousarray(s[a:b])) for a, b in parts]
    fused = q4.concat_n(ws)
    assert fused.N == 117
    for kernel in ("gemv", "gemm"):
        gu.note("fused concat kernel=%s" % kernel)
        y = q4.linear(xd[:20], fused, kernel=kernel)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref[:20, 0:117])
    for (a, b), v in zip(parts, q4.split_n(fused, [48, 32, 37])):
        y = q4.linear(xd[:20], v, kernel="gemv")
        assert np.array_equal(y.cpu().numpy().view(np.uint32), ref[:20, a:b])
    with pytest.raises(ValueError):
        q4.concat_n([ws[2], ws[0]])  # a part before the last with N % 16 != 0
    with pytest.raises(ValueError):
        q4.split_n(fused, [40, 77])
