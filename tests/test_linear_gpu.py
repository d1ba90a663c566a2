"""Parity of the HIP path with the fp64 oracle, through the C ABI.

Tolerance: max |y_gpu - y_ref| / A <= 2e-3 with A = sum_k |x w| (the bound
the library promises); the expected error of the fixed reduction order is
about 1e-6 (fp16: at most about 73 u of A for any input; bf16: see
test_bf16_sparse_deviation).  Bit-exact where every partial sum is
representable (one-hot read-out, the exact regime, the hand-worked
example)."""
import numpy as np
import pytest

import bit_quantized_matmul_q4_amd as q4
import oracle
import synth
from tests import gpu_util as gu
from tests import oracle_pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    gu.require_gpu()


def check(x_bits, bf16, codes, s_bits, kernel, tol=gu.TOL):
    y = gu.run_linear(x_bits, bf16, codes, s_bits, kernel=kernel).cpu().numpy()
    y_ref, a_ref = oracle.linear(x_bits, bf16, oracle.pack(codes), s_bits)
    err = oracle.max_normalised_error(y, y_ref, a_ref)
    assert err <= tol, "normalised error %.3g > %.3g" % (err, tol)
    return y, y_ref, a_ref


KERNELS = ["gemv", "gemm", "auto"]


@pytest.mark.parametrize("kernel", KERNELS)
def test_hand_example_exact(kernel):
    gu.note("hand example kernel=%s" % kernel)
    g, xv, codes, scales, packed = oracle_pins.hand_example_inputs()
    y_exp = np.array([float(v) for v in g["y"]], np.float32)
    for bf16 in (True, False):
        xb = synth.f64_to_bf16_bits(xv) if bf16 else synth.f64_to_f16_bits(xv)
        y = gu.run_linear(xb, bf16, codes, scales, kernel=kernel).cpu().numpy()
        assert np.array_equal(y[:, 0], y_exp), (kernel, bf16, y[:, 0])


# (M, N, K, bf16): several tiles, ragged N and M tails, K with a short last
# quad, the smallest K, segment counts 1..16; K above 8192 with a short last
# quad (the matrix-matrix kernel's 32-row units, split over K); eight runs a
# tile with a short last quad at 2..8 rows and 5..8 rows with fewer runs,
# one with a short last quad (x in the slot layout, one and two rows per lane
# group);
# 4097 column tiles with K outside the segment form's range (one stream per
# wave: x staged in LDS up to 4 rows, else in the ring)
SHAPES = [
    (1, 896, 896, False), (2, 128, 896, False), (4, 4864, 896, False), (3, 896, 4864, False),
    (1, 16, 32, True), (5, 17, 64, True), (16, 40, 96, True), (17, 33, 160, True),
    (8, 100, 32 * 37, True), (7, 512, 3584, True), (33, 70, 1024, True), (64, 64, 2048, False),
    (100, 130, 640, True), (124, 48, 3584, True), (128, 96, 256, False), (9, 1, 32 * 67, True),
    (40, 50, 8224, True), (70, 150, 9024, False),
    (2, 17, 4128, True), (5, 200, 4128, True), (7, 33, 8224, False), (8, 70, 8224, True),
    (6, 300, 3616, True), (8, 40, 896, False),
    (3, 4100, 3584, True), (2, 4100, 4128, True), (7, 6150, 4864, False),
    (3, 65552, 1024, True), (6, 65552, 1024, False),
    # one row: the prefill's x first (slot layout; a run the prefill holds
    # whole, and a longer one), and x staged once per workgroup for K >= 8192
    # with eight runs a tile, read in the slot layout (bf16; fp16 with a
    # short last quad)
    (1, 512, 3584, True), (1, 200, 4864, True), (1, 130, 18944, True), (1, 70, 8224, False),
]


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
@pytest.mark.parametrize("M,N,K,bf16", SHAPES)
def test_parity_random(M, N, K, bf16, kernel):
    gu.note("parity M=%d N=%d K=%d bf16=%s kernel=%s" % (M, N, K, bf16, kernel))
    x, codes, s = synth.problem(N, K, M, "bf16" if bf16 else "f16", workload=91, matrix=N * 7 + K)
    check(x, bf16, codes, s, kernel)


# Wide N with 2048 <= K <= 6144 takes the matrix-vector kernel's
# segment-stationary form (above 256 column tiles with 1-quad segments, above
# 512 otherwise or from 5 rows on): segments of 1, 2 and 3 quads, a short
# last quad, ragged last tile and rows, 1..3 tiles per workgroup with a
# partial last workgroup.
SEG_SHAPES = [
    (1, 4100, 2048, True), (2, 4112, 2080, False), (3, 8210, 3584, True), (2, 8210, 4128, True),
    (9, 4100, 2048, False), (1, 8210, 2048, True), (8, 4352, 3584, True), (16, 4112, 3584, True),
    (13, 8210, 2080, False),
    # up to four rows x staged by the workgroup, scales in groups, a short
    # last quad
    (2, 8210, 2080, True), (4, 12000, 3616, False),
]


@pytest.mark.parametrize("M,N,K,bf16", SEG_SHAPES)
def test_segment_form_parity_and_bits(M, N, K, bf16):
    gu.note("segment form M=%d N=%d K=%d bf16=%s" % (M, N, K, bf16))
    x, codes, s = synth.problem(N, K, M, "bf16" if bf16 else "f16", workload=92, matrix=N * 7 + K)
    y, _, _ = check(x, bf16, codes, s, "gemv")
    y_mm = gu.run_linear(x, bf16, codes, s, kernel="gemm").cpu().numpy()
    assert np.array_equal(y.view(np.uint32), y_mm.view(np.uint32))


# bf16 split-form runs that the prefill holds whole (at most 4 quads) take x
# first and compute every stage's corrections before the codes arrive, up to
# 8 rows, x in the slot layout: eight runs of 3-4 quads a tile (K = 3584) and
# runs of 1-2 quads (K = 896), 2-3 quads (K = 1184) and 4 quads (K = 992),
# the last two with a short last quad.
WHOLE_RUN_SHAPES = [(512, 3584), (300, 896), (70, 1184), (600, 992)]


@pytest.mark.parametrize("N,K", WHOLE_RUN_SHAPES)
def test_runs_held_whole_parity_and_bits(N, K):
    x, codes, s = synth.problem(N, K, 8, "bf16", workload=94, matrix=N * 7 + K)
    y_mm = gu.run_linear(x, True, codes, s, kernel="gemm").cpu().numpy().view(np.uint32)
    for M in range(1, 9):
        gu.note("whole runs M=%d N=%d K=%d" % (M, N, K))
        y, _, _ = check(x[:M], True, codes, s, "gemv")
        assert np.array_equal(y.view(np.uint32), y_mm[:M]), M


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
@pytest.mark.parametrize("bf16", [True, False])
def test_one_hot_readout_exact(kernel, bf16):
    """x = e_k reads out (q[n][k] - 8) d[n][k/32] exactly for every k."""
    gu.note("one-hot kernel=%s bf16=%s" % (kernel, bf16))
    rng = np.random.default_rng(21)
    N, K = 40, 128
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = oracle_pins.random_scale_bits(rng, (N, K // 32))
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = 0x3F80 if bf16 else 0x3C00
    y = gu.run_linear(x, bf16, codes, s, kernel=kernel).cpu().numpy()
    y_ref, _ = oracle.linear(x, bf16, oracle.pack(codes), s)
    assert np.array_equal(y, y_ref.astype(np.float32))


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("K", [32, 3584, 18944])
def test_exact_regime(kernel, bf16, K):
    """Integer x in [-4, 4], scales 2^-1..2^-4: every block dot is an integer
    (bf16: D and E below 2^12, and their difference; fp16: the exact-operand
    sum, at most 1024 in magnitude), and every partial is a multiple of 2^-4
    below 2^19, so all are exact and the outputs equal the oracle's."""
    gu.note("exact regime kernel=%s bf16=%s K=%d" % (kernel, bf16, K))
    rng = np.random.default_rng(22 + K + int(bf16))
    M, N = 6, 48
    xv = rng.integers(-4, 5, size=(M, K)).astype(np.float64)
    x = synth.f64_to_bf16_bits(xv) if bf16 else synth.f64_to_f16_bits(xv)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = synth.f64_to_f16_bits(2.0 ** -rng.integers(1, 5, size=(N, K // 32)))
    y = gu.run_linear(x, bf16, codes, s, kernel=kernel).cpu().numpy()
    y_ref, _ = oracle.linear(x, bf16, oracle.pack(codes), s)
    assert np.array_equal(y, y_ref.astype(np.float32))


def sparse_deviation_codes(rng, N, K):
    """Codes 8 everywhere except one 7 or 9 per block of 32: every block has a
    single non-zero weight, so A is as small as the weights allow."""
    codes = np.full((N, K), 8, np.uint8)
    nb = K // 32
    pos = 32 * np.arange(nb)[None, :] + rng.integers(0, 32, size=(N, nb))
    codes[np.arange(N)[:, None], pos] = rng.choice(np.array([7, 9], np.uint8), size=(N, nb))
    return codes


# u = 2^-24; fp16 block dots have exact operands, so a zero weight adds
# nothing and the error of the whole order is at most about
# (31 + L + log2 S + 1) u of A (L <= 37 blocks per segment)
F16_ORDER_BOUND = (31 + 37 + 4 + 1) * 2.0 ** -24


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
@pytest.mark.parametrize("K", [32, 896])
def test_f16_sparse_deviation_worst_regime(kernel, K):
    """fp16 activations of one sign between 1 and 4000 (per row) against
    blocks with a single non-zero weight: where an offset operand would
    cancel most.  The exact (q - 8) operand keeps the error at the order's
    accumulation bound, far below 2e-3."""
    gu.note("fp16 sparse deviation kernel=%s K=%d" % (kernel, K))
    rng = np.random.default_rng(24 + K)
    M, N = 24, 80
    sign = np.where(rng.random((M, 1)) < 0.5, 1.0, -1.0)
    xv = sign * rng.uniform(1.0, 4000.0, size=(M, K))
    x = synth.f64_to_f16_bits(xv)
    codes = sparse_deviation_codes(rng, N, K)
    s = synth.scales(N, K, workload=94)
    y = gu.run_linear(x, False, codes, s, kernel=kernel).cpu().numpy()
    y_ref, a_ref = oracle.linear(x, False, oracle.pack(codes), s)
    err = oracle.max_normalised_error(y, y_ref, a_ref)
    assert err <= gu.TOL, err
    assert err <= F16_ORDER_BOUND, err


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
@pytest.mark.parametrize("K", [32, 896, 3584])
def test_bf16_sparse_deviation(kernel, K):
    """bf16 with one non-zero weight per block.  The bf16 block dot is the
    MFMA of the operand 16 + q with the correction MFMA(x, -24) as its
    accumulator input, so its error is bounded by the block's sum of |x|
    rather than by A: |s_b - exact| <= 33 u (31 + 24 (2 + 33 u)) sum|x|.
    Checked output by output against the oracle with
    that bound carried through the scale and accumulation steps.  Against
    2e-3 of A: integer activations up to 4000 (every D and E exact), and
    N(0, 1) activations from K = 896 on (at K = 32 a block whose only
    non-zero weight meets a tiny activation can exceed it: the known limit
    of the offset operand)."""
    gu.note("bf16 sparse deviation kernel=%s K=%d" % (kernel, K))
    rng = np.random.default_rng(25 + K)
    M, N = 24, 80
    codes = sparse_deviation_codes(rng, N, K)
    s = synth.scales(N, K, workload=95)
    d = gu.f16_bits_to_f64(s)
    u = 2.0 ** -24
    for name, xv in (("normal", rng.normal(0.0, 1.0, size=(M, K))),
                     ("integers", np.where(rng.random((M, 1)) < 0.5, 1.0, -1.0)
                      * rng.integers(1, 4001, size=(M, K)).astype(np.float64))):
        x = synth.f64_to_bf16_bits(xv)
        y = gu.run_linear(x, True, codes, s, kernel=kernel).cpu().numpy()
        y_ref, a_ref = oracle.linear(x, True, oracle.pack(codes), s)
        if name == "integers" or K >= 896:
            err = oracle.max_normalised_error(y, y_ref, a_ref)
            assert err <= gu.TOL, (name, err)
        if name == "integers" and K == 32:  # one block: y = fl(d s), s exact
            assert np.array_equal(y, y_ref.astype(np.float32))
        # the absolute bound, from the blocks' sums of |x| and the scales
        xa = np.abs((np.asarray(x, np.uint32) << 16).view(np.float32).astype(np.float64))
        xsum = xa.reshape(M, K // 32, 32).sum(axis=2)  # [M, nb]
        blk = (33 * u * (31.0 + 24.0 * (2.0 + 33 * u))) * xsum @ d.T  # sum_b d_b (block-dot bound)
        bound = blk + F16_ORDER_BOUND * a_ref           # plus the accumulation's
        assert np.all(np.abs(y.astype(np.float64) - y_ref) <= bound), name


@pytest.mark.parametrize("kernel", ["gemv", "gemm"])
def test_special_cases(kernel):
    gu.note("special cases kernel=%s" % kernel)
    rng = np.random.default_rng(23)
    M, N, K = 5, 37, 256
    x = synth.activations(M, K, "bf16", workload=92)
    s = synth.scales(N, K, workload=92)
    # all codes 8 -> zeros
    y = gu.run_linear(x, True, np.full((N, K), 8, np.uint8), s, kernel=kernel)
    assert (y == 0).all()
    # zero input -> zeros
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    y = gu.run_linear(np.zeros((M, K), np.uint16), True, codes, s, kernel=kernel)
    assert (y == 0).all()
    # single block: y = fl(d * s) with s exact
    xk = synth.f64_to_bf16_bits(rng.integers(-3, 4, size=(M, 32)).astype(np.float64))
    y = gu.run_linear(xk, True, np.ascontiguousarray(codes[:, :32]), np.ascontiguousarray(s[:, :1]),
                      kernel=kernel).cpu().numpy()
    y_ref, _ = oracle.linear(xk, True, oracle.pack(codes[:, :32]), s[:, :1])
    assert np.array_equal(y, y_ref.astype(np.float32))
    # subnormal and zero scales, random bit-pattern activations
    s2 = oracle_pins.random_scale_bits(rng, (N, K // 32))
    x2 = oracle_pins.random_finite_bits(rng, (M, K), bf16=False)
    check(x2, False, codes, s2, kernel)


@pytest.mark.parametrize("workload", [1, 2])
def test_small_workloads_full(workload):
    """The 0.5B-shaped workloads, every matrix and every M, both kernels."""
    spec = synth.WORKLOADS[workload]
    bf16 = spec["x"] == "bf16"
    for mi, mat in enumerate(spec["matrices"]):
        Mmax = max(spec["Ms"])
        x, codes, s = synth.problem(mat.N, mat.K, Mmax, spec["x"], workload, mi)
        y_ref, a_ref = oracle.linear(x, bf16, oracle.pack(codes), s)
        w = gu.pack_dev(codes, s)
        for M in spec["Ms"]:
            for kernel in ("auto", "gemv", "gemm"):
                gu.note("workload %d %s M=%d kernel=%s" % (workload, mat.name, M, kernel))
                y = q4.linear(gu.x_to_dev(x[:M], bf16), w, kernel=kernel).cpu().numpy()
                err = oracle.max_normalised_error(y, y_ref[:M], a_ref[:M])
                assert err <= gu.TOL, (mat.name, M, kernel, err)


# The matrix-matrix kernel's grid: many row units (M = 300: 19 units of 16
# rows), column units that do not fill the last group of eight (the spare
# workgroups return), 32-row units above K = 8192, and K split over 2..16
# groups with a short last quad; with and without the split workspace.
GEMM_GRID_SHAPES = [
    (300, 200, 1024, True), (70, 1000, 9024, False), (33, 4100, 2080, True), (129, 16, 4128, True),
]


@pytest.mark.parametrize("M,N,K,bf16", GEMM_GRID_SHAPES)
def test_gemm_grid_parity_and_bits(M, N, K, bf16):
    gu.note("gemm grid M=%d N=%d K=%d bf16=%s" % (M, N, K, bf16))
    x, codes, s = synth.problem(N, K, M, "bf16" if bf16 else "f16", workload=93, matrix=N * 7 + K)
    y, _, _ = check(x, bf16, codes, s, "gemm")
    w = gu.pack_dev(codes, s)
    xd = gu.x_to_dev(x, bf16)
    y_plain = q4.linear(xd, w, kernel="gemm", workspace=None).cpu().numpy()  # no K split
    y_mv = q4.linear(xd, w, kernel="gemv").cpu().numpy()
    assert np.array_equal(y.view(np.uint32), y_plain.view(np.uint32))
    assert np.array_equal(y.view(np.uint32), y_mv.view(np.uint32))
