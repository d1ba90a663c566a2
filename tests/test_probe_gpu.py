"""Hardware checks of what the fixed reduction order rests on (gfx950).

* the MFMA 16x16x32 lane layout the kernels assume;
* slot invariance: an MFMA result element depends only on its own A row and
  B column -- not on the slot it sits in nor on the other rows/columns --
  which is what lets a row's bits ignore M and the other rows;
* run-to-run determinism;
* exactness when every partial sum is representable;
* the nibble dequantization gives the operand exactly for every code at
  every position of a packed word: 16 + q in bf16, q - 8 in fp16;
* the bf16 corrected block dot: the correction C = MFMA(x, -24) is the same
  for every column and the exact negation of MFMA(x, 24); the block dot is
  the MFMA of the dequantized operand 16 + q with C as its accumulator
  input, and is within the fp32 accumulation bound of the exact sum of
  x (q - 8);
* the fp16 block dot D = MFMA(x, q - 8) is within the fp32 accumulation
  bound of the exact sum relative to sum |x (q - 8)| (zero weights add
  exactly nothing), and a block with one non-zero weight is exact;
* fmaf(d, s, 0) is the single-rounded product (no flush of subnormals).
"""
import numpy as np
import pytest

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    gu.require_gpu()
    return gu.Probe()


def enc(v: np.ndarray, bf16: bool) -> np.ndarray:
    v = np.asarray(v, np.float64)
    if bf16:
        return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    return v.astype(np.float16).view(np.uint16)


def dec(bits: np.ndarray, bf16: bool) -> np.ndarray:
    b = np.asarray(bits, np.uint16)
    if bf16:
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return b.view(np.float16).astype(np.float64)


def to_lanes(A: np.ndarray, B: np.ndarray):
    """A [w,16,32], B [w,32,16] (uint16 bits) -> lane arrays [w,64,8] in the
    assumed layout: lane l holds A[l%16][8(l/16)+e] and B[8(l/16)+e][l%16]."""
    w = A.shape[0]
    l = np.arange(64)
    e = np.arange(8)
    rows = (l % 16)[:, None]
    ks = (8 * (l // 16))[:, None] + e[None, :]
    a = A[:, rows, ks]
    b = B[:, ks, rows]
    return a.reshape(w, 64, 8), b.reshape(w, 64, 8)


def from_lanes(d: np.ndarray) -> np.ndarray:
    """[w,64,4] -> D [w,16,16] with lane l, reg i = D[4(l/16)+i][l%16]."""
    w = d.shape[0]
    D = np.empty((w, 16, 16), np.float32)
    for l in range(64):
        for i in range(4):
            D[:, 4 * (l // 16) + i, l % 16] = d[:, l, i]
    return D


@pytest.mark.parametrize("bf16", [True, False])
def test_mfma_layout_exact(probe, bf16):
    gu.note("mfma layout bf16=%s" % bf16)
    rng = np.random.default_rng(10)
    w = 16
    A = rng.integers(-4, 5, size=(w, 16, 32)).astype(np.float64)
    B = rng.integers(-4, 5, size=(w, 32, 16)).astype(np.float64)
    a, b = to_lanes(enc(A, bf16), enc(B, bf16))
    D = from_lanes(probe.mfma(a, b, bf16))
    assert np.array_equal(D, (A @ B).astype(np.float32))


@pytest.mark.parametrize("bf16", [True, False])
def test_mfma_exact_regime(probe, bf16):
    """Integers times dyadic values whose every partial sum fits fp32: exact."""
    gu.note("mfma exact regime bf16=%s" % bf16)
    rng = np.random.default_rng(11)
    w = 32
    A = rng.integers(-4, 5, size=(w, 16, 32)) * 2.0 ** rng.integers(-6, 7, size=(w, 16, 1))
    B = (rng.integers(0, 16, size=(w, 32, 16)) - 8) / 16.0
    a, b = to_lanes(enc(A, bf16), enc(B, bf16))
    D = from_lanes(probe.mfma(a, b, bf16))
    assert np.array_equal(D, np.einsum("wik,wkj->wij", A, B).astype(np.float32))


@pytest.mark.parametrize("bf16", [True, False])
def test_mfma_slot_invariance_and_determinism(probe, bf16):
    gu.note("mfma slot invariance bf16=%s" % bf16)
    rng = np.random.default_rng(12)
    w = 256
    A = enc(rng.normal(0, 1, size=(w, 16, 32)), bf16)
    Bq = (rng.integers(0, 16, size=(w, 32, 16)) - 8) / 16.0
    B = enc(Bq, bf16)
    a, b = to_lanes(A, B)
    D = from_lanes(probe.mfma(a, b, bf16))
    # determinism
    for _ in range(3):
        assert np.array_equal(from_lanes(probe.mfma(a, b, bf16)).view(np.uint32), D.view(np.uint32))
    # permuted slots: rows and columns move, values keep their bits
    pr = np.stack([rng.permutation(16) for _ in range(w)])
    pc = np.stack([rng.permutation(16) for _ in range(w)])
    A2 = np.take_along_axis(A, pr[:, :, None], axis=1)
    B2 = np.take_along_axis(B, pc[:, None, :], axis=2)
    a2, b2 = to_lanes(A2, B2)
    D2 = from_lanes(probe.mfma(a2, b2, bf16))
    expect = np.take_along_axis(np.take_along_axis(D, pr[:, :, None], axis=1), pc[:, None, :], axis=2)
    assert np.array_equal(D2.view(np.uint32), expect.view(np.uint32))
    # other rows replaced by unrelated data: row 0 and column 0 keep their bits
    A3 = enc(rng.normal(0, 100, size=(w, 16, 32)), bf16)
    A3[:, 0, :] = A[:, 0, :]
    B3 = enc(rng.normal(0, 1, size=(w, 32, 16)), bf16)
    B3[:, :, 0] = B[:, :, 0]
    a3, b3 = to_lanes(A3, B3)
    D3 = from_lanes(probe.mfma(a3, b3, bf16))
    assert np.array_equal(D3[:, 0, 0].view(np.uint32), D[:, 0, 0].view(np.uint32))
    # zero rows (unused batch slots) do not change the used ones
    A4 = A.copy()
    A4[:, 1:, :] = 0
    a4, b4 = to_lanes(A4, B)
    D4 = from_lanes(probe.mfma(a4, b4, bf16))
    assert np.array_equal(D4[:, 0, :].view(np.uint32), D[:, 0, :].view(np.uint32))
    assert np.all(D4[:, 1:, :] == 0)


SHIFTS = (4 * (np.arange(8) // 2) + 16 * (np.arange(8) % 2)).astype(np.uint32)  # code r's bit


def operand_bits(q: np.ndarray, bf16: bool) -> np.ndarray:
    """The B operand the order defines for codes q: 16 + q (bf16), q - 8 (fp16)."""
    q = np.asarray(q, np.int64)
    return enc(q + 16.0, True) if bf16 else enc(q - 8.0, False)


def lane_words(q: np.ndarray) -> np.ndarray:
    """Codes [w, 32, 16] (k, column) -> one packed word per lane [w, 64]:
    lane l = 16 g + c holds column c, k = 8 g + r, code r at SHIFTS[r]."""
    l = np.arange(64)
    ks = (8 * (l // 16))[:, None] + np.arange(8)[None, :]
    lane_codes = q[:, ks, (l % 16)[:, None]].astype(np.uint32)  # [w, 64, 8]
    return (lane_codes << SHIFTS).sum(axis=-1, dtype=np.uint32)


@pytest.mark.parametrize("bf16", [True, False])
def test_dequant_every_code_every_position(probe, bf16):
    gu.note("dequant bf16=%s" % bf16)
    rng = np.random.default_rng(13)
    words = np.concatenate([np.arange(16, dtype=np.uint64) * 0x11111111,
                            rng.integers(0, 1 << 32, size=4096, dtype=np.uint64)]).astype(np.uint32)
    got = probe.dequant(words, bf16)
    codes = (words[:, None] >> SHIFTS[None, :]) & 0xF
    assert np.array_equal(got, operand_bits(codes, bf16))
    if bf16:  # the pattern itself: 16 with the code in the top mantissa bits
        assert np.array_equal(got, (0x4180 | (codes << 3)).astype(np.uint16))


def test_corrected_block_dot_bf16(probe):
    gu.note("corrected block dot bf16")
    rng = np.random.default_rng(16)
    w = 96
    xv = rng.normal(0, 1, size=(w, 16, 32)) * np.exp(rng.normal(0, 1.5, size=(w, 16, 1)))
    A = enc(xv, True)
    q = rng.integers(0, 16, size=(w, 32, 16)).astype(np.uint32)
    q[:16] = 8  # all-8 blocks
    a4, b4 = to_lanes(A, operand_bits(q, True))
    D, C = probe.q4dot(a4, lane_words(q), True)
    Dm, Cm = from_lanes(D), from_lanes(C)
    # the correction depends on the row only: the MFMA against -24
    # everywhere, and bit for bit the negation of the MFMA against 24
    assert np.array_equal(Cm.view(np.uint32), np.repeat(Cm[:, :, :1], 16, axis=2).view(np.uint32))
    _, bm24 = to_lanes(A, np.full((w, 32, 16), enc(np.array([-24.0]), True)[0], np.uint16))
    assert np.array_equal(C.view(np.uint32), probe.mfma(a4, bm24, True).view(np.uint32))
    _, b24 = to_lanes(A, np.full((w, 32, 16), enc(np.array([24.0]), True)[0], np.uint16))
    assert np.array_equal(C.view(np.uint32), (-probe.mfma(a4, b24, True)).view(np.uint32))
    # the block dot is the MFMA of the dequantized operand with the
    # correction as accumulator input
    assert np.array_equal(D.view(np.uint32), probe.mfma_acc(a4, b4, C, True).view(np.uint32))
    # against the exact sum: the block dot sums 32 exact products (operands
    # at most 31) and C, the correction 32 exact products (24), each within
    # 33 u of its sum of magnitudes, |C| at most 24 (1 + 33 u) sum|x|
    xd = dec(A, True)
    s = Dm.astype(np.float64)
    exact = np.einsum("wmk,wkn->wmn", xd, q.astype(np.float64) - 8.0)
    u = 2.0 ** -24
    bound = 33 * u * (31.0 + 24.0 * (2.0 + 33 * u)) * np.abs(xd).sum(axis=2)[:, :, None]
    assert np.all(np.abs(s - exact) <= bound)
    # a block of all-8 codes: the exact value is 0, the result within the bound
    assert np.all(np.abs(s[:16]) <= bound[:16])


def test_exact_operand_block_dot_f16(probe):
    gu.note("exact-operand block dot fp16")
    rng = np.random.default_rng(17)
    w = 128
    # wide-ranging same-sign and mixed-sign activations
    xv = rng.uniform(1.0, 4000.0, size=(w, 16, 32)) * np.where(rng.random((w, 16, 1)) < 0.5, 1.0, -1.0)
    xv[w // 2:] *= np.where(rng.random((w // 2, 16, 32)) < 0.5, 1.0, -1.0)
    A = enc(xv, False)
    q = rng.integers(0, 16, size=(w, 32, 16)).astype(np.uint32)
    # a quarter of the blocks: codes 8 except one 7 or 9 (one non-zero weight)
    sp = slice(0, w // 4)
    q[sp] = 8
    kk = rng.integers(0, 32, size=(w // 4, 16))
    q[sp][np.arange(w // 4)[:, None], kk, np.arange(16)[None, :]] = rng.choice([7, 9], size=(w // 4, 16))
    a4, b4 = to_lanes(A, operand_bits(q, False))
    D, E = probe.q4dot(a4, lane_words(q), False)
    assert np.array_equal(D.view(np.uint32), probe.mfma(a4, b4, False).view(np.uint32))
    assert np.all(E == 0)  # no correction in fp16
    Dm = from_lanes(D).astype(np.float64)
    xd = dec(A, False)
    wq = q.astype(np.float64) - 8.0
    exact = np.einsum("wmk,wkn->wmn", xd, wq)
    mag = np.einsum("wmk,wkn->wmn", np.abs(xd), np.abs(wq))
    # one non-zero weight: the single exact product, exactly
    assert np.array_equal(Dm[sp], exact[sp])
    # otherwise within 33 u of the sum of the products' magnitudes
    assert np.all(np.abs(Dm - exact) <= 33 * 2.0 ** -24 * mag)


def test_fma0_single_rounding(probe):
    gu.note("fma0")
    rng = np.random.default_rng(14)
    n = 1 << 16
    d = np.abs(rng.normal(0, 0.02, n)).astype(np.float16).astype(np.float32)
    d[: n // 8] = (rng.integers(1, 1024, n // 8) * 2.0 ** -24).astype(np.float32)  # fp16 subnormals
    s = (rng.normal(0, 1, n) * 2.0 ** rng.integers(-120, 20, n)).astype(np.float32)
    got = probe.fma0(d, s)
    expect = (d.astype(np.float64) * s.astype(np.float64)).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), expect.view(np.uint32))
