"""Pins of the CPU oracle to things other than itself.

Each pin takes an oracle library handle (``oracle.load_library()`` or a
separately compiled copy) and raises AssertionError when the oracle
disagrees with what the definition and the mathematics fix:

* decoders   -- every fp16 and bf16 bit pattern against numpy's own decoding;
* hand       -- the hand-worked example in ``golden/hand_example_k64.txt``;
* brute      -- exact rational (Fraction) sums on tiny random problems, with
                an independent decoder (Python's struct);
* dense      -- numpy's fp64 matrix product on a dequantized matrix built
                with numpy's own fp16 decoding and bit operations;
* pack       -- numpy nibble packing, and unpack(pack(c)) == c & 15;
* special    -- closed forms: one-hot input reads out one weight exactly,
                all codes 8 give 0, zero input gives 0, one block with unit
                input gives d * sum(q - 8);
* tiled      -- the tiled layout against numpy's reshape construction, its
                round trip, and tiled products equal to canonical ones.

The definition being pinned ("Why Continuous Batching Slowed Down My LLM
Inference Engine: A Metal Kernel Investigation", section "Two Rows of Input,
Two Different Kernels"): y[m][n] = sum_k x[m][k] (q[n][k] - 8) d[n][k//32].
"""
from __future__ import annotations

import os
import struct
from fractions import Fraction

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict:
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


# ---------------------------------------------------------------- helpers
def np_f16(bits) -> np.ndarray:
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def np_bf16(bits) -> np.ndarray:
    with np.errstate(invalid="ignore"):  # signalling-nan patterns are expected
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def np_pack(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, np.uint8) & 0x0F
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def frac_f16(bits: int) -> Fraction:
    return Fraction(struct.unpack("<e", struct.pack("<H", bits))[0])


def frac_bf16(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", bits << 16))[0])


def random_finite_bits(rng, shape, bf16: bool) -> np.ndarray:
    """Uniform random bit patterns with inf/nan exponents excluded: exercises
    subnormals, signed zeros and the full exponent range."""
    b = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    emask, eall = (0x7F80, 0x7F80) if bf16 else (0x7C00, 0x7C00)
    bad = (b & emask) == eall
    b[bad] &= np.uint16(~0x4000 & 0xFFFF)  # clear the top exponent bit
    return b


def random_scale_bits(rng, shape) -> np.ndarray:
    """fp16 scales: mix of |N(0, .02)| values, subnormals, zero and random
    finite patterns."""
    v = np.abs(rng.normal(0, 0.02, size=shape)).astype(np.float16).view(np.uint16)
    pick = rng.integers(0, 8, size=shape)
    v = np.where(pick == 0, rng.integers(0, 0x400, size=shape), v)  # subnormal / zero
    v = np.where(pick == 1, random_finite_bits(rng, shape, bf16=False), v)
    return v.astype(np.uint16)


# ------------------------------------------------------------------- pins
def pin_decoders(lib) -> None:
    bits = np.arange(1 << 16, dtype=np.uint32)
    f16 = np_f16(bits.astype(np.uint16))
    bf = np_bf16(bits.astype(np.uint16))
    for b in range(1 << 16):
        v = lib.q4o_f16_to_f64(b)
        ref = f16[b]
        assert (np.isnan(v) and np.isnan(ref)) or (v == ref and np.signbit(v) == np.signbit(ref)), \
            "fp16 0x%04x -> %r, numpy %r" % (b, v, ref)
        v = lib.q4o_bf16_to_f64(b)
        ref = bf[b]
        assert (np.isnan(v) and np.isnan(ref)) or (v == ref and np.signbit(v) == np.signbit(ref)), \
            "bf16 0x%04x -> %r, numpy %r" % (b, v, ref)


def hand_example_inputs():
    g = read_golden("hand_example_k64.txt")
    K = int(g["K"][0])
    x0 = np.arange(1, K + 1, dtype=np.float64)
    x1 = np.ones(K)
    codes = np.full((1, K), 8, np.uint8)
    codes[0, :32] = np.arange(32) % 16
    codes[0, 32] = 15
    codes[0, 33] = 0
    scales = np.array([[int(h, 16) for h in g["scales_f16_hex"]]], np.uint16)
    packed = np.array([[int(h, 16) for h in g["packed_hex"]]], np.uint8)
    return g, np.stack([x0, x1]), codes, scales, packed


def pin_hand(lib) -> None:
    g, xv, codes, scales, packed = hand_example_inputs()
    wq = oracle.pack(codes, lib=lib)
    assert np.array_equal(wq, packed), "pack of the hand example: %s" % wq.tobytes().hex()
    assert np.array_equal(oracle.unpack(packed, 64, lib=lib), codes)
    y_exp = np.array([float(v) for v in g["y"]])
    a_exp = np.array([float(v) for v in g["A"]])
    for bf16, enc in ((False, lambda v: v.astype(np.float16).view(np.uint16)),
                      (True, lambda v: (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))):
        y, a = oracle.linear(enc(xv), bf16, packed, scales, lib=lib)
        assert np.array_equal(y[:, 0], y_exp), "hand example y = %s (bf16=%s)" % (y[:, 0], bf16)
        assert np.array_equal(a[:, 0], a_exp), "hand example A = %s (bf16=%s)" % (a[:, 0], bf16)


def exact_linear(x_bits, bf16, codes, s_bits):
    dec = frac_bf16 if bf16 else frac_f16
    M, K = x_bits.shape
    N = codes.shape[0]
    y = [[Fraction(0)] * N for _ in range(M)]
    a = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        xs = [dec(int(b)) for b in x_bits[m]]
        for n in range(N):
            acc = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                t = xs[k] * (int(codes[n, k]) - 8) * frac_f16(int(s_bits[n, k // 32]))
                acc += t
                mag += abs(t)
            y[m][n] = acc
            a[m][n] = mag
    return y, a


def pin_brute(lib, seed: int = 1, cases: int = 12) -> None:
    rng = np.random.default_rng(seed)
    for c in range(cases):
        M = int(rng.integers(1, 4))
        N = int(rng.integers(1, 6))
        K = 32 * int(rng.integers(1, 5))
        bf16 = bool(c % 2)
        if c % 3 == 0:
            x_bits = random_finite_bits(rng, (M, K), bf16)
        else:
            v = rng.normal(0, 1, size=(M, K))
            x_bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) if bf16 \
                else v.astype(np.float16).view(np.uint16)
        codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        s_bits = random_scale_bits(rng, (N, K // 32))
        y_ex, a_ex = exact_linear(x_bits, bf16, codes, s_bits)
        y, a = oracle.linear(x_bits, bf16, np_pack(codes), s_bits, lib=lib)
        tol = Fraction(2 * K, 1 << 53)
        for m in range(M):
            for n in range(N):
                ye, ae = y_ex[m][n], a_ex[m][n]
                if not np.isfinite(y[m, n]) or not np.isfinite(a[m, n]):
                    # fp64 overflow is impossible for finite 16-bit inputs
                    raise AssertionError("non-finite oracle output")
                assert abs(Fraction(y[m, n]) - ye) <= tol * ae, \
                    "case %d (%d,%d): oracle %r exact %r" % (c, m, n, y[m, n], float(ye))
                assert abs(Fraction(a[m, n]) - ae) <= tol * ae, \
                    "case %d (%d,%d): oracle A %r exact %r" % (c, m, n, a[m, n], float(ae))


def pin_dense(lib, seed: int = 2) -> None:
    rng = np.random.default_rng(seed)
    for (M, N, K, bf16) in ((5, 37, 320, False), (3, 64, 1024, True), (1, 7, 32, True), (8, 16, 96, False)):
        v = rng.normal(0, 1, size=(M, K))
        x_bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16) if bf16 \
            else v.astype(np.float16).view(np.uint16)
        codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
        s_bits = np.abs(rng.normal(0, 0.02, size=(N, K // 32))).astype(np.float16).view(np.uint16)
        xs = np_bf16(x_bits) if bf16 else np_f16(x_bits)
        W = (codes.astype(np.float64) - 8.0) * np.repeat(np_f16(s_bits), 32, axis=1)
        y_np = xs @ W.T
        a_np = np.abs(xs) @ np.abs(W).T
        y, a = oracle.linear(x_bits, bf16, np_pack(codes), s_bits, lib=lib)
        assert np.all(np.abs(y - y_np) <= 1e-12 * a_np), "dense pin (M,N,K)=(%d,%d,%d)" % (M, N, K)
        assert np.all(np.abs(a - a_np) <= 1e-12 * a_np), "dense pin A (M,N,K)=(%d,%d,%d)" % (M, N, K)


def pin_pack(lib, seed: int = 3) -> None:
    rng = np.random.default_rng(seed)
    for (N, K) in ((1, 32), (3, 64), (17, 96), (5, 2)):
        codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)  # high bits must be ignored
        wq = oracle.pack(codes, lib=lib)
        assert np.array_equal(wq, np_pack(codes)), "pack (%d,%d)" % (N, K)
        assert np.array_equal(oracle.unpack(wq, K, lib=lib), codes & 0x0F), "unpack (%d,%d)" % (N, K)


def np_pack_tiled(codes: np.ndarray, scales: np.ndarray):
    """The tiled layout built with numpy reshapes: pad to 16 rows and 4-block
    quads, gather each lane's eight codes (k = 32 b + 8 g + r) into one
    little-endian 32-bit word with code r at bit 4 (r // 2) + 16 (r % 2),
    then order the words (tile, quad, g, row, block)."""
    N, K = codes.shape
    nb = K // 32
    n16 = -(-N // 16) * 16
    nb4 = -(-nb // 4) * 4
    Q = nb4 // 4
    c = np.zeros((n16, nb4 * 32), np.uint32)
    c[:N, :K] = np.asarray(codes, np.uint8) & 0x0F
    r = np.arange(8)
    shifts = (4 * (r // 2) + 16 * (r % 2)).astype(np.uint32)
    words = (c.reshape(n16 // 16, 16, Q, 4, 4, 8) << shifts).sum(axis=-1, dtype=np.uint32)  # t, row, q, i, g
    wq = np.ascontiguousarray(words.transpose(0, 2, 4, 1, 3)).astype("<u4").view(np.uint8).reshape(-1)
    s = np.zeros((n16, nb4), np.uint16)
    s[:N, :nb] = scales
    sc = s.reshape(n16 // 16, 16, Q, 4).transpose(0, 2, 1, 3).reshape(-1)
    return wq, sc


def pin_tiled(lib, seed: int = 6) -> None:
    """Tiled layout: numpy's construction of the bytes, a round trip, and the
    product from tiled weights equal (bit for bit) to the canonical one."""
    rng = np.random.default_rng(seed)
    for (M, N, K) in ((2, 1, 32), (3, 17, 96), (1, 16, 128), (4, 40, 320), (2, 33, 32 * 13)):
        codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
        s_bits = random_scale_bits(rng, (N, K // 32))
        wq_t, sc_t = oracle.pack_tiled(codes, s_bits, lib=lib)
        wq_np, sc_np = np_pack_tiled(codes, s_bits)
        assert np.array_equal(wq_t, wq_np), "tiled code bytes (%d, %d)" % (N, K)
        assert np.array_equal(sc_t, sc_np), "tiled scales (%d, %d)" % (N, K)
        c2, s2 = oracle.unpack_tiled(wq_t, sc_t, N, K, lib=lib)
        assert np.array_equal(c2, codes & 0x0F) and np.array_equal(s2, s_bits), "tiled round trip"
        x = rng.normal(0, 1, size=(M, K)).astype(np.float16).view(np.uint16)
        y_c, a_c = oracle.linear(x, False, np_pack(codes), s_bits, lib=lib)
        y_t, a_t = oracle.linear_tiled(x, False, wq_t, sc_t, N, K, lib=lib)
        assert np.array_equal(y_c, y_t) and np.array_equal(a_c, a_t), "tiled product (%d, %d)" % (N, K)
    # the hand-worked example through the tiled layout
    g, xv, codes, scales, packed = hand_example_inputs()
    wq_t, sc_t = oracle.pack_tiled(codes, scales, lib=lib)
    y, _ = oracle.linear_tiled(xv.astype(np.float16).view(np.uint16), False, wq_t, sc_t, 1, 64, lib=lib)
    assert np.array_equal(y[:, 0], np.array([float(v) for v in g["y"]])), "hand example, tiled"


def pin_special(lib, seed: int = 4) -> None:
    rng = np.random.default_rng(seed)
    N, K = 6, 128
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s_bits = random_scale_bits(rng, (N, K // 32))
    d = np_f16(s_bits)
    wq = np_pack(codes)
    # one-hot read-out: x = e_k (one row per k) -> y[k][n] = (q[n][k]-8) d[n][k//32] exactly
    for bf16, one in ((False, 0x3C00), (True, 0x3F80)):
        x_bits = np.zeros((K, K), np.uint16)
        x_bits[np.arange(K), np.arange(K)] = one
        y, a = oracle.linear(x_bits, bf16, wq, s_bits, lib=lib)
        expect = ((codes.astype(np.float64) - 8.0) * np.repeat(d, 32, axis=1)).T
        assert np.array_equal(y, expect), "one-hot read-out (bf16=%s)" % bf16
        assert np.array_equal(a, np.abs(expect)), "one-hot normaliser (bf16=%s)" % bf16
    # all codes 8 -> exactly zero output and zero normaliser
    x_bits = rng.normal(0, 1, size=(3, K)).astype(np.float16).view(np.uint16)
    y, a = oracle.linear(x_bits, False, np_pack(np.full((N, K), 8, np.uint8)), s_bits, lib=lib)
    assert np.all(y == 0) and np.all(a == 0), "all codes 8"
    # zero input -> zero output
    y, a = oracle.linear(np.zeros((2, K), np.uint16), True, wq, s_bits, lib=lib)
    assert np.all(y == 0) and np.all(a == 0), "zero input"
    # one block, unit input: y = d * sum(q - 8), an exact small sum
    c1 = codes[:, :32]
    y, _ = oracle.linear(np.full((1, 32), 0x3C00, np.uint16), False, np_pack(c1), s_bits[:, :1], lib=lib)
    expect = d[:, 0] * (c1.astype(np.int64) - 8).sum(axis=1)
    assert np.array_equal(y[0], expect), "single block with unit input"
    # rows are independent: row m of a batch equals the same row computed alone
    x_bits = rng.normal(0, 1, size=(4, K)).astype(np.float16).view(np.uint16)
    y_all, _ = oracle.linear(x_bits, False, wq, s_bits, lib=lib)
    for m in range(4):
        y_one, _ = oracle.linear(x_bits[m:m + 1], False, wq, s_bits, lib=lib)
        assert np.array_equal(y_all[m], y_one[0]), "row %d depends on the batch" % m


# ------------------------------------------------------------ quantizer
def pin_f16_encoder(lib, seed: int = 8) -> None:
    """fp64 -> binary16 (nearest, ties to even) against numpy's conversion,
    on random magnitudes over the whole range, every exact midpoint between
    neighbouring binary16 values of a random sample, and the edges."""
    rng = np.random.default_rng(seed)
    vals = list(rng.uniform(1, 2, 4000) * np.exp2(rng.integers(-30, 17, 4000)) * rng.choice([-1, 1], 4000))
    b = rng.integers(0, 0x7BFF, 3000)
    lo, hi = np_f16(b), np_f16(b + 1)
    vals += list((lo + hi) / 2)                           # exact midpoints: ties
    vals += list(np.nextafter((lo + hi) / 2, np.inf))     # just above a midpoint
    vals += [0.0, -0.0, 2.0 ** -25, 2.0 ** -24, 3 * 2.0 ** -26, 65504.0, 65519.99, 65520.0, 1e6, -1e6]
    for v in vals:
        got = lib.q4o_f64_to_f16(float(v))
        with np.errstate(over="ignore"):  # 65520 and above round to infinity
            ref = int(np.array(v, np.float64).astype(np.float16).view(np.uint16))
        assert got == ref, "f64 %r -> 0x%04x, numpy 0x%04x" % (v, got, ref)


_F16_POS = None


def _f16_nearest(v: Fraction) -> int:
    """Bits of the binary16 value nearest to v >= 0 (ties to the even
    pattern), by search over every finite positive binary16 value."""
    global _F16_POS
    if _F16_POS is None:
        _F16_POS = [frac_f16(b) for b in range(0x7C00)]
    import bisect
    i = bisect.bisect_left(_F16_POS, v)
    if i == len(_F16_POS):
        return 0x7C00
    if _F16_POS[i] == v or i == 0:
        return i
    below, above = _F16_POS[i - 1], _F16_POS[i]
    if v - below < above - v:
        return i - 1
    if above - v < v - below:
        return i
    return i if i % 2 == 0 else i - 1


def exact_quantize(w_vals):
    """The block rule in exact rational arithmetic: w_vals [N][K] Fractions."""
    N, K = len(w_vals), len(w_vals[0])
    codes = np.zeros((N, K), np.uint8)
    scales = np.zeros((N, K // 32), np.uint16)
    for n in range(N):
        for b in range(K // 32):
            blk = w_vals[n][32 * b:32 * b + 32]
            dbits = _f16_nearest(max(abs(v) for v in blk) / 7)
            scales[n, b] = dbits
            d = frac_f16(dbits)
            for k, v in enumerate(blk):
                q = 8 if d == 0 else min(7, max(-8, round(v / d))) + 8  # round(): half to even
                codes[n, 32 * b + k] = q
    return codes, scales


def pin_quantize(lib, seed: int = 9) -> None:
    rng = np.random.default_rng(seed)
    # exact rational brute force, each input kind, with tie-rich blocks
    for kind in ("f32", "bf16", "f16"):
        N, K = 3, 96
        v = rng.normal(0, 0.02, size=(N, K))
        v[1, :32] = np.round(rng.normal(0, 3, 32)) / 2 * 0.25   # multiples of d/2 when absmax hits 7 d
        v[1, 0] = 7 * 0.25
        v[2, 32:64] = 0.0                                       # zero block
        v[2, 64:96] *= 1e-9                                     # d rounds to zero / subnormal
        if kind == "f32":
            w = v.astype(np.float32)
            fr = [[Fraction(float(t)) for t in row] for row in w]
        elif kind == "f16":
            w = v.astype(np.float16).view(np.uint16)
            fr = [[frac_f16(int(t)) for t in row] for row in w]
        else:
            w = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
            fr = [[frac_bf16(int(t)) for t in row] for row in w]
        codes, scales = oracle.quantize(w, kind, lib=lib)
        ec, es = exact_quantize(fr)
        assert np.array_equal(scales, es), "quantize scales (%s)" % kind
        assert np.array_equal(codes, ec), "quantize codes (%s)" % kind
    # closed form: w = k d0, k in -7..7 with both ends present -> codes k + 8, d = d0
    k = np.tile(np.arange(-7, 8), 3)[:32].astype(np.float64)
    k[0], k[1] = 7, -7
    codes, scales = oracle.quantize((k * 2.0 ** -5)[None, :].astype(np.float32), "f32", lib=lib)
    assert np.array_equal(codes[0], (k + 8).astype(np.uint8)) and scales[0, 0] == 0x2800, "grid block"
    # ties go to the even integer: d = 1 (absmax 7), w = +-0.5, +-1.5, 2.5, 3.5
    w = np.zeros(32, np.float32)
    w[:8] = [7, 0.5, -0.5, 1.5, -1.5, 2.5, 3.5, -3.5]
    codes, scales = oracle.quantize(w[None, :], "f32", lib=lib)
    assert scales[0, 0] == 0x3C00 and list(codes[0, :8]) == [15, 8, 8, 10, 6, 10, 12, 4], "half-even ties"
    # a scale tie: absmax / 7 exactly midway between two binary16 values
    mid = (1 + 2.0 ** -10 / 2)  # between 1 and 1 + 2^-10: ties to 1 (even pattern 0x3C00)
    w = np.zeros(32, np.float32)
    w[0] = 7 * mid
    _, scales = oracle.quantize(w[None, :], "f32", lib=lib)
    assert scales[0, 0] == 0x3C00, "scale tie"
    w[0] = 7 * (1 + 3 * 2.0 ** -11)  # between 0x3C01 and 0x3C02: ties to 0x3C02
    _, scales = oracle.quantize(w[None, :], "f32", lib=lib)
    assert scales[0, 0] == 0x3C02, "scale tie (odd below)"
    # a subnormal scale rounds coarsely: absmax / 7 = 3.4 x 2^-24 gives
    # d = 3 x 2^-24, so +-absmax / d = +-7.93 round to +-8 and the clamp
    # keeps +8 at 7 (code 15) and -8 as it is (code 0)
    w = np.zeros(32, np.float32)
    w[0], w[1] = 7 * 3.4 * 2.0 ** -24, -7 * 3.4 * 2.0 ** -24
    codes, scales = oracle.quantize(w[None, :], "f32", lib=lib)
    assert scales[0, 0] == 3 and codes[0, 0] == 15 and codes[0, 1] == 0, "clamp with a subnormal scale"
    # invariants on random data: codes within 1..15 (the largest magnitude
    # maps to 7 d for normal scales), and dequant(quantize(w)) within d/2 of w
    w = rng.normal(0, 0.02, size=(8, 256)).astype(np.float32)
    codes, scales = oracle.quantize(w, "f32", lib=lib)
    d = np.repeat(np_f16(scales), 32, axis=1)
    assert codes.min() >= 1 and codes.max() <= 15, "code range"
    assert np.all(np.abs((codes.astype(np.float64) - 8) * d - w) <= d / 2), "round-trip error"
    # idempotent on its own output: quantizing the dequantized weights gives them back
    back = ((codes.astype(np.float64) - 8) * d).astype(np.float32)
    c2, s2 = oracle.quantize(back, "f32", lib=lib)
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales), "idempotence"


ALL_PINS = {
    "decoders": pin_decoders,
    "hand": pin_hand,
    "brute": pin_brute,
    "dense": pin_dense,
    "pack": pin_pack,
    "special": pin_special,
    "tiled": pin_tiled,
    "f16_encoder": pin_f16_encoder,
    "quantize": pin_quantize,
}
