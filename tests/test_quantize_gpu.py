"""The HIP quantizer (q4_quantize) against the fp64 oracle, bit for bit.

The rule (the pages leave it open): per block of 32 weights of a row,
d = absmax / 7 rounded once to binary16 (nearest, ties to even) and
q = clamp(round_half_even(w / d), -8, 7) + 8 on the exact quotient; a block
whose d rounds to zero gets d = 0 and codes 8.  Codes and scales are integer
decisions, so the bar is bit-exact, on inputs built to sit on and next to
every rounding boundary."""
import numpy as np
import pytest
import torch

import bit_quantized_matmul_q4_amd as q4
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    gu.require_gpu()


def tricky_f32(rng, N, K):
    """N(0, 0.02) weights with rows of boundary cases: codes on exact
    half-integers of d and one fp32 ulp either side, absmax / 7 exactly on a
    binary16 midpoint and one ulp either side, zero and underflowing blocks."""
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    nb = K // 32
    for n in range(0, N, 3):
        for b in range(nb):
            blk = w[n, 32 * b:32 * b + 32]
            kind = (n // 3 + b) % 5
            dbits = int(rng.integers(0x0400, 0x5800))  # a normal binary16 scale
            d = float(np.array(dbits, np.uint16).view(np.float16))
            if kind == 0:  # half-integer multiples of d, and their fp32 neighbours
                h = (rng.integers(-7, 7, 32) + 0.5) * d
                blk[:] = np.float32(h)
                blk[1::3] = np.nextafter(blk[1::3], np.float32(np.inf))
                blk[2::3] = np.nextafter(blk[2::3], np.float32(-np.inf))
                blk[0] = np.float32(7 * d)
            elif kind == 1:  # absmax / 7 on a binary16 midpoint (and next to it)
                lo = float(np.array(dbits, np.uint16).view(np.float16))
                hi = float(np.array(dbits + 1, np.uint16).view(np.float16))
                blk[:] *= 0.5 * hi / max(1e-30, float(np.abs(blk).max()))
                blk[0] = np.float32(7 * (lo + hi) / 2)
                if b % 2:
                    blk[0] = np.nextafter(blk[0], np.float32(np.inf) if b % 4 == 1 else np.float32(-np.inf))
            elif kind == 2:
                blk[:] = 0.0
            elif kind == 3:  # scale underflows or is subnormal
                blk[:] *= np.float32(10.0 ** -int(rng.integers(3, 8)))
    return w


KINDS = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def to_bits(w32: np.ndarray, kind: str) -> np.ndarray:
    if kind == "f32":
        return w32
    t = torch.from_numpy(w32).to(KINDS[kind])  # round the fp32 values into the input type
    return t.view(torch.int16).numpy().view(np.uint16)


def run(bits: np.ndarray, kind: str):
    if kind == "f32":
        wd = torch.from_numpy(bits).cuda()
    else:
        wd = torch.from_numpy(bits.view(np.int16)).cuda().view(KINDS[kind])
    codes, scales = q4.quantize(wd)
    return codes.cpu().numpy(), scales.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("kind", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N,K", [(1, 32), (37, 96), (200, 1024)])
def test_quantize_bit_exact(kind, N, K):
    gu.note("quantize %s N=%d K=%d" % (kind, N, K))
    rng = np.random.default_rng(N * 131 + K)
    bits = to_bits(tricky_f32(rng, N, K), kind)
    codes, scales = run(bits, kind)
    ec, es = oracle.quantize(bits, kind)
    assert np.array_equal(scales, es), "scales differ at %s" % (np.argwhere(scales != es)[:5],)
    assert np.array_equal(codes, ec), "codes differ at %s" % (np.argwhere(codes != ec)[:5],)


def test_quantize_full_shape():
    gu.note("quantize 18944x3584 f32")
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, size=(18944, 3584)).astype(np.float32)
    codes, scales = run(w, "f32")
    ec, es = oracle.quantize(w, "f32")
    assert np.array_equal(scales, es) and np.array_equal(codes, ec)


def test_quantize_pack_and_use():
    """quantize_pack gives the oracle's tiled pack of the oracle's codes, and
    the product with it stays within the quantization bound of the dense
    product: |y - x w^T| <= sum_k |x_k| d_k / 2 (plus rounding)."""
    gu.note("quantize_pack and use")
    rng = np.random.default_rng(11)
    N, K, M = 70, 512, 5
    w = rng.normal(0, 0.02, size=(N, K)).astype(np.float32)
    qw = q4.quantize_pack(torch.from_numpy(w).cuda())
    ec, es = oracle.quantize(w, "f32")
    wq_t, sc_t = oracle.pack_tiled(ec, es)
    assert np.array_equal(qw.codes.cpu().numpy(), wq_t)
    assert np.array_equal(qw.scales.view(torch.int16).cpu().numpy().view(np.uint16), sc_t)
    x = torch.from_numpy(rng.normal(0, 1, size=(M, K)).astype(np.float32)).to(torch.bfloat16)
    y = q4.linear(x.cuda(), qw).cpu().numpy().astype(np.float64)
    xd = x.float().numpy().astype(np.float64)
    exact = xd @ w.astype(np.float64).T
    d = np.repeat(gu.f16_bits_to_f64(es), 32, axis=1)  # [N, K]
    bound = np.abs(xd) @ (d / 2).T
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-3) + 1e-6)
