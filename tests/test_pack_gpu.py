"""q4_pack on the GPU against the oracle's packing: bit-exact."""
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


SHAPES = [(1, 32), (3, 64), (17, 96), (896, 896), (128, 896), (4864, 896), (896, 4864),
          (512, 3584), (5, 18944), (33, 32 * 37)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_pack_matches_oracle(N, K):
    gu.note("pack N=%d K=%d" % (N, K))
    codes = synth.codes(N, K, workload=90, matrix=N)
    got = q4.pack(gu.u8_to_dev(codes)).cpu().numpy()
    assert np.array_equal(got, oracle.pack(codes))


def test_pack_ignores_high_bits_and_unaligned_source():
    gu.note("pack high bits / unaligned")
    rng = np.random.default_rng(5)
    N, K = 9, 160
    raw = rng.integers(0, 256, size=N * K + 1, dtype=np.uint8)
    dev = gu.u8_to_dev(raw)
    codes_dev = dev[1:].view(N, K)          # 1-byte offset: unaligned source
    got = q4.pack(codes_dev).cpu().numpy()
    assert np.array_equal(got, oracle.pack(raw[1:].reshape(N, K)))
    assert np.array_equal(oracle.unpack(got, K), raw[1:].reshape(N, K) & 0x0F)
