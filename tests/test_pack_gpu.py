"""q4_pack on the GPU against the oracle's packing into the tiled layout:
bit-exact codes and scales, padding included."""
import numpy as np
import pytest
import torch

import bit_quantized_matmul_q4_amd as q4
import oracle
import synth
from tests import gpu_util as gu
from tests import oracle_pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    gu.require_gpu()


SHAPES = [(1, 32), (3, 64), (17, 96), (16, 128), (896, 896), (128, 896), (4864, 896), (896, 4864),
          (512, 3584), (5, 18944), (33, 32 * 37), (40, 32 * 13)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_pack_matches_oracle(N, K):
    gu.note("pack N=%d K=%d" % (N, K))
    codes = synth.codes(N, K, workload=90, matrix=N)
    s = synth.scales(N, K, workload=90, matrix=N)
    w = gu.pack_dev(codes, s)
    torch.cuda.synchronize()
    wq_t, sc_t = oracle.pack_tiled(codes, s)
    assert np.array_equal(w.codes.cpu().numpy(), wq_t)
    assert np.array_equal(w.scales.view(torch.int16).cpu().numpy().view(np.uint16), sc_t)


def test_pack_ignores_high_bits_and_unaligned_source():
    gu.note("pack high bits / unaligned")
    rng = np.random.default_rng(5)
    N, K = 9, 160
    raw = rng.integers(0, 256, size=N * K + 1, dtype=np.uint8)
    s = oracle_pins.random_scale_bits(rng, (N, K // 32))
    dev = gu.u8_to_dev(raw)
    codes_dev = dev[1:].view(N, K)          # 1-byte offset: unaligned source
    w = q4.pack(codes_dev, gu.scales_to_dev(s))
    torch.cuda.synchronize()
    wq_t, sc_t = oracle.pack_tiled(raw[1:].reshape(N, K), s)
    assert np.array_equal(w.codes.cpu().numpy(), wq_t)
    c2, s2 = oracle.unpack_tiled(w.codes.cpu().numpy(), w.scales.view(torch.int16).cpu().numpy(), N, K)
    assert np.array_equal(c2, raw[1:].reshape(N, K) & 0x0F) and np.array_equal(s2, s)
