"""The CPU oracle against its pins (see ``oracle_pins``): decoders, the
hand-worked example, exact rational brute force, numpy's dense fp64 product,
packing, and closed-form special cases."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def lib():
    return oracle.load_library()


@pytest.mark.parametrize("name", sorted(oracle_pins.ALL_PINS))
def test_oracle_pin(lib, name):
    oracle_pins.ALL_PINS[name](lib)


def test_oracle_rejects_bad_k(lib):
    import numpy as np
    with pytest.raises(ValueError):
        oracle.linear(np.zeros((1, 48), np.uint16), False, np.zeros((1, 24), np.uint8),
                      np.zeros((1, 1), np.uint16), lib=lib)


def test_sampled_matches_full(lib):
    import numpy as np
    rng = np.random.default_rng(7)
    M, N, K = 3, 40, 256
    x = rng.normal(0, 1, size=(M, K)).astype(np.float16).view(np.uint16)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    s = np.abs(rng.normal(0, .02, size=(N, K // 32))).astype(np.float16).view(np.uint16)
    wq = oracle_pins.np_pack(codes)
    y, a = oracle.linear(x, False, wq, s, lib=lib)
    ms = rng.integers(0, M, 50)
    ns = rng.integers(0, N, 50)
    ys, as_ = oracle.linear_sampled(x, False, wq, s, ms, ns, lib=lib)
    assert np.array_equal(ys, y[ms, ns]) and np.array_equal(as_, a[ms, ns])
