"""q4_linear_noalloc -- the entry point that allocates nothing -- against
q4_linear_ex with a caller-allocated workspace, through the C ABI: the same
bits, on two calls in a row (the second smaller, so it runs on what the
first left in the library's scratch buffer), for shapes whose matrix-matrix
calls split K (and so use the scratch) and one that does not, in both
activation types; each also within the oracle's tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from bit_quantized_matmul_q4_amd import _lib
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    gu.require_gpu()


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def run_ex(xd, w, M, N, K, bf16, kernel):
    lib = _lib.load()
    need = lib.q4_workspace_bytes(M, N, K, kernel)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=gu.DEV)
    y = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
    st = lib.q4_linear_ex(xd.data_ptr(), _lib.Q4_BF16 if bf16 else _lib.Q4_F16, w.codes.data_ptr(),
                          w.scales.data_ptr(), y.data_ptr(), M, N, K, kernel, ws.data_ptr() if need else None,
                          need, _stream())
    _lib.check(st, "q4_linear_ex")
    torch.cuda.synchronize()
    return y.cpu().numpy(), need


def run_noalloc(xd, w, M, N, K, bf16, kernel):
    lib = _lib.load()
    y = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
    st = lib.q4_linear_noalloc(xd.data_ptr(), _lib.Q4_BF16 if bf16 else _lib.Q4_F16, w.codes.data_ptr(),
                               w.scales.data_ptr(), y.data_ptr(), M, N, K, kernel, _stream())
    _lib.check(st, "q4_linear_noalloc")
    torch.cuda.synchronize()
    return y.cpu().numpy()


# (first call, second smaller call): (M, N, K, kernel)
PAIRS = [
    ((40, 512, 3584, _lib.Q4_GEMM), (20, 256, 2048, _lib.Q4_GEMM)),    # both split K
    ((16, 3584, 18944, _lib.Q4_AUTO), (12, 1024, 18944, _lib.Q4_AUTO)),  # long K: auto takes the split GEMM
    ((124, 300, 8224, _lib.Q4_GEMM), (3, 100, 896, _lib.Q4_AUTO)),     # the second runs the GEMV (no scratch)
]


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("pair", range(len(PAIRS)))
def test_noalloc_matches_workspace_call(pair, bf16):
    saw_split = False
    for (M, N, K, kernel) in PAIRS[pair]:
        gu.note("noalloc M=%d N=%d K=%d kernel=%d bf16=%s" % (M, N, K, kernel, bf16))
        x, codes, s = synth.problem(N, K, M, "bf16" if bf16 else "f16", workload=99, matrix=N + K)
        xd, w = gu.x_to_dev(x, bf16), gu.pack_dev(codes, s)
        y_ex, need = run_ex(xd, w, M, N, K, bf16, kernel)
        y_na = run_noalloc(xd, w, M, N, K, bf16, kernel)
        assert np.array_equal(y_na.view(np.uint32), y_ex.view(np.uint32))
        y_ref, a_ref = oracle.linear(x, bf16, oracle.pack(codes), s)
        assert oracle.max_normalised_error(y_na, y_ref, a_ref) <= gu.TOL
        saw_split = saw_split or need > 0
    assert saw_split  # the scratch buffer was used
