"""The pages' kernel-switching schemes and the continuous-batching row mix,
against the oracle; the spec entry points called as they are; and
GPT-2-small-shaped projections.

* Schemes ("Why Continuous Batching Slowed Down My LLM Inference Engine: A
  Metal Kernel Investigation", sections "Two Rows of Input, Two Different
  Kernels" and "Row-by-Row GEMV to the Rescue"): the engine first sent one
  row to the matrix-vector kernel and more rows to the matrix-matrix kernel;
  the fix sent up to 4 rows through the matrix-vector kernel one row at a
  time, each written into its row of y.  Here every scheme, this library's
  rule and all-rows-through-the-matrix-vector-kernel must match the oracle
  and give the same bits.
* Row counts: the pages' request counts 1..5, the continuous-batching
  iterations of "What continuous batching changes: reading three LLM
  inference traces" (section "Continuous batching: refill between
  iterations": 85, 44, 19 and 8 tokens) and the 124-row mixed batch.
* q4_linear / q4_linear_f16 (no workspace), including K = 18944 at 9..16
  rows where the automatic rule keeps the matrix-vector kernel.
* GPT-2 small ("Why LLM Decoding Is Slow, and Why Batching Is (Almost)
  Free", section "The Catch: Every User Brings Their Own Cache": 12 heads of
  64, so d_model = 768): the 768 x 768 projections and the fused
  q|k|v (2304 x 768) at 1..16 rows, both kernels, both activation types.
  K = 768 is 6 quads in 4 segments (1 or 2 quads each).
"""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_matmul_q4_amd as q4
import oracle
import synth
from bit_quantized_matmul_q4_amd import _lib
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SCHEME_MS = (1, 2, 3, 4, 5, 8, 19, 44, 85, 124)
SCHEMES = ("library", "one_row_gemv", "row_by_row_le4", "all_gemv")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    gu.require_gpu()


def run_scheme(name, xd, w, M):
    """One layer's call(s) under a scheme, writing into one y."""
    y = torch.empty((M, w.N), dtype=torch.float32, device=gu.DEV)
    if name == "library":
        q4.linear(xd[:M], w, out=y, kernel="auto")
    elif name == "all_gemv":
        q4.linear(xd[:M], w, out=y, kernel="gemv")
    elif name == "one_row_gemv" or M > 4:
        q4.linear(xd[:M], w, out=y, kernel="gemv" if M == 1 else "gemm")
    else:  # row by row, each into its row slice of y
        for r in range(M):
            q4.linear(xd[r:r + 1], w, out=y[r:r + 1], kernel="gemv")
    torch.cuda.synchronize()
    return y.cpu().numpy()


# 7B k_proj and a long-K slice of down_proj (the long-K rule), in bf16
@pytest.mark.parametrize("N,K", [(512, 3584), (192, 18944)])
def test_schemes_against_oracle(N, K):
    x, codes, s = synth.problem(N, K, max(SCHEME_MS), "bf16", workload=96, matrix=N + K)
    y_ref, a_ref = oracle.linear(x, True, oracle.pack(codes), s)
    xd, w = gu.x_to_dev(x, True), gu.pack_dev(codes, s)
    for M in SCHEME_MS:
        outs = {}
        for name in SCHEMES:
            gu.note("scheme %s M=%d N=%d K=%d" % (name, M, N, K))
            outs[name] = run_scheme(name, xd, w, M)
            err = oracle.max_normalised_error(outs[name], y_ref[:M], a_ref[:M])
            assert err <= gu.TOL, (name, M, err)
        for name in SCHEMES[1:]:
            assert np.array_equal(outs[name].view(np.uint32), outs["library"].view(np.uint32)), (name, M)


@pytest.mark.parametrize("kernel", ["auto", "gemv", "gemm"])
def test_continuous_batching_rows_q_proj(kernel):
    """The continuous-batching row counts on the 7B q_proj shape (3584 x 3584)
    against the oracle, and row by row equal to the one-row call."""
    N = K = 3584
    Ms = (8, 19, 44, 85)
    x, codes, s = synth.problem(N, K, max(Ms), "bf16", workload=97, matrix=0)
    y_ref, a_ref = oracle.linear(x, True, oracle.pack(codes), s)
    xd, w = gu.x_to_dev(x, True), gu.pack_dev(codes, s)
    one = q4.linear(xd[:1], w, kernel="gemv").cpu().numpy().view(np.uint32)
    for M in Ms:
        gu.note("continuous batching M=%d kernel=%s" % (M, kernel))
        y = q4.linear(xd[:M], w, kernel=kernel).cpu().numpy()
        err = oracle.max_normalised_error(y, y_ref[:M], a_ref[:M])
        assert err <= gu.TOL, (M, err)
        assert np.array_equal(y[:1].view(np.uint32), one)


def _call_spec(fn, x, w, y, M, N, K):
    lib = _lib.load()
    st = getattr(lib, fn)(x.data_ptr(), w.codes.data_ptr(), w.scales.data_ptr(), y.data_ptr(), M, N, K,
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    _lib.check(st, fn)
    torch.cuda.synchronize()


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("N,K", [(96, 18944), (300, 3584), (40, 896)])
def test_spec_entry_points(bf16, N, K):
    """q4_linear (bf16) and q4_linear_f16 (fp16), no workspace, at 1..16
    rows and 17 / 40: oracle parity and the same bits as q4_linear_ex with
    each kernel forced (at K = 18944 and 9..16 rows they keep the
    matrix-vector kernel, having no workspace for the split)."""
    fn = "q4_linear" if bf16 else "q4_linear_f16"
    x, codes, s = synth.problem(N, K, 40, "bf16" if bf16 else "f16", workload=98, matrix=N + K)
    y_ref, a_ref = oracle.linear(x, bf16, oracle.pack(codes), s)
    xd, w = gu.x_to_dev(x, bf16), gu.pack_dev(codes, s)
    for M in list(range(1, 17)) + [17, 40]:
        gu.note("%s M=%d N=%d K=%d" % (fn, M, N, K))
        y = torch.empty((M, N), dtype=torch.float32, device=gu.DEV)
        _call_spec(fn, xd[:M], w, y, M, N, K)
        yh = y.cpu().numpy()
        err = oracle.max_normalised_error(yh, y_ref[:M], a_ref[:M])
        assert err <= gu.TOL, (M, err)
        for kernel in ("gemv", "gemm"):
            yk = q4.linear(xd[:M], w, kernel=kernel).cpu().numpy()
            assert np.array_equal(yk.view(np.uint32), yh.view(np.uint32)), (M, kernel)


GPT2 = (("attn_q", 768, 768), ("attn_qkv_fused", 2304, 768), ("attn_out", 768, 768))


@pytest.mark.parametrize("bf16", [True, False])
@pytest.mark.parametrize("name,N,K", GPT2)
def test_gpt2_small_shapes(name, N, K, bf16):
    assert q4.segments(K) == 4
    x, codes, s = synth.problem(N, K, 16, "bf16" if bf16 else "f16", workload=6, matrix=N)
    y_ref, a_ref = oracle.linear(x, bf16, oracle.pack(codes), s)
    xd, w = gu.x_to_dev(x, bf16), gu.pack_dev(codes, s)
    ref_bits = None
    for M in range(1, 17):
        for kernel in ("auto", "gemv", "gemm"):
            gu.note("gpt2 %s M=%d bf16=%s kernel=%s" % (name, M, bf16, kernel))
            y = q4.linear(xd[:M], w, kernel=kernel).cpu().numpy()
            err = oracle.max_normalised_error(y, y_ref[:M], a_ref[:M])
            assert err <= gu.TOL, (M, kernel, err)
            if ref_bits is None:
                ref_bits = q4.linear(xd, w, kernel="gemv").cpu().numpy().view(np.uint32)
            assert np.array_equal(y.view(np.uint32), ref_bits[:M]), (M, kernel)
