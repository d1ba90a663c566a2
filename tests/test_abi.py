"""The C-ABI library on the CPU: it loads, exports every function the
header declares, and its host logic (argument checks, the segment schedule,
workspace sizing, the crossover setting) behaves as documented.  No call here
reaches a kernel launch: every compute call fails its argument checks, which
run before any HIP call."""
import ctypes
import os
import re

import pytest

from bit_quantized_matmul_q4_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q4.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from bit_quantized_matmul_q4_amd import build
        build.build_library()
    return _lib.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(lib, name), "libq4.so does not export %s" % name
    assert sorted(names) == sorted(_lib.EXPORTS)


def test_abi_and_strerror(lib):
    assert lib.q4_abi_version() == 6
    for st in (0, -1, -2, -3, -4, -5, -6, -7):
        assert lib.q4_strerror(st) and lib.q4_strerror(st) != b"unknown status"
    assert lib.q4_strerror(-99) == b"unknown status"
    assert lib.q4_last_hip_error() == 0


def plan(K):
    """The K-segment schedule, restated from its definition: quads of four
    blocks, S = min(16, largest power of two <= number of quads)."""
    nb = K // 32
    G = (nb + 3) // 4
    S = 1
    while S * 2 <= G and S < 16:
        S *= 2
    segs = [(4 * (j * G // S), min(nb, 4 * ((j + 1) * G // S))) for j in range(S)]
    return nb, G, S, segs


@pytest.mark.parametrize("K", [32, 64, 96, 128, 160, 256, 512, 896, 2048, 3584, 4864, 18944, 32 * 997])
def test_segments(lib, K):
    nb, G, S, segs = plan(K)
    assert lib.q4_segments(K) == S
    # segments tile the blocks in order, none empty, all starting on a quad
    assert segs[0][0] == 0 and segs[-1][1] == nb
    for (a, b), (c, _) in zip(segs, segs[1:]):
        assert b == c
    assert all(b > a and a % 4 == 0 for a, b in segs)


def test_segments_bad_k(lib):
    for K in (0, 16, 31, 33, -32):
        assert lib.q4_segments(K) == 0


def test_packed_sizes(lib):
    """Tiles of 16 rows by 4 blocks: 1024 code bytes and 128 scale bytes each."""
    import oracle
    for N, K in ((1, 32), (16, 128), (17, 160), (896, 896), (3584, 18944), (152064, 3584)):
        tiles = -(-N // 16) * -(-(K // 32) // 4)
        assert lib.q4_packed_code_bytes(N, K) == 1024 * tiles
        assert lib.q4_packed_scale_bytes(N, K) == 128 * tiles
        if N * K < 1 << 24:
            assert oracle.tiled_sizes(N, K) == (1024 * tiles, 64 * tiles)
    assert lib.q4_packed_code_bytes(4, 48) == 0
    assert lib.q4_packed_scale_bytes(0, 64) == 0


def test_crossover_get_set(lib):
    old = lib.q4_get_crossover()
    try:
        assert lib.q4_set_crossover(7) == 0
        assert lib.q4_get_crossover() == 7
        assert lib.q4_set_crossover(-1) == _lib.Q4_ERR_SHAPE
        assert lib.q4_get_crossover() == 7
    finally:
        lib.q4_set_crossover(old)


def test_workspace_bytes(lib):
    assert lib.q4_workspace_bytes(8, 3584, 3584, _lib.Q4_GEMV) == 0
    # k_proj at 124 rows: too few column units to fill the GPU, split over K
    ws = lib.q4_workspace_bytes(124, 512, 3584, _lib.Q4_GEMM)
    assert ws > 0 and ws % (124 * 512 * 4) == 0
    gk = ws // (124 * 512 * 4)
    assert gk & (gk - 1) == 0 and 2 <= gk <= 16
    # gate at 124 rows fills it without a split: no workspace
    assert lib.q4_workspace_bytes(124, 18944, 3584, _lib.Q4_GEMM) == 0


def test_auto_rule_long_k(lib):
    """Q4_AUTO keeps the matrix-vector kernel up to T rows, except that for
    K > 8192 the split matrix-matrix kernel takes over above min(T, 8) rows
    (its workspace is what q4_workspace_bytes reports for Q4_AUTO)."""
    old = lib.q4_get_crossover()
    try:
        assert lib.q4_set_crossover(16) == 0
        auto, gemm = _lib.Q4_AUTO, _lib.Q4_GEMM
        assert lib.q4_workspace_bytes(8, 3584, 18944, auto) == 0           # matrix-vector
        assert lib.q4_workspace_bytes(12, 3584, 18944, auto) == lib.q4_workspace_bytes(12, 3584, 18944, gemm) > 0
        assert lib.q4_workspace_bytes(12, 3584, 3584, auto) == 0           # short K: matrix-vector up to T
        assert lib.q4_set_crossover(4) == 0
        assert lib.q4_workspace_bytes(6, 3584, 18944, auto) > 0            # above min(T, 8)
        assert lib.q4_workspace_bytes(4, 3584, 18944, auto) == 0
    finally:
        lib.q4_set_crossover(old)
    assert lib.q4_workspace_bytes(0, 16, 32, _lib.Q4_GEMM) == 0   # bad shape
    assert lib.q4_workspace_bytes(4, 16, 48, _lib.Q4_GEMM) == 0   # bad shape


FAKE = 1 << 20  # an aligned non-null address; never dereferenced (checks fail first)


def call(lib, x=FAKE, dt=_lib.Q4_BF16, w=FAKE, s=FAKE, y=FAKE, M=4, N=16, K=64,
         kern=_lib.Q4_AUTO, ws=None, wsb=0):
    return lib.q4_linear_ex(x, dt, w, s, y, M, N, K, kern, ws, wsb, None)


def test_argument_checks(lib):
    assert call(lib, x=None) == _lib.Q4_ERR_NULL
    assert call(lib, w=None) == _lib.Q4_ERR_NULL
    assert call(lib, s=None) == _lib.Q4_ERR_NULL
    assert call(lib, y=None) == _lib.Q4_ERR_NULL
    assert call(lib, dt=2) == _lib.Q4_ERR_ENUM
    assert call(lib, kern=3) == _lib.Q4_ERR_ENUM
    assert call(lib, kern=-1) == _lib.Q4_ERR_ENUM
    for M, N, K in ((0, 16, 64), (4, 0, 64), (4, 16, 0), (4, 16, 48), (4, 16, 16), (-1, 16, 64),
                    (1 << 30, 1 << 30, 32), (1, 16, (1 << 25) + 32)):
        assert call(lib, M=M, N=N, K=K) == _lib.Q4_ERR_SHAPE, (M, N, K)
    assert call(lib, x=FAKE + 2) == _lib.Q4_ERR_ALIGN
    assert call(lib, w=FAKE + 8) == _lib.Q4_ERR_ALIGN
    assert call(lib, s=FAKE + 1) == _lib.Q4_ERR_ALIGN
    assert call(lib, y=FAKE + 2) == _lib.Q4_ERR_ALIGN
    assert call(lib, ws=None, wsb=64) == _lib.Q4_ERR_WORKSPACE
    assert call(lib, ws=FAKE + 16, wsb=64) == _lib.Q4_ERR_ALIGN
    # the short forms run the same checks
    assert lib.q4_linear(None, FAKE, FAKE, FAKE, 1, 16, 64, None) == _lib.Q4_ERR_NULL
    assert lib.q4_linear_f16(FAKE, FAKE, FAKE, FAKE, 1, 16, 40, None) == _lib.Q4_ERR_SHAPE
    assert lib.q4_pack(None, FAKE, FAKE, FAKE, 4, 64, None) == _lib.Q4_ERR_NULL
    assert lib.q4_pack(FAKE, None, FAKE, FAKE, 4, 64, None) == _lib.Q4_ERR_NULL
    assert lib.q4_pack(FAKE, FAKE, FAKE, FAKE, 4, 40, None) == _lib.Q4_ERR_SHAPE
    assert lib.q4_pack(FAKE, FAKE, FAKE + 4, FAKE, 4, 64, None) == _lib.Q4_ERR_ALIGN
    assert lib.q4_pack(FAKE, FAKE, FAKE, FAKE + 4, 4, 64, None) == _lib.Q4_ERR_ALIGN
    assert lib.q4_pack(FAKE, FAKE + 1, FAKE, FAKE, 4, 64, None) == _lib.Q4_ERR_ALIGN
    assert call(lib, s=FAKE + 4) == _lib.Q4_ERR_ALIGN
    q = lib.q4_quantize
    assert q(None, _lib.Q4_F32, FAKE, FAKE, 4, 64, None) == _lib.Q4_ERR_NULL
    assert q(FAKE, _lib.Q4_F32, None, FAKE, 4, 64, None) == _lib.Q4_ERR_NULL
    assert q(FAKE, _lib.Q4_F32, FAKE, None, 4, 64, None) == _lib.Q4_ERR_NULL
    assert q(FAKE, 3, FAKE, FAKE, 4, 64, None) == _lib.Q4_ERR_ENUM
    assert q(FAKE, _lib.Q4_BF16, FAKE, FAKE, 4, 48, None) == _lib.Q4_ERR_SHAPE
    assert q(FAKE, _lib.Q4_F16, FAKE, FAKE, 0, 64, None) == _lib.Q4_ERR_SHAPE
    assert q(FAKE + 8, _lib.Q4_F32, FAKE, FAKE, 4, 64, None) == _lib.Q4_ERR_ALIGN
    assert q(FAKE, _lib.Q4_F32, FAKE + 8, FAKE, 4, 64, None) == _lib.Q4_ERR_ALIGN
    assert q(FAKE, _lib.Q4_F32, FAKE, FAKE + 1, 4, 64, None) == _lib.Q4_ERR_ALIGN
    assert lib.q4_last_hip_error() == 0


SCRATCH_BYTES = 4 << 20  # Q4_SCRATCH_BYTES


def test_scratch_covers_every_workspace_need(lib):
    """The fixed scratch buffer of q4_linear_noalloc holds the workspace the
    matrix-matrix kernel asks for at every shape of a wide sweep (so the
    entry point's size check never fires for the current kernels)."""
    worst = 0
    for K in (32, 64, 128, 256, 512, 768, 896, 1024, 2048, 3584, 4864, 8192, 8224, 18944, 32768):
        for N in list(range(1, 2100, 37)) + [2304, 3263, 3584, 4096, 4864, 18944, 37888, 152064]:
            for M in list(range(1, 260, 3)) + [512, 1024, 4096]:
                for kernel in (0, 2):
                    worst = max(worst, lib.q4_workspace_bytes(M, N, K, kernel))
    assert 0 < worst <= SCRATCH_BYTES, worst


def test_noalloc_argument_checks(lib):
    """q4_linear_noalloc rejects bad arguments before any HIP call."""
    p = ctypes.c_void_p(4096)
    y = ctypes.c_void_p(4096)
    assert lib.q4_linear_noalloc(None, 1, p, p, y, 1, 16, 32, 0, None) == -1
    assert lib.q4_linear_noalloc(p, 7, p, p, y, 1, 16, 32, 0, None) == -4
    assert lib.q4_linear_noalloc(p, 1, p, p, y, 1, 16, 32, 9, None) == -4
    assert lib.q4_linear_noalloc(p, 1, p, p, y, 0, 16, 32, 0, None) == -2
    assert lib.q4_linear_noalloc(p, 1, p, p, y, 1, 16, 48, 0, None) == -2
    assert lib.q4_linear_noalloc(ctypes.c_void_p(4104), 1, p, p, y, 1, 16, 32, 0, None) == -3


def test_grouped_argument_checks(lib):
    """q4_linear_grouped checks the group and every item before any HIP call."""
    p = ctypes.c_void_p(4096)
    items = (_lib.GroupItem * 9)()
    for i in range(9):
        items[i] = _lib.GroupItem(4096, 4096, 4096, 64)
    assert lib.q4_linear_grouped(p, 1, items, 0, 1, 3584, None, 0, None) == -2
    assert lib.q4_linear_grouped(p, 1, items, 9, 1, 3584, None, 0, None) == -2
    assert lib.q4_linear_grouped(None, 1, items, 2, 1, 3584, None, 0, None) == -1
    assert lib.q4_linear_grouped(p, 5, items, 2, 1, 3584, None, 0, None) == -4
    assert lib.q4_linear_grouped(p, 1, items, 2, 1, 3000, None, 0, None) == -2
    items[1] = _lib.GroupItem(4096, None, 4096, 64)
    assert lib.q4_linear_grouped(p, 1, items, 2, 1, 3584, None, 0, None) == -1
    items[1] = _lib.GroupItem(4096, 4096, 4096, 0)
    assert lib.q4_linear_grouped(p, 1, items, 2, 1, 3584, None, 0, None) == -2
    items[1] = _lib.GroupItem(4104, 4096, 4096, 64)
    assert lib.q4_linear_grouped(p, 1, items, 2, 1, 3584, None, 0, None) == -3
    items[1] = _lib.GroupItem(4096, 4096, 4096, 64)
    assert lib.q4_linear_grouped(p, 1, items, 2, 1, 3584, None, 64, None) == -6
    assert lib.q4_linear_grouped(p, 1, items, 2, 1, 3584, ctypes.c_void_p(4160), 64, None) == -3


def test_pack_nibbles_argument_checks(lib):
    p = ctypes.c_void_p(4096)
    assert lib.q4_pack_nibbles(None, p, p, p, 16, 64, None) == -1
    assert lib.q4_pack_nibbles(p, p, p, p, 16, 48, None) == -2
    assert lib.q4_pack_nibbles(p, p, ctypes.c_void_p(4100), p, 16, 64, None) == -3
