"""Host-only checks of the GEMV kernels' launch plans (tf_gemv_plan): every
plan the launcher can produce stays inside the limits the kernels rely on.

The 16-row-chunk kernel stages each chunk's activations and metadata records
through a fixed number of registers per thread and walks its K range in
chunks of whole ring depths; a plan with an empty chunk, more staged units
than registers, or more LDS than the launcher allows would read or write out
of bounds.  The launcher refuses such plans, and this test shows the planner
never makes one, for every row count from 1 to 64, every group rule, both
bit widths and a spread of layer shapes and compute-unit counts.
"""

import ctypes
import os
import random

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_linear_layers_awq_amd", "libtilefuse.so")

FIELDS = ("kernel", "waves", "bpw", "splits", "split_tiles", "chunk_tiles", "depth", "row_chunks", "lds",
          "lds_limit", "x_capacity", "rec_capacity", "meta_cap", "xpitch")
RECORD_BYTES = {4: 40, 8: 48}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libtilefuse.so is not built (run __graft_entry__.build())")
    from quantized_linear_layers_awq_amd import load_library

    return load_library()


def gemv_plan(lib, bits, M, K, N, G, cus):
    out = (ctypes.c_int64 * 14)()
    st = lib.tf_gemv_plan(bits, M, K, N, G, cus, out)
    assert st == 0, (bits, M, K, N, G, cus, st)
    return dict(zip(FIELDS, (int(v) for v in out)))


def _chunks(K, ktiles, split_tiles, chunk_tiles):
    """(first, end) k-tiles of every staged chunk of every K range."""
    for b in range(0, ktiles, split_tiles):
        e = min(b + split_tiles, ktiles)
        for c0 in range(b, e, chunk_tiles):
            yield c0, min(c0 + chunk_tiles, e)


def _record_words(bits, K, G, c0, c1):
    """8-byte record words of the groups from the chunk's first row to its last."""
    k0, k1 = c0 * 128, min(c1 * 128, K)
    g0, g1 = k0 // G, (k1 - 1) // G
    return (g1 - g0 + 1) * RECORD_BYTES[bits] // 8


def _check(lib, bits, M, K, N, G, cus):
    p = gemv_plan(lib, bits, M, K, N, G, cus)
    ktiles = -(-K // 128)
    where = (bits, M, K, N, G, cus, p)
    assert p["chunk_tiles"] >= 1, where
    assert p["lds"] <= p["lds_limit"], where
    assert p["xpitch"] == p["chunk_tiles"] * 128 + 8, where
    assert (p["splits"] - 1) * p["split_tiles"] < ktiles <= p["splits"] * p["split_tiles"], where
    if p["kernel"] == 1:
        D = p["depth"]
        assert M <= 64 and p["row_chunks"] * 16 >= M, where
        assert p["split_tiles"] >= (2 if p["splits"] > 1 else 1) and p["splits"] <= 16, where
        # whole ring depths per chunk (the last chunk of a range may be short)
        assert p["chunk_tiles"] % D == 0 or p["chunk_tiles"] >= p["split_tiles"], where
        # one staging pass holds a chunk's activations: M rows x 16 units per k-tile
        assert M * p["chunk_tiles"] * 16 <= p["x_capacity"], where
        # LDS: two record buffers of 8 blocks and two activation buffers
        assert p["lds"] == 2 * 8 * p["meta_cap"] + 2 * M * p["xpitch"] * 2, where
        for c0, c1 in _chunks(K, ktiles, p["split_tiles"], p["chunk_tiles"]):
            rw = _record_words(bits, K, G, c0, c1)
            assert 8 * rw <= p["rec_capacity"], (where, c0, c1, rw)
            assert 8 * rw <= p["meta_cap"], (where, c0, c1, rw)
    else:
        assert M <= 16, where
        assert p["splits"] == 1 and p["waves"] % p["bpw"] == 0 and 1 <= p["waves"] <= 16, where
        assert p["bpw"] * p["meta_cap"] + M * p["xpitch"] * 2 <= p["lds"], where
        for c0, c1 in _chunks(K, ktiles, ktiles, p["chunk_tiles"]):
            assert _record_words(bits, K, G, c0, c1) * 8 <= p["meta_cap"], (where, c0, c1)
    return p


def _groups(K):
    gs = [g for g in (32, 64, 128, 256, 512) if K % g == 0 and (128 % g == 0 or g % 128 == 0)]
    return gs + [K]


@pytest.mark.parametrize("bits", [4, 8])
def test_gemv_plans_stay_inside_kernel_limits(lib, bits):
    shapes = [(4096, 4096), (4096, 1024), (4096, 14336), (14336, 4096), (4096, 6144), (4096, 28672),
              (8192, 8192), (8192, 32768), (28672, 8192), (96, 64), (160, 24), (2080, 40), (512, 8208)]
    rng = random.Random(2026 + bits)
    for _ in range(40):
        shapes.append((32 * rng.randint(1, 900), 8 * rng.randint(1, 4000)))
    n = 0
    for K, N in shapes:
        for G in _groups(K):
            for M in range(1, 65):
                for cus in (1, 80, 256, 304, 4096):
                    _check(lib, bits, M, K, N, G, cus)
                    n += 1
    assert n > 10000


def test_chunk_count_never_zero_above_32_rows(lib):
    """The case of the earlier fault: above 32 rows the staged chunk of the
    16-row-chunk kernel is short, and a plan with no k-tile in a chunk made
    its chunk count divide by zero.  Every row count has whole chunks."""
    for bits in (4, 8):
        for M in range(33, 65):
            for K, G in ((4096, 128), (14336, 128), (8192, 8192), (4096, 32), (28672, 128), (2080, 32)):
                p = _check(lib, bits, M, K, 4096, G, 256)
                assert p["kernel"] == 1 and p["chunk_tiles"] >= p["depth"] >= 4


def test_gemv_plan_rejects_bad_input(lib):
    out = (ctypes.c_int64 * 14)()
    assert lib.tf_gemv_plan(4, 0, 4096, 64, 128, 256, out) == 2
    assert lib.tf_gemv_plan(4, 65, 4096, 64, 128, 256, out) == 2
    assert lib.tf_gemv_plan(4, 1, 4096, 64, 128, 0, out) == 2
    assert lib.tf_gemv_plan(4, 1, 4096, 64, 96, 256, out) == 3
    assert lib.tf_gemv_plan(5, 1, 4096, 64, 128, 256, out) == 6
    assert lib.tf_gemv_plan(4, 1, 4096, 64, 128, 256, None) == 1


def test_every_split_plan_fits_the_noalloc_array(lib):
    """tf_gemm_w4a16_noalloc holds its split-K partials in a 64 MiB array:
    on 256 compute units no GEMM plan needs more (the bound is 256 x 256 x 256
    fp32 values: a split runs only while the tiles of at most 256 x 256 fill
    at most half the units)."""
    cap = 64 << 20
    worst = 0
    Ms = list(range(1, 65)) + [65, 96, 128, 129, 160, 200, 256, 300, 384, 512, 768, 1024]
    Ns = [128 * i for i in (1, 2, 4, 8, 16, 32, 48, 64, 128, 256)] + [1000, 5000]
    for M in Ms:
        for N in Ns:
            for K in (128, 1024, 4096, 14336, 28672):
                for G in (32, 128, K):
                    w = lib.tf_workspace_bytes_planned(4, 1, M, K, N, G, 256, 0)
                    worst = max(worst, w)
    assert 0 < worst <= cap
