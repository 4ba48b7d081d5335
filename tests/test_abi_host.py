"""Host-only checks of the C-ABI library: it loads, exports every symbol the
header declares, agrees with the oracle on buffer sizes, and rejects bad
arguments before any HIP call.

The validation cases pass fake device addresses, so they only run where no
GPU is visible: a validation bug there surfaces as TF_ERR_HIP (no device),
never as a launch on a real device.
"""

import ctypes
import glob
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_linear_layers_awq_amd", "libtilefuse.so")

TF_OK, TF_ERR_NULL, TF_ERR_SHAPE, TF_ERR_GROUP, TF_ERR_ALIGN, TF_ERR_BUFFER_TOO_SMALL = 0, 1, 2, 3, 4, 5


def _declared_symbols():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(tf_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libtilefuse.so is not built (run __graft_entry__.build())")
    from quantized_linear_layers_awq_amd import load_library

    return load_library()


def _no_gpu():
    try:
        import torch

        return not torch.cuda.is_available()
    except Exception:
        return True


def test_header_declares_the_boundary():
    names = _declared_symbols()
    for n in ("tf_repack_w4", "tf_repack_w8", "tf_gemv_w4a16", "tf_gemv_w8a16", "tf_gemm_w4a16", "tf_gemm_w8a16"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(LIB)
    missing = [n for n in _declared_symbols() if not hasattr(raw, n)]
    assert not missing, missing


def test_binding_names_match_header(lib):
    import quantized_linear_layers_awq_amd as q

    for n in _declared_symbols():
        assert hasattr(q, n), f"binding lacks {n}"


def test_status_strings(lib):
    assert lib.tf_status_string(0) == b"TF_OK"
    assert lib.tf_status_string(3).startswith(b"TF_ERR_GROUP")
    assert lib.tf_format_version() == 2


@pytest.mark.parametrize("bits,K,N,G", [
    (4, 4096, 4096, 128), (4, 14336, 4096, 128), (4, 28672, 8192, 128), (4, 64, 72, 32),
    (8, 8192, 8192, 8192), (8, 96, 100, 32), (4, 384, 64, 384), (4, 160, 24, 160), (8, 1024, 40, 256),
])
def test_packed_bytes_match_oracle(lib, bits, K, N, G):
    fn = lib.tf_packed_bytes_w4 if bits == 4 else lib.tf_packed_bytes_w8
    assert fn(K, N, G) == oracle.packed_bytes(bits, K, N, G) > 0


@pytest.mark.parametrize("K,N,G", [(100, 64, 100), (64, 12, 32), (64, 64, 48), (0, 64, 32), (64, 0, 32),
                                   (64, 64, 0), (64, 64, 128), (2**31, 64, 32), (384, 64, 96)])
def test_packed_bytes_invalid_shapes_are_zero(lib, K, N, G):
    assert lib.tf_packed_bytes_w4(K, N, G) == 0


ROUTE_AUTO, ROUTE_TILED, ROUTE_GEMV, ROUTE_TILED128 = 0, 1, 2, 3
OP_GEMV, OP_GEMM, OP_GEMV_SILU, OP_GEMM_SILU, OP_GEMV_F16, OP_GEMM_F16 = 0, 1, 2, 3, 4, 5


def test_f16_ops_plan_as_their_bf16_ops(lib):
    """The fp16 calls run the kernels and launch plans of the bf16 calls of
    the same name: every planned workspace size agrees; an op past the last
    is refused (size 0)."""
    n = 0
    for bits in (4, 8):
        for K, N, G in ((4096, 4096, 128), (14336, 4096, 128), (4096, 1024, 32), (8192, 8192, 8192), (4096, 28672, 128)):
            for M in (1, 4, 8, 16, 24, 40, 64, 65, 129, 300, 2048):
                for cus in (80, 256, 4096):
                    for route in (ROUTE_AUTO, ROUTE_TILED, ROUTE_GEMV, ROUTE_TILED128):
                        a = lib.tf_workspace_bytes_planned(bits, OP_GEMM, M, K, N, G, cus, route)
                        assert a == lib.tf_workspace_bytes_planned(bits, OP_GEMM_F16, M, K, N, G, cus, route)
                        if M <= 16:
                            g = lib.tf_workspace_bytes_planned(bits, OP_GEMV, M, K, N, G, cus, route)
                            assert g == lib.tf_workspace_bytes_planned(bits, OP_GEMV_F16, M, K, N, G, cus, route)
                        n += 1
    assert n > 1000
    assert lib.tf_workspace_bytes_planned(4, 6, 8, 4096, 4096, 128, 256, ROUTE_AUTO) == 0
    assert lib.tf_workspace_bytes_planned(4, OP_GEMV_F16, 17, 4096, 4096, 128, 256, ROUTE_AUTO) == 0


@pytest.mark.parametrize("route", [ROUTE_AUTO, ROUTE_TILED])
@pytest.mark.parametrize("M,K,N,G", [(1, 4096, 4096, 128), (8, 14336, 4096, 128), (16, 4096, 1024, 128),
                                     (1, 8192, 8192, 8192), (512, 8192, 8192, 8192), (2048, 4096, 14336, 128),
                                     (64, 4096, 4096, 128), (33, 14336, 4096, 128), (64, 256, 1024, 128)])
def test_workspace_cannot_hold_bf16_weights(lib, route, M, K, N, G):
    # The layer never materialises full-precision weights: its only scratch is
    # fp32 partial outputs of a K split (at most 16 x M x N, and at most one
    # range per two k-tiles), smaller than a bf16 copy of W for every shape.
    for bits in (4, 8):
        for op in (OP_GEMV, OP_GEMM):
            if op == OP_GEMV and M > 16:
                continue
            for cus in (1, 80, 256, 304):  # devices of up to 304 compute units
                ws = lib.tf_workspace_bytes_planned(bits, op, M, K, N, G, cus, route)
                assert ws <= 16 * M * N * 4
                assert ws < K * N * 2


def _plan(lib, M, N, cus, K=4096, G=128, bits=4, route=ROUTE_AUTO):
    out = (ctypes.c_int64 * 8)()
    st = lib.tf_gemm_plan(bits, M, K, N, G, cus, route, out)
    return st, tuple(out)


@pytest.mark.parametrize("route", [ROUTE_AUTO, ROUTE_TILED])
def test_workspace_only_for_split_k(lib, route):
    """A call needs S x M x N fp32 partial sums exactly when its plan splits
    K, whichever kernel it runs; tf_gemv_* below 8 rows never does.  The
    SiLU-product calls need what the plain call of their shape needs."""
    ws = lambda bits, op, M, K, N, G, cus=256: lib.tf_workspace_bytes_planned(bits, op, M, K, N, G, cus, route)
    assert ws(4, OP_GEMV, 1, 4096, 4096, 128) == 0
    assert ws(8, OP_GEMV, 7, 8192, 8192, 8192) == 0
    assert ws(4, OP_GEMV, 17, 4096, 4096, 128) == 0  # beyond the GEMV's M
    # 16 rows, per-channel W8 8192 x 8192: the 16-row-chunk kernel in four K ranges
    st, (_, _, _, splits, _, _, _, _) = _plan(lib, 16, 8192, 256, K=8192, G=8192, bits=8)
    assert ws(8, OP_GEMV, 16, 8192, 8192, 8192) == (16 * 8192 * 4 * splits if splits > 1 else 0)
    assert ws(8, OP_GEMV_SILU, 16, 8192, 8192, 8192) == ws(8, OP_GEMV, 16, 8192, 8192, 8192)
    assert lib.tf_workspace_bytes_planned(5, OP_GEMM, 1, 4096, 4096, 128, 256, route) == 0
    for bits, M, K, N, G in [(8, 512, 8192, 8192, 8192), (4, 1, 4096, 4096, 128), (4, 2048, 4096, 14336, 128),
                             (4, 100, 1024, 200, 64), (4, 64, 384, 64, 128), (4, 48, 4096, 4096, 128),
                             (8, 20, 8192, 1024, 8192), (4, 64, 4096, 28672, 128)]:
        st, (_, _, _, splits, _, _, _, _) = _plan(lib, M, N, 256, K=K, G=G, bits=bits, route=route)
        assert st == TF_OK
        want = splits * M * N * 4 if splits > 1 else 0
        assert ws(bits, OP_GEMM, M, K, N, G) == want
        assert ws(bits, OP_GEMM_SILU, M, K, N, G) == want
    assert _plan(lib, 512, 8192, 256, K=8192, G=8192, bits=8)[1][3] == 2   # W8 M=512: two K ranges
    assert _plan(lib, 2048, 14336, 256)[1][3] == 1                         # prefill: no split
    assert _plan(lib, 2048, 14336, 256, route=ROUTE_TILED128)[1][3] == 1


def test_plan_hooks_keep_no_state(lib):
    """The plan inputs are per call: a query with one route or compute-unit
    count leaves every later query unchanged (no process-wide setting)."""
    before = [_plan(lib, M, 4096, 256) for M in (1, 40, 64, 65, 2048)]
    ws_before = lib.tf_workspace_bytes(4, 1, 40, 4096, 4096, 128)
    for cus, route in ((1, ROUTE_TILED), (4096, ROUTE_GEMV), (7, ROUTE_TILED)):
        _plan(lib, 40, 4096, cus, route=route)
        lib.tf_workspace_bytes_planned(4, OP_GEMM, 40, 4096, 4096, 128, cus, route)
    assert [_plan(lib, M, 4096, 256) for M in (1, 40, 64, 65, 2048)] == before
    assert lib.tf_workspace_bytes(4, 1, 40, 4096, 4096, 128) == ws_before
    assert not hasattr(ctypes.CDLL(LIB), "tf_gemm_set_route")
    assert not hasattr(ctypes.CDLL(LIB), "tf_gemm_set_planning_cus")


def test_gemm_route_by_m(lib):
    """GEMM calls with M <= 64 run the GEMV kernel unless the tiled GEMM is
    forced; larger M always run the tiled GEMM."""
    for M in (1, 16, 17, 40, 64):
        assert _plan(lib, M, 4096, 256)[1][5] == 1
    for M in (65, 256, 2048):
        assert _plan(lib, M, 4096, 256)[1][5] == 0
    assert _plan(lib, 1, 4096, 256, route=ROUTE_TILED)[1][5] == 0
    assert _plan(lib, 64, 4096, 256, route=ROUTE_TILED)[1][5] == 0
    assert _plan(lib, 64, 4096, 256, route=ROUTE_GEMV)[1][5] == 1
    assert _plan(lib, 65, 4096, 256, route=ROUTE_GEMV)[1][5] == 0
    assert _plan(lib, 64, 4096, 256, route=9)[0] == 6  # TF_ERR_UNSUPPORTED


def test_gemv_route_plan_covers_k_once(lib):
    """The GEMV kernels' plan for a GEMM call: no K split below 8 rows.
    The 16-row-chunk kernel (above 16 rows, and from 8 rows unless its
    ranges would be shorter than 6 k-tiles) uses at most 16 ranges of at
    least two k-tiles that cover the k-tiles exactly once, their count
    minimising the launch's rounds of 128-column workgroups over the compute
    units times (the k-tiles per range + 4 for the round's fixed cost), plus
    eight k-tiles' worth for the summing launch when K is split."""
    rng = __import__("random").Random(11)
    cases = [(1, 4096, 256, 4096, 128), (16, 4096, 256, 14336, 128), (17, 4096, 256, 4096, 128),
             (64, 28672, 256, 4096, 128), (64, 4096, 256, 14336, 128), (40, 64, 256, 256, 128),
             (64, 8, 256, 128, 128), (33, 1000, 304, 8192, 8192)]
    for _ in range(300):
        G = rng.choice([32, 64, 128, 256, 512])
        K = G * rng.randint(1, 40) if G >= 128 else 128 * rng.randint(1, 40)
        cases.append((rng.randint(1, 64), 8 * rng.randint(1, 5000), rng.choice([1, 2, 3, 7, 64, 80, 256, 304]),
                      K, rng.choice([G, K])))
    for M, N, cus, K, G in cases:
        st, (mt, wide, narrow, splits, st_tiles, route, rows, cols) = _plan(lib, M, N, cus, K=K, G=G)
        assert st == TF_OK and route == 1 and mt == wide == narrow == rows == cols == 0, (M, N, cus, K, G)
        ktiles = -(-K // 128)
        groups = -(-N // 128)
        assert (splits - 1) * st_tiles < ktiles <= splits * st_tiles
        if M < 8:
            assert splits == 1
            continue
        if splits > 1:
            assert splits <= 16 and st_tiles >= 2

        def cost(s):
            st = -(-ktiles // s)
            return -(-(groups * s) // cus) * (st + 4) + (8 if s > 1 else 0)

        valid = [s for s in range(1, 17) if s == 1 or -(-ktiles // s) >= 2]
        best = min(cost(s) for s in valid)
        if M <= 16 and splits == 1:
            # either the plan needs no split, or its ranges would be short
            # and the call stays on the kernel for up to 16 rows
            opt = [s for s in valid if cost(s) == best]
            assert opt == [1] or -(-ktiles // opt[0]) < 6 or any(s == 1 for s in opt), (M, N, cus, K, G)
            continue
        if M <= 16:
            assert st_tiles >= 6
        assert cost(splits) == best, (M, N, cus, K, G, splits)


@pytest.mark.parametrize("route", [ROUTE_TILED, ROUTE_TILED128])
def test_gemm_plan_covers_every_column_once(lib, route):
    """The launch plan: wide tiles from column 0, then 64-column tiles,
    covering [0, N) with no tile wholly past N; 256-column tiles for groups
    of whole k-tiles above 128 rows (not on the 256 x 128 route), with
    no narrow launch; otherwise 128-column tiles and a narrow launch only when
    the wide tiles miss a whole number of rounds and it fits one round.  A K
    split uses wide tiles only, fits one round, and its ranges of whole
    groups cover the k-tiles exactly once."""
    rng = __import__("random").Random(7)
    cases = [(2048, 14336, 256, 4096, 128), (2048, 4096, 256, 14336, 128), (512, 8192, 256, 8192, 8192),
             (1, 8192, 256, 4096, 128), (4096, 32768, 256, 8192, 128), (1, 64, 256, 256, 128), (300, 24, 256, 512, 64),
             (513, 1048, 256, 4128, 32), (4096, 28672, 304, 8192, 128), (64, 4096, 256, 8192, 512)]
    for _ in range(400):
        G = rng.choice([32, 64, 128, 256, 512])
        K = G * rng.randint(1, 40) if G >= 128 else 128 * rng.randint(1, 40)
        cases.append((rng.randint(1, 9000), 8 * rng.randint(1, 5000), rng.choice([1, 2, 3, 7, 64, 80, 256, 304]),
                      K, rng.choice([G, K])))
    for bits in (4, 8):
        for M, N, cus, K, G in cases:
            st, (mt, wide, narrow, splits, st_tiles, gemv, rows, cols) = _plan(lib, M, N, cus, K=K, G=G, bits=bits,
                                                                             route=route)
            assert st == TF_OK and gemv == 0, (M, N, cus, K, G)
            big = route == ROUTE_TILED and (G % 128 == 0 or G == K) and M > 128
            assert cols == (256 if big else 128), (bits, M, N, cus, K, G)
            n_wide = -(-N // cols)
            tiles = mt * n_wide
            ktiles = -(-K // 128)
            assert rows == (128 if M <= 128 else 256)
            assert mt == -(-M // rows)
            if rows == 128 or big:
                assert narrow == 0  # short tiles and 256-column tiles come in one width
            if splits > 1:
                assert wide == n_wide and narrow == 0
                assert splits * tiles <= cus
                assert (splits - 1) * st_tiles < ktiles <= splits * st_tiles
                unit = G // 128 if G % 128 == 0 and G != K else 1
                assert st_tiles % unit == 0 and st_tiles >= 4
                continue
            assert st_tiles == ktiles
            if narrow == 0:
                assert wide == n_wide
            else:
                assert tiles % cus != 0
                assert wide * 128 < N <= wide * 128 + narrow * 64 < N + 64
                assert mt * narrow <= cus
                assert mt * wide <= (tiles // cus) * cus
    if route == ROUTE_TILED:
        # the headline prefill shapes on 256 x 256 tiles; the narrower one
        # splits K in two to fill the chip
        assert _plan(lib, 2048, 14336, 256)[1] == (8, 56, 0, 1, 32, 0, 256, 256)
        assert _plan(lib, 2048, 4096, 256, K=14336)[1] == (8, 16, 0, 2, 56, 0, 256, 256)
    else:
        # 3 whole rounds of 256 x 128 tiles, one of 256 x 64
        assert _plan(lib, 2048, 14336, 256, route=route)[1] == (8, 96, 32, 1, 32, 0, 256, 128)
        assert _plan(lib, 2048, 4096, 256, K=14336, route=route)[1] == (8, 32, 0, 1, 112, 0, 256, 128)
    # 65..128 rows: one 128-row tile per column tile
    assert _plan(lib, 100, 28672, 256, route=route)[1] == (1, 224, 0, 1, 32, 0, 128, 128)


def test_gemm_plan_rejects_bad_input(lib):
    assert _plan(lib, 0, 64, 256)[0] == TF_ERR_SHAPE
    assert _plan(lib, 64, 0, 256)[0] == TF_ERR_SHAPE
    assert _plan(lib, 64, 64, 0)[0] == TF_ERR_SHAPE
    assert _plan(lib, 64, 64, 256, K=4096, G=96)[0] == TF_ERR_GROUP
    out = (ctypes.c_int64 * 8)()
    assert lib.tf_gemm_plan(4, 64, 4096, 64, 128, 256, 0, None) == TF_ERR_NULL
    assert lib.tf_gemm_plan(5, 64, 4096, 64, 128, 256, 0, out) == 6  # TF_ERR_UNSUPPORTED


FAKE = 0x10000  # a 64 KiB-aligned fake device address; never dereferenced


@pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation cases run only where no GPU is visible")
class TestValidation:
    def _gemv(self, lib, M=1, K=256, N=128, G=128, x=FAKE, packed=FAKE, y=FAKE, nbytes=None, ws=FAKE,
              ws_bytes=1 << 30, fn="tf_gemv_w4a16"):
        if nbytes is None:
            nbytes = 1 << 30
        return getattr(lib, fn)(x, packed, nbytes, y, M, K, N, G, ws, ws_bytes, None)

    def test_shape_errors(self, lib):
        assert self._gemv(lib, K=33) == TF_ERR_SHAPE
        assert self._gemv(lib, N=12) == TF_ERR_SHAPE
        assert self._gemv(lib, M=17) == TF_ERR_SHAPE
        # K at the 32-bit offset limit of the kernels, for both entry points
        assert self._gemv(lib, K=1 << 25, G=1 << 25) == TF_ERR_SHAPE
        assert self._gemv(lib, M=64, K=1 << 25, G=128, fn="tf_gemm_w4a16") == TF_ERR_SHAPE
        assert self._gemv(lib, K=(1 << 25) - 32, G=(1 << 25) - 32, nbytes=10) == TF_ERR_BUFFER_TOO_SMALL
        assert self._gemv(lib, M=-1) == TF_ERR_SHAPE
        assert self._gemv(lib, K=0) == TF_ERR_SHAPE
        assert self._gemv(lib, M=2**30 + 1, fn="tf_gemm_w4a16") == TF_ERR_SHAPE

    @pytest.mark.parametrize("fn", ["tf_gemv_w4a16_f16", "tf_gemv_w8a16_f16", "tf_gemm_w4a16_f16",
                                    "tf_gemm_w8a16_f16"])
    def test_f16_entries_validate_like_bf16(self, lib, fn):
        gemm = "gemm" in fn
        assert self._gemv(lib, K=33, fn=fn) == TF_ERR_SHAPE
        assert self._gemv(lib, M=17 if not gemm else 2**30 + 1, fn=fn) == TF_ERR_SHAPE
        assert self._gemv(lib, G=48, fn=fn) == TF_ERR_GROUP
        assert self._gemv(lib, x=None, fn=fn) == TF_ERR_NULL
        assert self._gemv(lib, y=FAKE + 1, fn=fn) == TF_ERR_ALIGN
        assert self._gemv(lib, nbytes=10, fn=fn) == TF_ERR_BUFFER_TOO_SMALL
        assert self._gemv(lib, M=0, fn=fn) == TF_OK

    def test_group_errors(self, lib):
        assert self._gemv(lib, G=48) == TF_ERR_GROUP
        assert self._gemv(lib, G=512) == TF_ERR_GROUP
        assert self._gemv(lib, G=0) == TF_ERR_GROUP
        assert self._gemv(lib, K=384, G=96) == TF_ERR_GROUP   # neither divides 128 nor a multiple of it

    def test_null_and_alignment(self, lib):
        assert self._gemv(lib, x=None) == TF_ERR_NULL
        assert self._gemv(lib, y=None) == TF_ERR_NULL
        assert self._gemv(lib, packed=None) == TF_ERR_NULL
        assert self._gemv(lib, x=FAKE + 2) == TF_ERR_ALIGN
        assert self._gemv(lib, packed=FAKE + 8) == TF_ERR_ALIGN
        assert self._gemv(lib, y=FAKE + 1) == TF_ERR_ALIGN

    def test_buffer_sizes(self, lib):
        need = lib.tf_packed_bytes_w4(256, 128, 128)
        assert self._gemv(lib, nbytes=need - 1) == TF_ERR_BUFFER_TOO_SMALL
        need8 = lib.tf_packed_bytes_w8(256, 100, 256)
        assert self._gemv(lib, N=100, G=256, nbytes=need8 - 1, fn="tf_gemm_w8a16") == TF_ERR_BUFFER_TOO_SMALL

    def test_empty_problem_is_ok_without_launch(self, lib):
        assert self._gemv(lib, M=0, x=None, y=None, packed=None) == TF_OK
        assert self._gemv(lib, M=0, x=None, y=None, packed=None, fn="tf_gemm_w8a16") == TF_OK

    def _silu(self, lib, M=1, K=256, N=128, G=128, x=FAKE, packed=FAKE, y=FAKE, nbytes=1 << 30, ws=FAKE,
              ws_bytes=1 << 30, fn="tf_gemv_w4a16_silu_mul"):
        return getattr(lib, fn)(x, packed, nbytes, y, M, K, N, G, ws, ws_bytes, None)

    def test_silu_mul_validation(self, lib):
        assert self._silu(lib, N=104) == TF_ERR_SHAPE          # halves of 52 columns: not runs of 8
        assert self._silu(lib, N=100, fn="tf_gemv_w8a16_silu_mul") == TF_ERR_SHAPE
        assert lib.tf_repack_w4_gate_up(FAKE, FAKE, FAKE, 256, 104, 128, FAKE, 1 << 30, None) == TF_ERR_SHAPE
        assert lib.tf_repack_w8_gate_up(FAKE, FAKE, FAKE, 256, 100, 128, FAKE, 1 << 30, None) == TF_ERR_SHAPE
        assert lib.tf_repack_w4_gate_up(FAKE, None, FAKE, 256, 112, 128, FAKE, 10, None) == TF_ERR_BUFFER_TOO_SMALL
        assert self._silu(lib, M=17) == TF_ERR_SHAPE
        assert self._silu(lib, M=-1) == TF_ERR_SHAPE
        assert self._silu(lib, K=1 << 25, G=1 << 25) == TF_ERR_SHAPE
        assert self._silu(lib, G=48) == TF_ERR_GROUP
        assert self._silu(lib, x=None) == TF_ERR_NULL
        assert self._silu(lib, packed=None) == TF_ERR_NULL
        assert self._silu(lib, y=FAKE + 1) == TF_ERR_ALIGN
        assert self._silu(lib, x=FAKE + 8) == TF_ERR_ALIGN
        need = lib.tf_packed_bytes_w4(256, 128, 128)
        assert self._silu(lib, nbytes=need - 1) == TF_ERR_BUFFER_TOO_SMALL
        assert self._silu(lib, M=0, x=None, y=None, packed=None) == TF_OK
        # the prefill entry point: any M, same shape rules
        assert self._silu(lib, M=17, fn="tf_gemm_w4a16_silu_mul", nbytes=10) == TF_ERR_BUFFER_TOO_SMALL
        assert self._silu(lib, M=17) == TF_ERR_SHAPE                      # the GEMV call stops at 16 rows
        assert self._silu(lib, M=2048, N=104, fn="tf_gemm_w4a16_silu_mul") == TF_ERR_SHAPE
        assert self._silu(lib, M=2**30 + 1, fn="tf_gemm_w8a16_silu_mul") == TF_ERR_SHAPE
        # a shape the plain GEMV splits over K: the same workspace rules
        shape = dict(M=16, K=8192, N=8192, G=8192, fn="tf_gemv_w8a16_silu_mul")
        need = lib.tf_workspace_bytes(8, 0, 16, 8192, 8192, 8192)
        assert need > 0
        assert self._silu(lib, ws=None, **shape) == TF_ERR_NULL
        assert self._silu(lib, ws=FAKE + 64, **shape) == TF_ERR_ALIGN
        assert self._silu(lib, ws_bytes=need - 1, **shape) == TF_ERR_BUFFER_TOO_SMALL
        assert self._silu(lib, ws=None, ws_bytes=0, nbytes=10, M=4, K=8192, N=8192, G=8192,
                          fn="tf_gemv_w8a16_silu_mul") == TF_ERR_BUFFER_TOO_SMALL  # no workspace needed below 8 rows

    def test_repack_validation(self, lib):
        f = lib.tf_repack_w4
        assert f(FAKE, FAKE, FAKE, 256, 128, 128, FAKE, 10, None) == TF_ERR_BUFFER_TOO_SMALL
        assert f(None, FAKE, FAKE, 256, 128, 128, FAKE, 1 << 30, None) == TF_ERR_NULL
        assert f(FAKE, FAKE, None, 256, 128, 128, FAKE, 1 << 30, None) == TF_ERR_NULL
        assert f(FAKE, FAKE, FAKE, 256, 128, 128, None, 1 << 30, None) == TF_ERR_NULL
        # no zero-point tensor means symmetric quantization: validated, not rejected
        assert f(FAKE, None, FAKE, 256, 128, 128, FAKE, 10, None) == TF_ERR_BUFFER_TOO_SMALL
        assert lib.tf_repack_w8(FAKE, None, FAKE, 256, 100, 128, FAKE, 10, None) == TF_ERR_BUFFER_TOO_SMALL
        assert f(FAKE, FAKE, FAKE + 1, 256, 128, 128, FAKE, 1 << 30, None) == TF_ERR_ALIGN
        assert f(FAKE, FAKE, FAKE, 256, 128, 96, FAKE, 1 << 30, None) == TF_ERR_GROUP
        assert lib.tf_repack_w8(FAKE, FAKE, FAKE, 256, 3, 33, FAKE, 1 << 30, None) == TF_ERR_GROUP

    def test_probe_validation(self, lib):
        assert lib.tf_probe_stream_read(None, 1024, FAKE, None) == 1          # TF_ERR_NULL
        assert lib.tf_probe_stream_read(FAKE, 1000, FAKE, None) == TF_ERR_SHAPE
        assert lib.tf_probe_stream_read(FAKE, 0, FAKE, None) == TF_ERR_SHAPE
        assert lib.tf_probe_stream_read(FAKE + 8, 1024, FAKE, None) == TF_ERR_ALIGN
        flops = ctypes.c_int64(0)
        assert lib.tf_probe_mfma(0, 10, FAKE, ctypes.byref(flops), None) == TF_ERR_SHAPE
        assert lib.tf_probe_mfma(256, 0, FAKE, ctypes.byref(flops), None) == TF_ERR_SHAPE
        assert lib.tf_probe_mfma(256, 10, None, ctypes.byref(flops), None) == TF_ERR_NULL
        assert lib.tf_probe_mfma(256, 10, FAKE + 2, ctypes.byref(flops), None) == TF_ERR_ALIGN

    def test_block_read_probe_validation(self, lib):
        f = lib.tf_probe_block_read
        big = ctypes.c_size_t(1 << 30)

        def call(bits=4, p=FAKE, nb=big, K=4096, N=4096, G=128, waves=16, depth=2, sink=FAKE):
            return f(bits, ctypes.c_void_p(p), nb, ctypes.c_int64(K), ctypes.c_int64(N), ctypes.c_int64(G), waves,
                     depth, ctypes.c_void_p(sink), None)

        assert call(p=None) == TF_ERR_NULL
        assert call(sink=None) == TF_ERR_NULL
        assert call(bits=5) == 6  # TF_ERR_UNSUPPORTED
        assert call(N=12) == TF_ERR_SHAPE
        assert call(G=96) == TF_ERR_GROUP
        assert call(nb=ctypes.c_size_t(lib.tf_packed_bytes_w4(4096, 4096, 128) - 16)) == TF_ERR_BUFFER_TOO_SMALL
        assert call(waves=0) == TF_ERR_SHAPE
        assert call(waves=17) == TF_ERR_SHAPE
        assert call(K=256, waves=3) == TF_ERR_SHAPE  # more waves than k-tiles
        assert call(depth=3) == TF_ERR_SHAPE
        assert call(depth=16) == TF_ERR_SHAPE
        assert call(K=1 << 25) == TF_ERR_SHAPE
        assert call(p=FAKE + 8) == TF_ERR_ALIGN
        assert call(sink=FAKE + 2) == TF_ERR_ALIGN

    def test_noalloc_validation(self, lib):
        f = lib.tf_gemm_w4a16_noalloc
        call = lambda M=2048, K=4096, N=4096, G=128, x=FAKE, p=FAKE, y=FAKE, nb=1 << 30: f(x, p, nb, y, M, K, N, G, None)
        assert call(K=33) == TF_ERR_SHAPE
        assert call(N=12) == TF_ERR_SHAPE
        assert call(G=48) == TF_ERR_GROUP
        assert call(x=None) == TF_ERR_NULL
        assert call(y=FAKE + 1) == TF_ERR_ALIGN
        assert call(p=FAKE + 8) == TF_ERR_ALIGN
        assert call(nb=10) == TF_ERR_BUFFER_TOO_SMALL
        assert call(M=0, x=None, y=None, p=None) == TF_OK
        assert call(M=-1) == TF_ERR_SHAPE
        # a split plan with bad pointers is refused before the array is looked up
        assert lib.tf_workspace_bytes(4, 1, 48, 14336, 4096, 128) > 0
        assert call(M=48, K=14336, x=FAKE + 2) == TF_ERR_ALIGN

    def test_dequant_validation(self, lib):
        assert lib.tf_dequant_w4_f32(FAKE, 1, FAKE, 256, 128, 128, None) == TF_ERR_BUFFER_TOO_SMALL
        assert lib.tf_dequant_w8_f32(FAKE, 1 << 30, FAKE + 2, 256, 128, 128, None) == TF_ERR_ALIGN
        assert lib.tf_dequant_gemv_w4_f32(None, 1 << 30, FAKE, 256, 128, 128, None) == TF_ERR_NULL
        assert lib.tf_dequant_gemv_w8_f32(FAKE, 1 << 30, FAKE, 256, 128, 96, None) == TF_ERR_GROUP
