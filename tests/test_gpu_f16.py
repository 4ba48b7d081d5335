"""fp16 checkpoints through the *_f16 entry points: x, scales and y in IEEE
fp16 (the 16-bit format of many AWQ checkpoints).  Parity with the oracle on
every kernel and launch plan the bf16 calls use (GEMV kernels, the
16-row-chunk kernel, 256 x 256 and 256 x 128 GEMM tiles, wide + narrow
column tiles, split K), and special cases that fix the result exactly:
q == z gives 0, the unit-scale integer GEMM, and overflow to infinity."""

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import (bf16_to_f64, check_linear, gpu_or_skip, repack, run_linear, sample_indices, split_cus,
                         splitk_cus, to_device)

pytestmark = pytest.mark.gpu


def _case(bits, M, K, N, G, seed):
    return synth.make_inputs(bits, M, K, N, G, seed=(61, seed, bits, M, K, N, G), dtype="f16")


# the GEMV kernel (up to 16 rows; several blocks per workgroup on wide
# layers) and the 16-row-chunk kernel with K split (12..16 rows, narrow)
GEMV_SHAPES = [
    (4, 1, 128, 64, 128), (4, 3, 512, 200, 128), (4, 16, 1024, 136, 64), (4, 5, 4096, 72, 32),
    (4, 2, 384, 64, 384), (4, 1, 4096, 4096, 128), (8, 1, 256, 100, 256), (8, 8, 2048, 260, 2048),
    (8, 4, 512, 64, 64), (4, 4, 512, 8240, 128), (4, 16, 14336, 1024, 128), (8, 14, 14336, 264, 14336),
]

# GEMM calls of 17..64 rows: the 16-row-chunk GEMV kernel
MID_SHAPES = [
    (4, 17, 512, 200, 128), (4, 64, 2048, 4096, 128), (4, 48, 4096, 72, 32), (4, 64, 14336, 512, 128),
    (8, 40, 4096, 520, 128), (8, 63, 512, 64, 32),
]

# tiled GEMM: 256 x 256 tiles (W4, groups of whole k-tiles, above 128 rows)
# with ragged M and N, per channel, one block of columns; 256 x 128 tiles
# (W8, G = 32, and forced by route); 128-row tiles; K splits
GEMM_SHAPES = [
    (4, 300, 2048, 320, 128), (4, 600, 2048, 1000, 128), (4, 513, 4128, 520, 4128), (4, 200, 8192, 512, 512),
    (4, 129, 1024, 8, 128), (4, 1024, 4096, 2048, 128), (4, 300, 256, 264, 32), (4, 700, 512, 1000, 64),
    (8, 200, 1024, 192, 128), (8, 520, 1024, 456, 128), (4, 96, 4096, 256, 512), (8, 64, 3072, 128, 3072),
    (4, 100, 768, 136, 256),
]

PLAN_ROUTE = {"auto": 0, "tiled128": 3, "split": 3, "splitk": 1, "splitk128": 3}


def _rows(M):
    """Every row up to 600; above, the first and last row of every 256-row
    tile and a seeded sample."""
    if M <= 600:
        return None
    edges = sorted({r for t in range(0, M, 256) for r in (t, min(t + 255, M - 1))})
    return np.unique(np.concatenate([edges, sample_indices(M, 64, seed=M)]))


@pytest.mark.parametrize("shape", GEMV_SHAPES)
def test_gemv_f16_within_tolerance(shape):
    torch, q = gpu_or_skip()
    print(f"gemv f16 {shape}", flush=True)
    ok, ratio, y = check_linear(_case(*shape, seed=1), torch, q, gemm=False)
    assert y.dtype == torch.float16
    assert ok, f"worst error / bound = {ratio:.3f}"


@pytest.mark.parametrize("shape", MID_SHAPES)
def test_gemm_f16_on_the_gemv_kernels(shape):
    torch, q = gpu_or_skip()
    print(f"gemm f16 (gemv kernels) {shape} {q.tf_gemm_plan(*shape, 256)}", flush=True)
    ok, ratio, _ = check_linear(_case(*shape, seed=2), torch, q, gemm=True)
    assert ok, f"worst error / bound = {ratio:.3f}"


@pytest.mark.parametrize("plan", list(PLAN_ROUTE))
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm_f16_within_tolerance(shape, plan):
    torch, q = gpu_or_skip()
    route = PLAN_ROUTE[plan]
    if plan in ("tiled128", "splitk128") and q.tf_gemm_plan(*shape, 256, q.TF_ROUTE_TILED)[7] != 256:
        pytest.skip("the shape runs 256 x 128 tiles on every tiled route")
    cus = 0
    if plan == "split":
        cus = split_cus(q, *shape)
    elif plan.startswith("splitk"):
        cus = splitk_cus(q, *shape, route=route)
    if cus is None:
        pytest.skip(f"no compute-unit count gives a '{plan}' plan for this grid")
    print(f"gemm f16 {shape} plan={plan} cus={cus} {q.tf_gemm_plan(*shape, cus or 256, route)}", flush=True)
    ok, ratio, _ = check_linear(_case(*shape, seed=3), torch, q, gemm=True, rows=_rows(shape[1]), cus=cus,
                                route=route)
    assert ok, f"worst error / bound = {ratio:.3f}"


def _run(case, torch, q, gemm, cus=0, route=0):
    d = to_device(case, torch)
    packed = repack(case, d, q)
    op = q.TF_OP_GEMM_F16 if gemm else q.TF_OP_GEMV_F16
    y = run_linear(q, case.bits, op, d["x"], packed, case.K, case.N, case.G, cus=cus, route=route, torch=torch)
    torch.cuda.synchronize()
    return y


# (bits, gemm, M, K, N, G, route): the GEMV kernel, the 16-row-chunk kernel,
# 256 x 256 tiles, 256 x 128 tiles
EXACT_CASES = [
    (4, False, 3, 1024, 136, 128, 0), (8, False, 2, 512, 64, 512, 0), (4, True, 40, 2048, 264, 128, 0),
    (4, True, 300, 1024, 264, 128, 0), (8, True, 300, 1024, 200, 128, 0), (4, True, 260, 512, 136, 32, 3),
]


@pytest.mark.parametrize("case", EXACT_CASES)
def test_f16_q_equals_z_gives_exact_zero(case):
    torch, q = gpu_or_skip()
    bits, gemm, M, K, N, G, route = case
    c = _case(bits, M, K, N, G, seed=4)
    codes = c.zeros[np.arange(K) // G]
    cz = synth.gen.pack_case(bits, codes, c.zeros, c.scales, c.x, G, dtype="f16")
    y = bf16_to_f64(_run(cz, torch, q, gemm, route=route))
    assert np.all(y == 0.0)


@pytest.mark.parametrize("case", EXACT_CASES)
@pytest.mark.parametrize("scale", [1.0, 64.0])
def test_f16_integer_gemm_exact_and_overflow(case, scale):
    """Power-of-two scale and small integer x: every sum is an integer below
    2^24, exact in fp32, so the kernel's one rounding to fp16 must give the
    bits of the oracle's one rounding of the exact product.  Scale 1: zero
    point 8 / 128, x in {-1, 0, 1}.  Scale 64: zero point 0 and x mostly 1
    on 512 rows of k; the first half of the columns (codes over the full
    range) reaches sums of 1024 and more, i.e. 65536 and more after the
    scale, and rounds to infinity; the second half (codes 0 or 1) stays
    finite."""
    torch, q = gpu_or_skip()
    bits, gemm, M, K, N, G, route = case
    rng = np.random.default_rng(62 + bits + M)
    codes = rng.integers(0, 1 << bits, size=(K, N), dtype=np.uint8)
    xi = np.zeros((M, K), dtype=np.int64)
    if scale == 1.0:
        zval = 8 if bits == 4 else 128
        xi[:, :64] = rng.integers(-1, 2, size=(M, 64))
    else:
        zval = 0
        codes[:, N // 2:] = rng.integers(0, 2, size=(K, N - N // 2))
        xi[:, :512] = np.where(rng.random((M, 512)) < 0.9, 1, 0)
    zeros = np.full((K // G, N), zval, dtype=np.uint8)
    scales = np.full((K // G, N), np.float16(scale).view(np.uint16), dtype=np.uint16)
    c = synth.gen.pack_case(bits, codes, zeros, scales, xi.astype(np.float16).view(np.uint16), G, dtype="f16")
    exact = (xi @ (codes.astype(np.int64) - zval)).astype(np.float64) * scale
    if scale != 1.0:
        assert np.all(np.abs(exact[:, : N // 2]) >= 65520) and np.all(np.abs(exact[:, N // 2:]) < 65504)
    want = oracle.f64_to_f16(exact)
    assert np.array_equal(oracle.f64_to_f16(oracle.awq_linear(c)), want)
    y = _run(c, torch, q, gemm, route=route)
    got = y.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want), f"{int(np.sum(got != want))} of {want.size} differ"
