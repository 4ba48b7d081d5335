"""GEMV and GEMM parity on small and ragged shapes, special cases that fix the
result exactly, determinism and output guard bands."""

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import (bf16_bits, bf16_to_f64, check_linear, gpu_or_skip, linear_fn, repack, run_linear, split_cus,
                         splitk_cus, to_device, within_tolerance)

pytestmark = pytest.mark.gpu

# (bits, M, K, N, G): single and split-K plans, 128-row aligned and not,
# per-group and per-channel, ragged N (partial 64-column block), ragged K.
GEMV_SHAPES = [
    (4, 1, 128, 64, 128), (4, 3, 512, 200, 128), (4, 16, 1024, 136, 64), (4, 5, 4096, 72, 32),
    (4, 2, 384, 64, 384), (4, 1, 96, 64, 96), (4, 8, 4096, 128, 128), (4, 1, 8192, 256, 128),
    (8, 1, 256, 100, 256), (8, 8, 2048, 260, 2048), (8, 4, 512, 64, 64), (8, 12, 4096, 64, 128),
    # wide layers at M >= 2: two or four blocks per workgroup, last workgroup partial
    (4, 4, 512, 8240, 128), (4, 3, 1024, 16400, 64), (8, 8, 1024, 8208, 1024), (4, 2, 384, 16400, 384),
    # M = 16 over K = 4096: 128 KiB of staged activations (dynamic LDS above 64 KiB)
    (4, 16, 4096, 4096, 128),
    # 12..16 rows on the 16-row-chunk kernel: K split into long ranges (one
    # group per tile, per channel, G = 64), a wide layer split in three with
    # a partial last workgroup, a wide layer not split
    (4, 16, 14336, 1024, 128), (8, 14, 14336, 264, 14336), (4, 12, 8192, 4096, 64), (4, 13, 2048, 8200, 128),
    (4, 14, 4096, 28672, 128),
]

GEMM_SHAPES = [
    (4, 1, 256, 64, 128), (4, 33, 512, 200, 128), (4, 130, 1024, 136, 64), (4, 257, 384, 128, 384),
    (4, 64, 96, 64, 32), (4, 300, 2048, 320, 128), (8, 77, 512, 100, 512), (8, 128, 256, 256, 32),
    (8, 200, 1024, 192, 128),
    # K splits: groups of four k-tiles (ranges on group boundaries), one group
    # over all of K (each range a one-group layout), a ragged last k-tile
    (4, 96, 4096, 256, 512), (8, 64, 3072, 128, 3072), (4, 40, 2080, 128, 32), (4, 16, 2048, 136, 64),
    # between the GEMV kernels' 64 rows and one 256-row tile
    (4, 100, 768, 136, 256), (8, 77, 2080, 40, 32), (8, 128, 512, 64, 32),
    # W8 on 256 x 256 tiles: ragged N (rows not 16-byte multiples), per
    # channel with a ragged last k-tile, groups of whole k-tiles
    (8, 300, 1024, 100, 1024), (8, 600, 2080, 1000, 2080), (8, 513, 4096, 520, 256), (8, 600, 896, 1000, 128),
    # 256-row tiles whose plan can run 128- and 64-column tiles in two
    # launches, W4 and W8, every group rule
    (4, 600, 1024, 1000, 128), (8, 520, 1024, 456, 128), (8, 384, 2048, 264, 2048), (4, 300, 256, 264, 32),
    (8, 513, 1024, 392, 32), (4, 700, 512, 1000, 64),
    # K ranges of 32 rows: K = 32 on the tiled route, and a split whose last
    # range is one k-tile of 32 rows
    (4, 300, 32, 64, 32), (4, 100, 2592, 128, 32), (8, 140, 32, 40, 32),
    # 256 x 256 tiles (W4, groups of whole k-tiles, above 128 rows): ragged N
    # (a partial last tile and half a block), ragged M, groups of two and four
    # k-tiles, per channel with a ragged last k-tile, one row tile with K
    # split, one block of columns, K of one k-tile
    (4, 600, 2048, 1000, 128), (4, 260, 1024, 264, 256), (4, 513, 4128, 520, 4128), (4, 200, 8192, 512, 512),
    (4, 129, 1024, 8, 128), (4, 300, 128, 264, 128), (4, 1024, 4096, 2048, 128),
]

# GEMM calls with 17 <= M <= 64 run the GEMV kernel with two or four 16-row
# chunks per wave: every group mode, ragged N (a partial last workgroup of
# eight blocks), K over several staged chunks, a ragged last row chunk.
MID_SHAPES = [
    (4, 17, 512, 200, 128), (4, 32, 4096, 1024, 128), (4, 33, 1024, 136, 64), (4, 64, 2048, 4096, 128),
    (4, 48, 4096, 72, 32), (4, 64, 768, 256, 256), (4, 20, 384, 64, 384), (4, 64, 14336, 512, 128),
    (8, 24, 1024, 100, 1024), (8, 64, 2048, 260, 64), (8, 40, 4096, 520, 128), (8, 63, 512, 64, 32),
]


def _case(bits, M, K, N, G, seed):
    return synth.make_inputs(bits, M, K, N, G, seed=(51, seed, bits, M, K, N, G))


@pytest.mark.parametrize("shape", GEMV_SHAPES)
def test_gemv_within_tolerance(shape):
    torch, q = gpu_or_skip()
    print(f"gemv {shape}", flush=True)
    c = _case(*shape, seed=1)
    ok, ratio, _ = check_linear(c, torch, q, gemm=False)
    assert ok, f"worst error / bound = {ratio:.3f}"


def _plan_cus(q, plan, shape):
    """Compute units to plan the tiled GEMM for: the device's (auto, tiled,
    tiled128), one (one launch of wide tiles, no split), a count that splits
    the columns between 128- and 64-column tiles (with 256 x 128 tiles), or
    one that splits K."""
    if plan in ("auto", "tiled", "tiled128"):
        return 0
    if plan == "wide":
        return 1
    if plan == "split":
        cus = split_cus(q, *shape)
    else:
        cus = splitk_cus(q, *shape, route=q.TF_ROUTE_TILED128 if plan == "splitk128" else q.TF_ROUTE_TILED)
    if cus is None:
        pytest.skip(f"no compute-unit count gives a '{plan}' plan for this grid")
    return cus


PLAN_ROUTE = {"auto": 0, "tiled": 1, "tiled128": 3, "wide": 1, "split": 3, "splitk": 1, "splitk128": 3}


@pytest.mark.parametrize("plan", list(PLAN_ROUTE))
@pytest.mark.parametrize("shape", GEMM_SHAPES)
def test_gemm_within_tolerance(shape, plan):
    """auto: the kernel the call picks (the GEMV kernel for M <= 64); the
    other plans force a tiled GEMM: the route's choice of tile (tiled, wide,
    splitk) or 256 x 128 tiles (tiled128, split, splitk128)."""
    torch, q = gpu_or_skip()
    if plan == "tiled" and shape[1] > 64:
        pytest.skip("above 64 rows the automatic route is the tiled GEMM")
    route = PLAN_ROUTE[plan]
    if plan in ("tiled128", "splitk128") and q.tf_gemm_plan(*shape, 256, q.TF_ROUTE_TILED)[7] != 256:
        pytest.skip("the shape runs 256 x 128 tiles on every tiled route")
    cus = _plan_cus(q, plan, shape)
    print(f"gemm {shape} plan={plan} cus={cus} {q.tf_gemm_plan(*shape, cus or 256, route)}", flush=True)
    c = _case(*shape, seed=2)
    ok, ratio, _ = check_linear(c, torch, q, gemm=True, cus=cus, route=route)
    assert ok, f"worst error / bound = {ratio:.3f}"


def test_split_plans_exist_for_both_widths():
    """The wide + narrow plan is reachable for W4 and W8 shapes of the list
    above (so the 'split' parametrisations are not all skipped)."""
    _, q = gpu_or_skip()
    for bits in (4, 8):
        assert any(split_cus(q, *s) for s in GEMM_SHAPES if s[0] == bits), bits
    # and the 256 x 256 tiles, with and without a K split
    wide256 = [s for s in GEMM_SHAPES if q.tf_gemm_plan(*s, 256, q.TF_ROUTE_TILED)[7] == 256]
    assert any(q.tf_gemm_plan(*s, 256, q.TF_ROUTE_TILED)[3] > 1 for s in wide256)
    assert any(q.tf_gemm_plan(*s, 256, q.TF_ROUTE_TILED)[3] == 1 for s in wide256)


@pytest.mark.parametrize("shape", [(4, 300, 32, 64, 32), (4, 100, 2592, 128, 32), (8, 140, 32, 40, 32),
                                   (4, 257, 64, 128, 64)])
def test_gemm_short_k_ranges_stay_inside_x(shape):
    """K ranges of 32 or 64 rows: the activation loads of a stage that runs
    past K are clamped inside each row.  x sits at the start of a buffer
    whose remainder is NaN, so a load past the last row would reach the
    output (NaN times a zero weight is NaN)."""
    torch, q = gpu_or_skip()
    bits, M, K, N, G = shape
    cus = splitk_cus(q, *shape) if K > 128 else 0
    print(f"short-k {shape} cus={cus} {q.tf_gemm_plan(*shape, cus or 256, q.TF_ROUTE_TILED)}", flush=True)
    c = _case(*shape, seed=8)
    d = to_device(c, torch)
    p = repack(c, d, q)
    big = torch.full((M * K + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    big[:M * K] = d["x"].reshape(-1)
    x = big[:M * K].view(M, K)
    y = run_linear(q, bits, q.TF_OP_GEMM, x, p, K, N, G, cus=cus, route=q.TF_ROUTE_TILED, torch=torch)
    torch.cuda.synchronize()
    yh = bf16_to_f64(y)
    assert not np.isnan(yh).any()
    ok, ratio = within_tolerance(yh, oracle.awq_linear(c))
    assert ok, ratio


@pytest.mark.parametrize("cus", [0, 1, 4096])
@pytest.mark.parametrize("shape", MID_SHAPES)
def test_gemm_mid_m_gemv_kernel(shape, cus):
    """GEMM calls of 17..64 rows through the 16-row-chunk GEMV kernel, planned for the
    device (0), for one compute unit (K never split) and for 4096 (K split
    into as many ranges as the plan allows, fp32 partials summed in order)."""
    torch, q = gpu_or_skip()
    print(f"mid {shape} cus={cus} {q.tf_gemm_plan(*shape, cus or 256)}", flush=True)
    c = _case(*shape, seed=6)
    ok, ratio, _ = check_linear(c, torch, q, gemm=True, cus=cus)
    assert ok, f"worst error / bound = {ratio:.3f}"


@pytest.mark.parametrize("bits,M,K,N,G", [(4, 600, 1024, 1000, 128), (8, 300, 512, 456, 64), (4, 300, 256, 264, 32),
                                          (8, 600, 512, 520, 512)])
def test_gemm_plans_agree_bitwise(bits, M, K, N, G):
    """Every tile width computes each output with the same operations in the
    same order: the single wide launch and the wide + narrow plan (which each
    of these shapes has) give identical bits."""
    torch, q = gpu_or_skip()
    c = _case(bits, M, K, N, G, seed=5)
    d = to_device(c, torch)
    pk = repack(c, d, q)
    split = split_cus(q, bits, M, K, N, G)
    assert split is not None, "the shape must have a wide + narrow plan"
    outs = {}
    for cus in (1, split):
        plan = q.tf_gemm_plan(bits, M, K, N, G, cus, q.TF_ROUTE_TILED128)
        print(f"plans W{bits} M={M} K={K} N={N} G={G} cus={cus} {plan}", flush=True)
        assert plan[3] == 1
        outs[cus] = bf16_bits(run_linear(q, bits, q.TF_OP_GEMM, d["x"], pk, K, N, G, cus=cus,
                                         route=q.TF_ROUTE_TILED128, torch=torch))
    assert q.tf_gemm_plan(bits, M, K, N, G, split, q.TF_ROUTE_TILED128)[2] > 0
    assert np.array_equal(outs[split], outs[1]), "the wide + narrow plan differs from the single wide launch"


def _integer_case(bits, M, K, N, G, seed):
    """s = 1, z = 8 (W4) or 128 (W8), x in {-2..2}: y is an exact integer."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 1 << bits, size=(K, N), dtype=np.uint8)
    zval = 8 if bits == 4 else 128
    zeros = np.full((K // G, N), zval, np.uint8)
    scales = np.full((K // G, N), 0x3F80, np.uint16)
    xi = rng.integers(-2, 3, size=(M, K))
    c = synth.gen.pack_case(bits, codes, zeros, scales, synth.f32_to_bf16_bits(xi.astype(np.float32)), G)
    exact = xi.astype(np.int64) @ (codes.astype(np.int64) - zval)
    return c, exact


# gemm: False tf_gemv_*, "auto" tf_gemm_* as routed, "tiled" tf_gemm_* forced
# onto the tiled GEMM; cus 4096 makes the GEMV kernel split K at M > 16.
@pytest.mark.parametrize("gemm", [False, "auto", "tiled"])
@pytest.mark.parametrize("bits,M,K,N,G", [(4, 1, 1024, 128, 128), (4, 7, 2048, 200, 64), (8, 4, 1024, 72, 1024),
                                          (4, 16, 14336, 64, 128), (8, 3, 512, 64, 32), (4, 40, 2048, 200, 64),
                                          (8, 64, 1024, 72, 1024), (4, 33, 4096, 128, 128),
                                          (4, 300, 2048, 520, 128), (4, 260, 1024, 264, 512),
                                          (8, 300, 2048, 520, 128), (8, 260, 1024, 100, 1024)])
def test_integer_case_is_bit_exact(gemm, bits, M, K, N, G):
    torch, q = gpu_or_skip()
    if not gemm and M > 16:
        pytest.skip("tf_gemv takes M <= 16")
    print(f"integer gemm={gemm} W{bits} M={M} K={K} N={N} G={G}", flush=True)
    c, exact = _integer_case(bits, M, K, N, G, seed=K + N)
    d = to_device(c, torch)
    op = q.TF_OP_GEMM if gemm else q.TF_OP_GEMV
    y = run_linear(q, bits, op, d["x"], repack(c, d, q), K, N, G, cus=4096 if M > 16 else 0,
                   route=q.TF_ROUTE_TILED if gemm == "tiled" else q.TF_ROUTE_AUTO, torch=torch)
    torch.cuda.synchronize()
    # every partial sum is an integer below 2^24, so fp32 holds it exactly and
    # the only rounding is the final one to bf16
    assert np.abs(exact).max() < 2**24
    assert np.array_equal(bf16_bits(y), oracle.f64_to_bf16(exact.astype(np.float64)))


@pytest.mark.parametrize("gemm,M", [(False, 5), ("auto", 5), ("tiled", 5), ("auto", 40), ("tiled", 40), ("auto", 300)])
@pytest.mark.parametrize("bits", [4, 8])
def test_q_equal_zero_point_gives_zero(gemm, M, bits):
    torch, q = gpu_or_skip()
    c0 = _case(bits, M, 1024, 136, 128, seed=3)
    codes = c0.zeros[np.arange(c0.K) // c0.G]
    c = synth.gen.pack_case(bits, codes, c0.zeros, c0.scales, c0.x, c0.G)
    d = to_device(c, torch)
    op = q.TF_OP_GEMM if gemm else q.TF_OP_GEMV
    y = run_linear(q, bits, op, d["x"], repack(c, d, q), c.K, c.N, c.G, cus=4096 if M > 16 else 0,
                   route=q.TF_ROUTE_TILED if gemm == "tiled" else q.TF_ROUTE_AUTO, torch=torch)
    torch.cuda.synchronize()
    assert np.all(bf16_to_f64(y) == 0.0)


@pytest.mark.parametrize("gemm,M", [(False, 1), (False, 8), (True, 64)])
def test_runs_are_bitwise_deterministic(gemm, M):
    torch, q = gpu_or_skip()
    c = _case(4, M, 4096, 1024, 128, seed=4)
    d = to_device(c, torch)
    p = repack(c, d, q)
    fn = linear_fn(q, 4, gemm)
    a = bf16_bits(fn(d["x"], p, c.K, c.N, c.G))
    b = bf16_bits(fn(d["x"], p, c.K, c.N, c.G))
    assert np.array_equal(a, b)


@pytest.mark.parametrize("gemm,M", [(False, 3), (True, 40)])
def test_output_guard_bands_untouched(gemm, M):
    torch, q = gpu_or_skip()
    c = _case(4, M, 2048, 200, 128, seed=5)
    d = to_device(c, torch)
    p = repack(c, d, q)
    pad = 4096
    big = torch.full((M * c.N + 2 * pad,), -7.25, dtype=torch.bfloat16, device="cuda:0")
    y = big[pad:pad + M * c.N].view(M, c.N)
    linear_fn(q, 4, gemm)(d["x"], p, c.K, c.N, c.G, y=y)
    torch.cuda.synchronize()
    host = big.float().cpu().numpy()
    assert np.all(host[:pad] == -7.25) and np.all(host[-pad:] == -7.25)
    ref = oracle.awq_linear(c)
    yh = host[pad:pad + M * c.N].reshape(M, c.N).astype(np.float64)
    rms = np.sqrt(np.mean(ref**2, axis=1, keepdims=True))
    assert np.all(np.abs(yh - ref) <= 1e-2 * np.maximum(np.abs(ref), rms))


def test_empty_batch_is_a_no_op():
    torch, q = gpu_or_skip()
    c = _case(4, 1, 256, 64, 128, seed=6)
    d = to_device(c, torch)
    p = repack(c, d, q)
    x0 = torch.empty((0, c.K), dtype=torch.bfloat16, device="cuda:0")
    for gemm in (False, True):
        y = linear_fn(q, 4, gemm)(x0, p, c.K, c.N, c.G)
        assert tuple(y.shape) == (0, c.N)


def test_errors_raise_before_launch():
    torch, q = gpu_or_skip()
    c = _case(4, 2, 256, 64, 128, seed=7)
    d = to_device(c, torch)
    p = repack(c, d, q)
    with pytest.raises(q.TileFuseError) as e:
        q.tf_gemv_w4a16(d["x"], p[:100], c.K, c.N, c.G)
    assert e.value.name == "TF_ERR_BUFFER_TOO_SMALL"
    with pytest.raises(q.TileFuseError) as e:
        q.tf_gemm_w4a16(d["x"], p, c.K, c.N, 96)
    assert e.value.name == "TF_ERR_GROUP"
    x17 = torch.zeros((17, c.K), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(q.TileFuseError) as e:
        q.tf_gemv_w4a16(x17, p, c.K, c.N, c.G)
    assert e.value.name == "TF_ERR_SHAPE"


@pytest.mark.parametrize("bits,K,N,G", [(4, 4096, 6144, 128), (4, 14336, 4096, 128), (8, 8192, 264, 8192),
                                        (4, 160, 40, 32)])
def test_block_read_probe_runs_on_packed_buffers(bits, K, N, G):
    """The measurement probe that mirrors a GEMV launch's code stream runs on
    exactly-sized packed buffers for every ring depth and the GEMV plan's wave
    count (a probe: it computes nothing to compare; it must launch cleanly,
    leave the packed buffer unchanged and not touch its sink in practice)."""
    torch, q = gpu_or_skip()
    case = synth.make_inputs(bits, 1, K, N, G, seed=(55, bits, K, N))
    d = to_device(case, torch)
    packed = repack(case, d, q)
    before = packed.clone()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    waves = q.tf_gemv_plan(bits, 1, K, N, G, cus)["waves"]
    for w in sorted({1, waves, min(16, -(-K // 128))}):
        for depth in (2, 4, 8):
            q.tf_probe_block_read(bits, packed, K, N, G, w, depth, sink)
    torch.cuda.synchronize()
    assert torch.equal(packed, before)
    assert int(sink.abs().sum()) == 0


def _swing_case(bits, M, K, N, G, seed):
    """A case whose nonzero scales swing across groups by 2^60: 2^30 (1 + u)
    for groups 0, 1, 4, 5, ... and 2^-30 (1 + u) for groups 2, 3, 6, 7, ...,
    so the 256 x 256 tiles' one chain and each of the 256 x 128 tiles' two
    chains (even and odd groups) rescale by about 2^60 at every other step."""
    c = synth.make_inputs(bits, M, K, N, G, seed=(93, seed, bits, M, K, N, G))
    ng = K // G
    rng = np.random.default_rng(seed)
    e = np.where((np.arange(ng) // 2) % 2 == 0, 30.0, -30.0).astype(np.float32)[:, None]
    s = (np.float32(1.0) + rng.random((ng, N), dtype=np.float32)) * np.exp2(e)
    return synth.pack_case(bits, c.codes, c.zeros, synth.f32_to_bf16_bits(s), c.x, G)


# (bits, M, K, N, G, route name): 256 x 256 tiles (one chain), 256 x 128 tiles
# (two chains), a K split on each, groups of two k-tiles, W8, and the GEMV
SWING_CASES = [(4, 300, 1024, 320, 128, "wide"), (4, 300, 1024, 320, 128, "tiled"),
               (4, 300, 1024, 320, 128, "tiled128"),
               (4, 130, 4096, 256, 128, "splitk"), (4, 130, 4096, 256, 128, "splitk128"),
               (4, 257, 2048, 256, 256, "tiled"), (8, 200, 1024, 192, 128, "tiled128"),
               (4, 4, 2048, 256, 128, "gemv")]


@pytest.mark.parametrize("case", SWING_CASES)
def test_scales_swinging_by_2_pow_60_inside_the_fold_domain(case):
    """The GEMM carries each column's running sum divided by the scale of its
    latest group; the header bounds that quotient.  Scales that swing by 2^60
    between groups (normal activations) stay inside the bound and match the
    oracle, which takes every scale as given."""
    torch, q = gpu_or_skip()
    bits, M, K, N, G, plan = case
    c = _swing_case(bits, M, K, N, G, seed=4)
    if plan == "gemv":
        ok, ratio, _ = check_linear(c, torch, q, gemm=False)
    else:
        route = PLAN_ROUTE[plan]
        cus = _plan_cus(q, plan, (bits, M, K, N, G))
        pl = q.tf_gemm_plan(bits, M, K, N, G, cus or 256, route)
        print(f"swing {case} cus={cus} plan={pl}", flush=True)
        if plan.startswith("splitk"):
            assert pl[3] > 1, "the plan splits K"
        ok, ratio, _ = check_linear(c, torch, q, gemm=True, cus=cus, route=route)
    assert ok, f"worst error / bound = {ratio:.3f}"


# Tiled GEMM launches without a K split write their outputs from LDS in
# 16-byte units where y and its rows are 16-byte aligned, else element by
# element from the same units.  (bits, M, K, N, G, column tile): K of four
# k-tiles, so no split; a partial last row tile; a last column tile of one
# 8-column unit (W4) or of a ragged width with rows that are not 16-byte
# multiples (W8, N = 100) on the 256 x 256 tiles, the 64-column tiles
# (G = 32) and the 128-row tiles.
UNSPLIT_TILED = [(4, 300, 512, 264, 128, 256), (4, 300, 512, 272, 128, 256), (8, 300, 512, 100, 512, 256),
                 (8, 300, 512, 100, 32, 128), (8, 100, 512, 100, 512, 128), (4, 100, 512, 264, 128, 128),
                 (4, 100, 512, 272, 128, 128)]


@pytest.mark.parametrize("op", ["plain", "f16", "silu_mul"])
@pytest.mark.parametrize("shape", UNSPLIT_TILED, ids=[str(s) for s in UNSPLIT_TILED])
def test_tiled_gemm_unaligned_y_matches_aligned(shape, op):
    torch, q = gpu_or_skip()
    bits, M, K, N, G, width = shape
    if op == "silu_mul" and N % 16:
        pytest.skip("the SiLU product pairs 16-column blocks (N % 16 == 0)")
    if op != "silu_mul" and bits == 4 and N % 16 == 0:
        pytest.skip("the plain and fp16 calls take the shape with half a block")
    plan = q.tf_gemm_plan(bits, M, K, N, G, torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan[7] == width and plan[3] == 1 and plan[5] == 0, f"not an unsplit tiled launch: {plan}"
    print(f"tiled gemm unaligned y op={op} shape={shape}", flush=True)
    c = synth.make_inputs(bits, M, K, N, G, seed=(81, bits, M, K, N), dtype="f16" if op == "f16" else "bf16")
    d = to_device(c, torch)
    if op == "silu_mul":
        p = (q.tf_repack_w4_gate_up if bits == 4 else q.tf_repack_w8_gate_up)(d["qweight"], d["qzeros"], d["scales"],
                                                                              K, N, G)
        fn = q.tf_gemm_w4a16_silu_mul if bits == 4 else q.tf_gemm_w8a16_silu_mul
        n_out, dt = N // 2, torch.bfloat16
    else:
        p = repack(c, d, q)
        if op == "f16":
            fn, dt = (q.tf_gemm_w4a16_f16 if bits == 4 else q.tf_gemm_w8a16_f16), torch.float16
        else:
            fn, dt = linear_fn(q, bits, True), torch.bfloat16
        n_out = N
    want = fn(d["x"], p, K, N, G)
    pad = 4097  # odd: y starts 2 bytes past a 16-byte boundary
    big = torch.full((M * n_out + 2 * pad,), -7.25, dtype=dt, device="cuda:0")
    y = big[pad:pad + M * n_out].view(M, n_out)
    assert y.data_ptr() % 16 != 0
    fn(d["x"], p, K, N, G, y=y)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), want.view(torch.int16))
    host = big.float().cpu().numpy()
    assert np.all(host[:pad] == -7.25) and np.all(host[-pad:] == -7.25)
    ref = oracle.awq_linear_silu_mul(c) if op == "silu_mul" else oracle.awq_linear(c)
    ok, ratio = within_tolerance(bf16_to_f64(want) if dt == torch.bfloat16 else want.double().cpu().numpy(), ref)
    assert ok, f"worst error / bound = {ratio:.3f}"
