"""Fused [gate | up] GEMV with the SiLU product (tf_gemv_*_silu_mul) against
the oracle: y[m][n] = silu(g) * u from the unrounded sums of columns n and
N/2 + n, one rounding to bf16; the gate/up repack bit for bit."""

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bf16_bits, bf16_to_f64, gpu_or_skip, run_linear, sample_indices, to_device, within_tolerance

pytestmark = pytest.mark.gpu

# (bits, M, K, N, G), N the fused width: halves of whole and half blocks
# (N/2 = 56, 40), one, two and four blocks per workgroup with a partial last
# workgroup, ragged K, G = 32 / 64 / 128 / per channel, up to 16 rows
SHAPES = [
    (4, 1, 512, 320, 128), (4, 3, 352, 64, 32), (4, 8, 1024, 4096, 64), (4, 16, 4096, 4096, 128),
    (4, 2, 256, 16384, 128), (4, 5, 128, 32784, 128), (4, 1, 384, 112, 384), (4, 4, 512, 8208, 128),
    (8, 1, 256, 80, 256), (8, 4, 2048, 8192, 128), (8, 12, 1024, 16400, 1024), (8, 16, 512, 64, 32),
]


def _fn(q, bits):
    return q.tf_gemv_w4a16_silu_mul if bits == 4 else q.tf_gemv_w8a16_silu_mul


def repack_gate_up(case, d, q):
    fn = q.tf_repack_w4_gate_up if case.bits == 4 else q.tf_repack_w8_gate_up
    return fn(d["qweight"], d["qzeros"], d["scales"], case.K, case.N, case.G)


def _run(case, torch, q, d=None, p=None, y=None, cus=0):
    """The GEMV SiLU-product call, planned for `cus` compute units (0: the
    device's, through the product entry point)."""
    d = d or to_device(case, torch)
    p = p if p is not None else repack_gate_up(case, d, q)
    out = run_linear(q, case.bits, q.TF_OP_GEMV_SILU_MUL, d["x"], p, case.K, case.N, case.G, cus=cus, y=y,
                     torch=torch)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("shape", SHAPES, ids=[str(s) for s in SHAPES])
def test_silu_mul_within_tolerance(shape):
    torch, q = gpu_or_skip()
    bits, M, K, N, G = shape
    print(f"silu_mul shape={shape}", flush=True)
    c = synth.make_inputs(bits, M, K, N, G, seed=(61, bits, M, K, N))
    y = _run(c, torch, q)
    assert tuple(y.shape) == (M, N // 2)
    ref = oracle.awq_linear_silu_mul(c)
    ok, ratio = within_tolerance(bf16_to_f64(y), ref)
    assert ok, f"worst error / bound = {ratio:.3f}"


# The kernel and K split the plain GEMV of the shape would run, forced by
# the compute units the plan assumes (1: never a split; 256, 4096: long-K
# layers split into 4..16 ranges from 8 rows, partials summed by the SiLU
# sum kernel; wide layers from 2 rows run the 16-row-chunk kernel unsplit).
# (bits, M, K, N, G) -> K ranges at 1 / 256 / 4096 compute units
ROUTE_SHAPES = {
    (4, 8, 14336, 4096, 128): (1, 8, 16), (8, 16, 8192, 8192, 8192): (1, 4, 1),
    (4, 12, 14336, 1024, 64): (1, 16, 16), (8, 8, 8192, 4112, 2048): (1, 7, 1),
    (4, 10, 28672, 528, 32): (1, 16, 16), (4, 16, 4096, 28672, 128): (1, 1, 1),
    (4, 2, 1024, 8192, 128): (1, 1, 1), (4, 5, 2048, 1040, 32): (1, 1, 1),
}


@pytest.mark.parametrize("cus", [1, 256, 4096])
@pytest.mark.parametrize("shape", list(ROUTE_SHAPES), ids=[str(s) for s in ROUTE_SHAPES])
def test_silu_mul_routes(shape, cus):
    torch, q = gpu_or_skip()
    bits, M, K, N, G = shape
    print(f"silu_mul route shape={shape} cus={cus}", flush=True)
    c = synth.make_inputs(bits, M, K, N, G, seed=(69, bits, M, K), keep_codes=False)
    splits = ROUTE_SHAPES[shape][(1, 256, 4096).index(cus)]
    assert q.tf_workspace_bytes_planned(bits, q.TF_OP_GEMV_SILU_MUL, M, K, N, G, cus) == \
        (4 * splits * M * N if splits > 1 else 0)
    assert q.tf_workspace_bytes_planned(bits, q.TF_OP_GEMV, M, K, N, G, cus) == \
        q.tf_workspace_bytes_planned(bits, q.TF_OP_GEMV_SILU_MUL, M, K, N, G, cus)
    y = _run(c, torch, q, cus=cus)
    cols = sample_indices(N // 2, 512, seed=70)
    ok, ratio = within_tolerance(bf16_to_f64(y)[:, cols], oracle.awq_linear_silu_mul(c, cols=cols))
    assert ok, f"worst error / bound = {ratio:.3f}"


@pytest.mark.parametrize("bits,M", [(4, 1), (4, 8), (4, 16), (8, 1)])
def test_silu_mul_decoder_gate_up(bits, M):
    """The decoder layer's gate and up projections (K = 4096, 2 x 14336
    columns), on sampled output columns."""
    torch, q = gpu_or_skip()
    K, N, G = 4096, 28672, 128
    print(f"silu_mul gate_up W{bits} M={M}", flush=True)
    c = synth.make_inputs(bits, M, K, N, G, seed=(62, bits, M), keep_codes=False)
    y = _run(c, torch, q)
    cols = sample_indices(N // 2, 384, seed=63)
    ref = oracle.awq_linear_silu_mul(c, cols=cols)
    ok, ratio = within_tolerance(bf16_to_f64(y)[:, cols], ref)
    assert ok, f"worst error / bound = {ratio:.3f}"


@pytest.mark.parametrize("half", ["gate", "up"])
@pytest.mark.parametrize("bits,M,cus", [(4, 1, 0), (4, 6, 0), (8, 3, 0), (4, 8, 256), (4, 12, 1)])
def test_zero_half_gives_exact_zero(bits, M, cus, half):
    """q == z on the gate half makes g exactly 0 and silu(0) = 0; on the up
    half u is exactly 0.  Either way every output is exactly zero."""
    torch, q = gpu_or_skip()
    # a long-K layer where the plan splits K: partials summed by the SiLU sum kernel
    K, N, G = (14336, 1024, 128) if cus == 256 else (1024, 2 * 1056, 128)
    c0 = synth.make_inputs(bits, M, K, N, G, seed=(64, bits, M))
    codes = c0.codes.copy()
    cols = slice(0, N // 2) if half == "gate" else slice(N // 2, N)
    codes[:, cols] = c0.zeros[np.arange(K) // G][:, cols]
    c = synth.gen.pack_case(bits, codes, c0.zeros, c0.scales, c0.x, G)
    assert (q.tf_workspace_bytes_planned(bits, q.TF_OP_GEMV, M, K, N, G, cus or 256) > 0) == (cus == 256)
    y = _run(c, torch, q, cus=cus)
    assert np.all(bf16_to_f64(y) == 0.0)


def test_silu_mul_deterministic_and_guard_bands():
    torch, q = gpu_or_skip()
    c = synth.make_inputs(4, 7, 2048, 2 * 1040, 128, seed=(65,))
    d = to_device(c, torch)
    p = repack_gate_up(c, d, q)
    a = bf16_bits(_run(c, torch, q, d, p))
    pad, n = 4096, c.M * (c.N // 2)
    big = torch.full((n + 2 * pad,), -7.25, dtype=torch.bfloat16, device="cuda:0")
    _run(c, torch, q, d, p, y=big[pad:pad + n].view(c.M, c.N // 2))
    host = big.float().cpu().numpy()
    assert np.all(host[:pad] == -7.25) and np.all(host[-pad:] == -7.25)
    assert np.array_equal(bf16_bits(big[pad:pad + n]).reshape(c.M, -1), a)


@pytest.mark.parametrize("bits,K,N,G", [(4, 256, 48, 128), (4, 4096, 28672, 128), (4, 352, 112, 32),
                                         (8, 384, 80, 384), (8, 1024, 4112, 64)])
def test_gate_up_repack_matches_oracle(bits, K, N, G):
    torch, q = gpu_or_skip()
    c = synth.make_inputs(bits, 1, K, N, G, seed=(68, bits, N), keep_codes=False)
    d = to_device(c, torch)
    got = repack_gate_up(c, d, q).cpu().numpy()
    want = oracle.repack_gate_up(bits, c.qweight, c.qzeros, c.scales, K, N, G)
    assert np.array_equal(got, want)


def test_silu_mul_rejects_bad_shapes_before_launch():
    torch, q = gpu_or_skip()
    c = synth.make_inputs(4, 2, 256, 72, 128, seed=(66,))
    d = to_device(c, torch)
    p = q.tf_repack_w4(d["qweight"], d["qzeros"], d["scales"], c.K, c.N, c.G)
    with pytest.raises(q.TileFuseError):
        q.tf_gemv_w4a16_silu_mul(d["x"], p, c.K, c.N, c.G)  # halves of 36 columns
    with pytest.raises(q.TileFuseError):
        repack_gate_up(c, d, q)
    x17 = torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda:0")
    c2 = synth.make_inputs(4, 1, 256, 128, 128, seed=(67,))
    d2 = to_device(c2, torch)
    with pytest.raises(q.TileFuseError):
        q.tf_gemv_w4a16_silu_mul(x17, repack_gate_up(c2, d2, q), 256, 128, 128)


@pytest.mark.parametrize("bits,M", [(4, 1), (4, 8), (8, 3)])
def test_silu_mul_large_sums(bits, M):
    """Scales raised by 2^12 put the sums in the thousands, so e^-g
    overflows fp32 wherever g < -89: silu there is -0, never NaN."""
    torch, q = gpu_or_skip()
    c0 = synth.make_inputs(bits, M, 1024, 2 * 528, 128, seed=(72, bits, M))
    scales = (c0.scales.astype(np.uint32) + (12 << 7)).astype(np.uint16)  # x 2^12, exact in bf16
    c = synth.gen.pack_case(bits, c0.codes, c0.zeros, scales, c0.x, c0.G)
    y = bf16_to_f64(_run(c, torch, q))
    assert not np.any(np.isnan(y))
    ref = oracle.awq_linear_silu_mul(c)
    gate = oracle.awq_linear(c, cols=np.arange(c.N // 2))
    assert np.any(gate < -89.0), "expected sums past the fp32 exponent range"
    ok, ratio = within_tolerance(y, ref)
    assert ok, f"worst error / bound = {ratio:.3f}"


# tf_gemm_*_silu_mul: every route of the plain GEMM call of the same shape.
# (bits, M, K, N, G, cus, route): the 16-row-chunk kernel at 17..64 rows (one
# to four row chunks, K split or not), 128-row tiles (forced at 64 rows, and
# at 96 and 100) with K split, 256-row tiles with K split, as wide + narrow
# launches, and as narrow tiles only; W8 on 256 x 256 tiles
GEMM_SILU = [
    (4, 17, 1024, 1056, 128, 0, 0), (4, 40, 2048, 2080, 64, 0, 0), (8, 64, 1024, 528, 1024, 0, 0),
    (4, 64, 1024, 1056, 128, 0, 1), (4, 100, 4096, 1024, 128, 0, 0), (4, 96, 4096, 256, 512, 4096, 0),
    (4, 300, 1024, 2080, 128, 0, 0), (4, 520, 512, 4096, 32, 40, 0), (8, 257, 384, 1040, 64, 0, 0),
    (8, 257, 384, 1040, 384, 0, 0),
]


@pytest.mark.parametrize("shape", GEMM_SILU, ids=[str(s) for s in GEMM_SILU])
def test_gemm_silu_mul_routes(shape):
    torch, q = gpu_or_skip()
    bits, M, K, N, G, cus, route = shape
    print(f"gemm silu_mul shape={shape}", flush=True)
    c = synth.make_inputs(bits, M, K, N, G, seed=(73, bits, M, K), keep_codes=False)
    d = to_device(c, torch)
    p = repack_gate_up(c, d, q)
    y = run_linear(q, bits, q.TF_OP_GEMM_SILU_MUL, d["x"], p, K, N, G, cus=cus, route=route, torch=torch)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (M, N // 2)
    rows = sample_indices(M, 48, seed=74)
    cols = sample_indices(N // 2, 384, seed=75)
    ref = oracle.awq_linear_silu_mul(c, cols=cols, rows=rows)
    ok, ratio = within_tolerance(bf16_to_f64(y)[rows][:, cols], ref)
    assert ok, f"worst error / bound = {ratio:.3f}"


def test_gemm_silu_mul_plans_cover_the_routes():
    """The shapes above reach the plans they are meant to (host-side plan)."""
    torch, q = gpu_or_skip()
    assert q.tf_gemm_plan(4, 96, 4096, 256, 512, 4096)[3] > 1               # K split
    assert q.tf_gemm_plan(4, 300, 1024, 2080, 128, 256)[3] > 1              # K split, 256-row tiles
    wide, narrow = q.tf_gemm_plan(4, 520, 512, 4096, 32, 40)[1:3]
    assert wide > 0 and narrow > 0                                          # wide + narrow launches
    assert q.tf_gemm_plan(8, 257, 384, 1040, 64, 256)[1:3] == (0, 17)       # narrow tiles only
    assert q.tf_gemm_plan(8, 257, 384, 1040, 384, 256)[7] == 256            # W8, 256 x 256 tiles
    assert q.tf_gemm_plan(4, 100, 4096, 1024, 128, 256)[6] == 128           # 128-row tiles
    assert q.tf_gemm_plan(4, 40, 2048, 2080, 64, 256)[5] == 1               # the GEMV kernel


def test_gemm_silu_mul_decoder_prefill():
    """The decoder layer's gate/up at 2048 rows (K = 4096, 2 x 14336 columns:
    seven rounds of 256 x 128 tiles), on sampled rows and columns."""
    torch, q = gpu_or_skip()
    c = synth.make_inputs(4, 2048, 4096, 28672, 128, seed=(76,), keep_codes=False)
    d = to_device(c, torch)
    y = q.tf_gemm_w4a16_silu_mul(d["x"], repack_gate_up(c, d, q), 4096, 28672, 128)
    torch.cuda.synchronize()
    rows = sample_indices(2048, 24, seed=77)
    cols = sample_indices(14336, 256, seed=78)
    ok, ratio = within_tolerance(bf16_to_f64(y)[rows][:, cols], oracle.awq_linear_silu_mul(c, cols=cols, rows=rows))
    assert ok, f"worst error / bound = {ratio:.3f}"


@pytest.mark.parametrize("M,cus", [(300, 0), (96, 4096), (40, 0)])
def test_gemm_silu_mul_zero_gate_gives_zero(M, cus):
    torch, q = gpu_or_skip()
    K, N, G = 4096, 1056, 512
    c0 = synth.make_inputs(4, M, K, N, G, seed=(79, M))
    codes = c0.codes.copy()
    codes[:, : N // 2] = c0.zeros[np.arange(K) // G][:, : N // 2]
    c = synth.gen.pack_case(4, codes, c0.zeros, c0.scales, c0.x, G)
    d = to_device(c, torch)
    y = run_linear(q, 4, q.TF_OP_GEMM_SILU_MUL, d["x"], repack_gate_up(c, d, q), K, N, G, cus=cus, torch=torch)
    torch.cuda.synchronize()
    assert np.all(bf16_to_f64(y) == 0.0)
