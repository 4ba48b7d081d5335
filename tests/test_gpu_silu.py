"""Fused [gate | up] GEMV with the SiLU product (tf_gemv_*_silu_mul) against
the oracle: y[m][n] = silu(g) * u from the unrounded sums of columns n and
N/2 + n, one rounding to bf16."""

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bf16_bits, bf16_to_f64, gpu_or_skip, repack, sample_indices, to_device, within_tolerance

pytestmark = pytest.mark.gpu

# (bits, M, K, N, G), N the fused width: one or two gate/up pairs per
# workgroup, an odd number of pairs where two per workgroup would not
# divide them, ragged K, G = 32 / 64 / 128 / per channel, up to 16 rows
SHAPES = [
    (4, 1, 512, 320, 128), (4, 3, 352, 64, 32), (4, 8, 1024, 4096, 64), (4, 16, 4096, 4096, 128),
    (4, 2, 256, 16384, 128), (4, 5, 128, 32800, 128), (4, 1, 384, 96, 384),
    (8, 1, 256, 96, 256), (8, 4, 2048, 8192, 128), (8, 12, 1024, 16384, 1024), (8, 16, 512, 64, 32),
]


def _fn(q, bits):
    return q.tf_gemv_w4a16_silu_mul if bits == 4 else q.tf_gemv_w8a16_silu_mul


def _run(case, torch, q, d=None, p=None, y=None):
    d = d or to_device(case, torch)
    p = p if p is not None else repack(case, d, q)
    out = _fn(q, case.bits)(d["x"], p, case.K, case.N, case.G, y=y)
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
@pytest.mark.parametrize("bits,M", [(4, 1), (4, 6), (8, 3)])
def test_zero_half_gives_exact_zero(bits, M, half):
    """q == z on the gate half makes g exactly 0 and silu(0) = 0; on the up
    half u is exactly 0.  Either way every output is exactly zero."""
    torch, q = gpu_or_skip()
    K, N, G = 1024, 2 * 1056, 128
    c0 = synth.make_inputs(bits, M, K, N, G, seed=(64, bits, M))
    codes = c0.codes.copy()
    cols = slice(0, N // 2) if half == "gate" else slice(N // 2, N)
    codes[:, cols] = c0.zeros[np.arange(K) // G][:, cols]
    c = synth.gen.pack_case(bits, codes, c0.zeros, c0.scales, c0.x, G)
    y = _run(c, torch, q)
    assert np.all(bf16_to_f64(y) == 0.0)


def test_silu_mul_deterministic_and_guard_bands():
    torch, q = gpu_or_skip()
    c = synth.make_inputs(4, 7, 2048, 2 * 1040, 128, seed=(65,))
    d = to_device(c, torch)
    p = repack(c, d, q)
    a = bf16_bits(_run(c, torch, q, d, p))
    pad, n = 4096, c.M * (c.N // 2)
    big = torch.full((n + 2 * pad,), -7.25, dtype=torch.bfloat16, device="cuda:0")
    _run(c, torch, q, d, p, y=big[pad:pad + n].view(c.M, c.N // 2))
    host = big.float().cpu().numpy()
    assert np.all(host[:pad] == -7.25) and np.all(host[-pad:] == -7.25)
    assert np.array_equal(bf16_bits(big[pad:pad + n]).reshape(c.M, -1), a)


def test_silu_mul_rejects_bad_shapes_before_launch():
    torch, q = gpu_or_skip()
    c = synth.make_inputs(4, 2, 256, 80, 128, seed=(66,))
    d = to_device(c, torch)
    p = repack(c, d, q)
    with pytest.raises(q.TileFuseError):
        q.tf_gemv_w4a16_silu_mul(d["x"], p, c.K, c.N, c.G)  # 40-column halves: not whole blocks
    x17 = torch.zeros((17, 256), dtype=torch.bfloat16, device="cuda:0")
    c2 = synth.make_inputs(4, 1, 256, 128, 128, seed=(67,))
    d2 = to_device(c2, torch)
    with pytest.raises(q.TileFuseError):
        q.tf_gemv_w4a16_silu_mul(x17, repack(c2, d2, q), 256, 128, 128)
