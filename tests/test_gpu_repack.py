"""GPU repack and dequant hook against the oracle: bit-exact."""

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import gpu_or_skip, repack, to_device

pytestmark = pytest.mark.gpu

SMALL = [
    (4, 64, 128, 32), (4, 256, 200, 128), (4, 384, 64, 384), (4, 192, 8, 64), (4, 96, 136, 96),
    (8, 64, 128, 32), (8, 256, 100, 256), (8, 128, 4, 64), (8, 96, 72, 32), (8, 512, 130, 128),
]


@pytest.mark.parametrize("bits,K,N,G", SMALL)
def test_repack_matches_oracle_bytes(bits, K, N, G):
    torch, q = gpu_or_skip()
    print(f"repack W{bits} K={K} N={N} G={G}", flush=True)
    c = synth.make_inputs(bits, 1, K, N, G, seed=(41, bits, K, N))
    packed = repack(c, to_device(c, torch), q)
    torch.cuda.synchronize()
    got = packed.cpu().numpy()
    want = oracle.repack(bits, c.qweight, c.qzeros, c.scales, K, N, G)
    assert got.size == want.size
    assert np.array_equal(got, want)
    codes, zeros, scales = oracle.unrepack(bits, got, K, N, G)
    assert np.array_equal(codes, c.codes) and np.array_equal(zeros, c.zeros) and np.array_equal(scales, c.scales)


@pytest.mark.parametrize("config,shape_id", [(0, 0), (1, 1), (2, 0), (3, 1), (4, 1)])
def test_repack_matches_oracle_bytes_full_size(config, shape_id):
    torch, q = gpu_or_skip()
    c = synth.make_case(config, shape_id, 1, keep_codes=False)
    print(f"repack full {c.name}", flush=True)
    packed = repack(c, to_device(c, torch), q)
    torch.cuda.synchronize()
    want = oracle.repack(c.bits, c.qweight, c.qzeros, c.scales, c.K, c.N, c.G)
    assert np.array_equal(packed.cpu().numpy(), want)


@pytest.mark.parametrize("hook", ["gemm", "gemv"])
@pytest.mark.parametrize("bits,K,N,G", SMALL + [(4, 4096, 4096, 128), (8, 8192, 512, 8192), (8, 4096, 512, 32)])
def test_dequant_f32_bit_exact(bits, K, N, G, hook):
    """The fp32 weights decoded by each kernel's own operand builder (the
    GEMM's exact bf16 q - z, the GEMV's 128 + q and 128 + z) equal the
    oracle's (q - z) * s bit for bit."""
    torch, q = gpu_or_skip()
    print(f"dequant {hook} W{bits} K={K} N={N} G={G}", flush=True)
    c = synth.make_inputs(bits, 1, K, N, G, seed=(42, bits, K, N))
    packed = repack(c, to_device(c, torch), q)
    fn = {("gemm", 4): q.tf_dequant_w4_f32, ("gemm", 8): q.tf_dequant_w8_f32,
          ("gemv", 4): q.tf_dequant_gemv_w4_f32, ("gemv", 8): q.tf_dequant_gemv_w8_f32}[(hook, bits)]
    w = fn(packed, K, N, G)
    torch.cuda.synchronize()
    want = oracle.dequant(bits, c.qweight, c.qzeros, c.scales, K, N, G)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("hook", ["gemm", "gemv"])
@pytest.mark.parametrize("bits", [4, 8])
def test_dequant_every_code_and_zero_point(bits, hook):
    """Every (q, z) pair of the bit width, with scales of both signs and
    exponents from 2^-100 to 2^100: still the oracle's value bit for bit."""
    torch, q = gpu_or_skip()
    levels = 1 << bits
    G = 32
    K = G * levels                      # group g has zero point (g + n) % levels
    N = 16 if bits == 4 else 64
    k = np.arange(K)
    codes = ((k[:, None] + 7 * np.arange(N)[None, :]) % levels).astype(np.uint8)
    if bits == 8:                       # 32 rows per group: column n holds q in 32 (n % 8) .. + 31
        codes = ((k[:, None] % G) + G * (np.arange(N)[None, :] % 8)).astype(np.uint8)
    zeros = ((np.arange(K // G)[:, None] + np.arange(N)[None, :]) % levels).astype(np.uint8)
    rng = np.random.default_rng(44)
    exps = rng.integers(-100, 101, size=(K // G, N))
    mant = rng.uniform(1.0, 2.0, size=(K // G, N)) * rng.choice([-1.0, 1.0], size=(K // G, N))
    scales = synth.f32_to_bf16_bits((mant * np.exp2(exps)).astype(np.float32))
    x = synth.f32_to_bf16_bits(np.zeros((1, K), np.float32))
    c = synth.gen.pack_case(bits, codes, zeros, scales, x, G)
    packed = repack(c, to_device(c, torch), q)
    fn = {("gemm", 4): q.tf_dequant_w4_f32, ("gemm", 8): q.tf_dequant_w8_f32,
          ("gemv", 4): q.tf_dequant_gemv_w4_f32, ("gemv", 8): q.tf_dequant_gemv_w8_f32}[(hook, bits)]
    w = fn(packed, K, N, G)
    torch.cuda.synchronize()
    want = oracle.dequant(bits, c.qweight, c.qzeros, c.scales, K, N, G)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_packed_size_and_version_agree():
    torch, q = gpu_or_skip()
    assert q.tf_format_version() == 2
    assert q.tf_packed_bytes_w4(4096, 4096, 128) == oracle.packed_bytes(4, 4096, 4096, 128)


def _symmetric(c):
    """The case with every zero point 2^(bits-1): what a checkpoint without a
    zero-point tensor means."""
    zeros = np.full_like(c.zeros, 1 << (c.bits - 1))
    return synth.gen.pack_case(c.bits, c.codes, zeros, c.scales, c.x, c.G)


@pytest.mark.parametrize("bits,K,N,G", [(4, 256, 200, 128), (4, 384, 64, 384), (4, 192, 8, 64), (8, 256, 100, 256),
                                        (8, 96, 72, 32), (4, 4096, 1024, 128)])
def test_symmetric_repack_matches_oracle_bytes(bits, K, N, G):
    """No zero-point tensor (NULL) packs exactly as an explicit tensor of
    2^(bits-1), as the oracle packs it."""
    torch, q = gpu_or_skip()
    print(f"symmetric repack W{bits} K={K} N={N} G={G}", flush=True)
    c = _symmetric(synth.make_inputs(bits, 1, K, N, G, seed=(43, bits, K, N)))
    d = to_device(c, torch)
    fn = q.tf_repack_w4 if bits == 4 else q.tf_repack_w8
    packed = fn(d["qweight"], None, d["scales"], K, N, G)
    torch.cuda.synchronize()
    want = oracle.repack(bits, c.qweight, c.qzeros, c.scales, K, N, G)
    assert np.array_equal(packed.cpu().numpy(), want)


@pytest.mark.parametrize("gemm,M", [(False, 1), (False, 12), (True, 40), (True, 300)])
@pytest.mark.parametrize("bits", [4, 8])
def test_symmetric_linear_within_tolerance(gemm, M, bits):
    torch, q = gpu_or_skip()
    from gpu_harness import bf16_to_f64, linear_fn, within_tolerance

    K, N, G = 2048, 264, 128
    print(f"symmetric linear gemm={gemm} W{bits} M={M}", flush=True)
    c = _symmetric(synth.make_inputs(bits, M, K, N, G, seed=(44, bits, M)))
    d = to_device(c, torch)
    fn = q.tf_repack_w4 if bits == 4 else q.tf_repack_w8
    packed = fn(d["qweight"], None, d["scales"], K, N, G)
    y = linear_fn(q, bits, gemm)(d["x"], packed, K, N, G)
    torch.cuda.synchronize()
    ok, ratio = within_tolerance(bf16_to_f64(y), oracle.awq_linear(c))
    assert ok, f"worst error / bound = {ratio:.3f}"
