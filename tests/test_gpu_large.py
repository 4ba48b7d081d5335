"""Maximum sizes: buffers past 4 GiB, where a 32-bit byte offset would wrap.

Inputs are drawn on the GPU from seeded generators (the full arrays are too
large to build on the host in reasonable time); the oracle checks sampled
outputs from host copies of just the rows, or the 8-column words, they
need.  AWQ packs eight columns per word, so a set of words is an exact
sub-problem of its own."""

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bf16_to_f64, gpu_or_skip, within_tolerance

pytestmark = pytest.mark.gpu


def test_gemm_activations_past_4gib():
    """x of 135000 x 16384 bf16 (4.4 GB): rows on both sides of byte offset
    2^32, through the tiled GEMM (256-row tiles, a ragged last tile and a
    ragged last column block)."""
    torch, q = gpu_or_skip()
    M, K, N, G = 135000, 16384, 136, 128
    print(f"large gemm M={M} K={K} N={N}", flush=True)
    c = synth.make_inputs(4, 1, K, N, G, seed=(81, K, N))
    dev = "cuda:0"
    gen = torch.Generator(device=dev).manual_seed(8101)
    x = torch.randn((M, K), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    assert x.numel() * 2 > 2**32
    qw = torch.from_numpy(c.qweight.view(np.int32)).to(dev)
    qz = torch.from_numpy(c.qzeros.view(np.int32)).to(dev)
    sc = torch.from_numpy(c.scales.view(np.int16)).to(dev)
    packed = q.tf_repack_w4(qw, qz, sc, K, N, G)
    y = q.tf_gemm_w4a16(x, packed, K, N, G)
    torch.cuda.synchronize()
    edge = (2**32) // (2 * K)  # first row at or past byte offset 2^32
    rows = np.array(sorted({0, 1, 255, 256, edge - 1, edge, edge + 1, edge + 255, M - 257, M - 256, M - 1}))
    xr = x[torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    w = oracle.dequant(4, c.qweight, c.qzeros, c.scales, K, N, G)
    ref = oracle.linear(xr, w)
    ok, ratio = within_tolerance(bf16_to_f64(y[torch.from_numpy(rows).to(dev)]), ref)
    assert ok, f"worst error / bound = {ratio:.3f}"


@pytest.mark.parametrize("M,gemm", [(1, False), (3, False), (40, True)])
def test_gemv_packed_past_4gib(M, gemm):
    """W4, K = 8192, N = 2^20 + 16: the packed buffer is 4.46 GB, so blocks
    past the 63 000th start beyond byte offset 2^32 (the GEMV kernels: M = 1
    the kernel for up to 16 rows, M = 3 and 40 the 16-row-chunk kernel)."""
    torch, q = gpu_or_skip()
    K, N, G = 8192, (1 << 20) + 16, 128
    print(f"large gemv M={M} K={K} N={N}", flush=True)
    dev = "cuda:0"
    gen = torch.Generator(device=dev).manual_seed(8202)
    i32 = torch.iinfo(torch.int32)
    qw = torch.randint(i32.min, i32.max, (K, N // 8), generator=gen, device=dev, dtype=torch.int32)
    qz = torch.randint(i32.min, i32.max, (K // G, N // 8), generator=gen, device=dev, dtype=torch.int32)
    sc = (torch.rand((K // G, N), generator=gen, device=dev) * 0.02 + 0.002).to(torch.bfloat16)
    x = torch.randn((M, K), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    packed = q.tf_repack_w4(qw, qz, sc.view(torch.int16), K, N, G)
    assert packed.numel() > 2**32
    fn = q.tf_gemm_w4a16 if gemm else q.tf_gemv_w4a16
    y = fn(x, packed, K, N, G)
    torch.cuda.synchronize()
    block_bytes = packed.numel() // (N // 16)
    first_far = -(-(2**32) // block_bytes) * 2  # a word of the first block past 2^32
    words = np.array(sorted({0, 1, first_far - 2, first_far, first_far + 1, N // 8 - 2, N // 8 - 1}))
    wt = torch.from_numpy(words).to(dev)
    cols = (8 * words[:, None] + np.arange(8)[None, :]).reshape(-1)
    qw_s = qw[:, wt].cpu().numpy().view(np.uint32)
    qz_s = qz[:, wt].cpu().numpy().view(np.uint32)
    sc_s = sc.view(torch.int16)[:, torch.from_numpy(cols).to(dev)].cpu().numpy().view(np.uint16)
    xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
    w = oracle.dequant(4, qw_s, qz_s, sc_s, K, cols.size, G)
    ref = oracle.linear(xb, w)
    got = bf16_to_f64(y[:, torch.from_numpy(cols).to(dev)])
    ok, ratio = within_tolerance(got, ref)
    assert ok, f"worst error / bound = {ratio:.3f}"
