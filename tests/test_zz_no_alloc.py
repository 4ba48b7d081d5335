"""tf_gemm_w4a16_noalloc: the W4 GEMM call whose split-K partial sums live in
the library's fixed per-GPU array instead of a caller's workspace.  Checked
through the C ABI against tf_gemm_w4a16 with a workspace (same kernels and
plan, so bit for bit), on two calls in a row, the second with a smaller
input, for both kernels that split K; and against the oracle."""

import ctypes

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bf16_bits, bf16_to_f64, gpu_or_skip, repack, to_device, within_tolerance

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20

# (M, K, N): the 16-row-chunk GEMV kernel with K split (M <= 64), and the
# tiled GEMM with K split (128-row tiles); each pair runs larger then smaller
PAIRS = [((48, 14336, 4096), (24, 4096, 1024)), ((100, 4096, 2048), (80, 2048, 512))]


def _call_raw(q, x, packed, y, M, K, N, G):
    L = q.load_library()
    import torch

    stream = torch.cuda.current_stream().cuda_stream
    return L.tf_gemm_w4a16_noalloc(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(packed.data_ptr()),
                                   packed.numel(), ctypes.c_void_p(y.data_ptr()), M, K, N, G,
                                   ctypes.c_void_p(stream))


@pytest.mark.parametrize("pair", PAIRS)
def test_noalloc_matches_workspace_call(pair):
    torch, q = gpu_or_skip()
    for i, (M, K, N) in enumerate(pair):
        G = 128
        need = q.tf_workspace_bytes(4, True, M, K, N, G)
        print(f"noalloc M={M} K={K} N={N} workspace={need}", flush=True)
        assert 0 < need <= SCRATCH_BYTES, "the case must split K within the array"
        c = synth.make_inputs(4, M, K, N, G, seed=(91, i, M, K))
        d = to_device(c, torch)
        p = repack(c, d, q)
        ref = q.tf_gemm_w4a16(d["x"], p, K, N, G)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        assert _call_raw(q, d["x"], p, y, M, K, N, G) == 0
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), bf16_bits(ref))
        ok, ratio = within_tolerance(bf16_to_f64(y), oracle.awq_linear(c))
        assert ok, ratio


def test_noalloc_largest_split_fits_the_array():
    """The largest split plan on this device (256 x 256 tiles filling half
    the compute units, K in two ranges) runs from the array, and matches the
    workspace call bit for bit."""
    torch, q = gpu_or_skip()
    M, K, N, G = 2048, 4096, 4096, 128
    need = q.tf_workspace_bytes(4, True, M, K, N, G)
    print(f"noalloc largest split: {need} bytes", flush=True)
    assert 0 < need <= SCRATCH_BYTES
    c = synth.make_inputs(4, M, K, N, G, seed=(93,), keep_codes=False)
    d = to_device(c, torch)
    p = repack(c, d, q)
    ref = q.tf_gemm_w4a16(d["x"], p, K, N, G)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    assert _call_raw(q, d["x"], p, y, M, K, N, G) == 0
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y), bf16_bits(ref))


def test_noalloc_without_split_and_empty():
    torch, q = gpu_or_skip()
    M, K, N, G = 2048, 4096, 8192, 128  # 256 output tiles: no K split
    assert q.tf_workspace_bytes(4, True, M, K, N, G) == 0
    c = synth.make_inputs(4, M, K, N, G, seed=(92,), keep_codes=False)
    d = to_device(c, torch)
    p = repack(c, d, q)
    y = q.tf_gemm_w4a16_noalloc(d["x"], p, K, N, G)
    ref = q.tf_gemm_w4a16(d["x"], p, K, N, G)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(y), bf16_bits(ref))
    x0 = torch.empty((0, K), dtype=torch.bfloat16, device="cuda:0")
    assert tuple(q.tf_gemm_w4a16_noalloc(x0, p, K, N, G).shape) == (0, N)
