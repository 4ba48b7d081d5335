"""The layer under HIP-graph capture: the kernels use no memset and no
counters (a split launch writes its partial sums and a second kernel adds
them), so a captured graph replays correctly.  Each replay is checked bitwise
against the eager result, with eager work and synchronisations between
replays."""

import numpy as np
import pytest

import synth
from gpu_harness import gpu_or_skip, linear_fn, repack, to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gemm,bits,M,K,N,G", [(False, 4, 1, 4096, 1024, 128), (False, 8, 8, 8192, 512, 8192),
                                               (False, 4, 16, 14336, 1024, 128),
                                               (True, 4, 96, 1024, 320, 128), (True, 4, 48, 4096, 4096, 128)])
def test_graph_replays_match_eager(gemm, bits, M, K, N, G):
    torch, q = gpu_or_skip()
    print(f"graph gemm={gemm} W{bits} M={M} K={K} N={N} G={G}", flush=True)
    c = synth.make_inputs(bits, M, K, N, G, seed=(71, bits, M))
    d = to_device(c, torch)
    p = repack(c, d, q)
    fn = linear_fn(q, bits, gemm)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(d["x"], p, K, N, G, y=y)  # warm-up on the capture stream (creates its workspace)
        torch.cuda.synchronize()
        eager = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn(d["x"], p, K, N, G, y=y)
    torch.cuda.synchronize()
    other = torch.empty_like(y)
    for it in range(4):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {it} differs"
        fn(d["x"], p, K, N, G, y=other)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, eager)


@pytest.mark.parametrize("gemm,M,K,N,cus", [(False, 1, 4096, 2112, 0), (False, 12, 14336, 1024, 256),
                                            (True, 40, 2048, 2080, 0), (True, 300, 1024, 2080, 0)])
def test_graph_replays_match_eager_silu_mul(gemm, M, K, N, cus):
    """The SiLU-product calls under capture, with and without a K split."""
    torch, q = gpu_or_skip()
    from gpu_harness import planning_cus

    print(f"graph silu_mul gemm={gemm} M={M} K={K} N={N}", flush=True)
    c = synth.make_inputs(4, M, K, N, 128, seed=(82, M), keep_codes=False)
    d = to_device(c, torch)
    p = q.tf_repack_w4_gate_up(d["qweight"], d["qzeros"], d["scales"], K, N, 128)
    fn = q.tf_gemm_w4a16_silu_mul if gemm else q.tf_gemv_w4a16_silu_mul
    y = torch.empty((M, N // 2), dtype=torch.bfloat16, device="cuda:0")
    with planning_cus(q, cus):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(d["x"], p, K, N, 128, y=y)
            torch.cuda.synchronize()
            eager = y.clone()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                fn(d["x"], p, K, N, 128, y=y)
        torch.cuda.synchronize()
        other = torch.empty_like(y)
        for it in range(3):
            y.fill_(0)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, eager), f"replay {it} differs"
            fn(d["x"], p, K, N, 128, y=other)
            torch.cuda.synchronize()
            assert torch.equal(other, eager)
