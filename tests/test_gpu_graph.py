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
