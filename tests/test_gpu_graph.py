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
    from gpu_harness import run_linear

    print(f"graph silu_mul gemm={gemm} M={M} K={K} N={N}", flush=True)
    c = synth.make_inputs(4, M, K, N, 128, seed=(82, M), keep_codes=False)
    d = to_device(c, torch)
    p = q.tf_repack_w4_gate_up(d["qweight"], d["qzeros"], d["scales"], K, N, 128)
    op = q.TF_OP_GEMM_SILU_MUL if gemm else q.TF_OP_GEMV_SILU_MUL

    def fn(x, pk, K, N, G, y):
        return run_linear(q, 4, op, x, pk, K, N, G, cus=cus, y=y, torch=torch)

    y = torch.empty((M, N // 2), dtype=torch.bfloat16, device="cuda:0")
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


def test_graph_survives_workspace_growth_on_its_stream():
    """A graph captured with a small K split holds the stream's workspace;
    a later eager call on that stream that needs a larger workspace must not
    free it (the binding keeps replaced workspaces), so replays still match."""
    torch, q = gpu_or_skip()
    small = (4, 48, 2048, 1024, 128)
    large = (4, 64, 14336, 4096, 128)
    cases = [synth.make_inputs(*shape, seed=(83, i), keep_codes=False)
             for i, shape in enumerate((small, large))]
    dev = [to_device(c, torch) for c in cases]
    packs = [repack(c, d, q) for c, d in zip(cases, dev)]
    need = [q.tf_workspace_bytes(c.bits, True, c.M, c.K, c.N, c.G) for c in cases]
    print(f"graph workspace growth: {need}", flush=True)
    assert 0 < need[0] < need[1], "the second call must need a larger workspace"
    c0, d0, p0 = cases[0], dev[0], packs[0]
    fn = linear_fn(q, 4, True)
    y = torch.empty((c0.M, c0.N), dtype=torch.bfloat16, device="cuda:0")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(d0["x"], p0, c0.K, c0.N, c0.G, y=y)
        torch.cuda.synchronize()
        eager = y.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            fn(d0["x"], p0, c0.K, c0.N, c0.G, y=y)
        torch.cuda.synchronize()
        c1, d1, p1 = cases[1], dev[1], packs[1]
        big = fn(d1["x"], p1, c1.K, c1.N, c1.G)  # grows the stream's workspace
        torch.cuda.synchronize()
        # fresh allocations that would reuse the old workspace were it freed:
        # a replay would then overwrite them with its partial sums
        junk = [torch.full((need[0] // 4,), 3.0, device="cuda:0") for _ in range(8)]
    for it in range(3):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {it} differs"
        assert all(bool((j == 3.0).all()) for j in junk), f"replay {it} wrote into memory it does not own"
    del junk, big
