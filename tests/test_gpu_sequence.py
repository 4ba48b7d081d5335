"""Calls of different shapes and widths queued back to back on one stream,
checked only after all of them ran: no call may depend on state a previous
call left behind."""

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bf16_to_f64, gpu_or_skip, linear_fn, repack, to_device, within_tolerance

pytestmark = pytest.mark.gpu


def test_mixed_shapes_back_to_back():
    torch, q = gpu_or_skip()
    plan = [(4, False, 1, 4096, 1024, 128), (4, False, 8, 4096, 14336, 128), (8, False, 3, 8192, 512, 8192),
            (4, True, 130, 1024, 320, 64), (4, False, 16, 14336, 4096, 128), (8, True, 64, 512, 100, 512),
            (4, True, 40, 4096, 4096, 128), (8, True, 20, 2048, 8192, 2048), (4, False, 1, 4096, 1024, 128)]
    runs = []
    for it, (bits, gemm, M, K, N, G) in enumerate(plan):
        c = synth.make_inputs(bits, M, K, N, G, seed=(61, it))
        d = to_device(c, torch)
        runs.append((c, linear_fn(q, bits, gemm)(d["x"], repack(c, d, q), K, N, G)))
    torch.cuda.synchronize()
    for c, y in runs:
        print(f"sequence W{c.bits} M={c.M} K={c.K} N={c.N}", flush=True)
        cols = np.unique(np.concatenate([[0, c.N - 1], np.arange(0, c.N, max(1, c.N // 512))]))
        ok, ratio = within_tolerance(bf16_to_f64(y)[:, cols], oracle.awq_linear(c, cols=cols))
        assert ok, ratio


def test_explicit_stream_workspace_growth():
    """Split calls on a side stream passed as stream=, the second needing a
    larger workspace than the first (the binding then allocates a new one on
    that stream while the first call may still be queued)."""
    torch, q = gpu_or_skip()
    s = torch.cuda.Stream()
    shapes = [(4, True, 48, 2048, 1024, 128), (4, True, 64, 14336, 4096, 128), (4, False, 16, 14336, 2048, 128)]
    runs = []
    for it, (bits, gemm, M, K, N, G) in enumerate(shapes):
        c = synth.make_inputs(bits, M, K, N, G, seed=(62, it), keep_codes=False)
        d = to_device(c, torch)
        p = repack(c, d, q)
        assert q.tf_workspace_bytes(bits, gemm, M, K, N, G) > 0, "expected a K split"
        s.wait_stream(torch.cuda.current_stream())
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        y.record_stream(s)
        linear_fn(q, bits, gemm)(d["x"], p, K, N, G, y=y, stream=s)
        runs.append((c, y, d, p))
    torch.cuda.synchronize()
    for c, y, _, _ in runs:
        print(f"side stream W{c.bits} M={c.M} K={c.K} N={c.N}", flush=True)
        cols = np.unique(np.concatenate([[0, c.N - 1], np.arange(0, c.N, max(1, c.N // 256))]))
        ok, ratio = within_tolerance(bf16_to_f64(y)[:, cols], oracle.awq_linear(c, cols=cols))
        assert ok, ratio
