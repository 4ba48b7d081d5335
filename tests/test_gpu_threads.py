"""Calls from several host threads at once, each thread on a stream of its own.

The library keeps no per-call state outside its arguments: the device's
compute-unit count is cached once per device, and the binding keeps one
split-K workspace per (device, stream).  Every kernel sums in a fixed order,
so each thread's outputs must equal, bit for bit, those of the same calls
made one at a time on the default stream.  The cases cover the GEMV at M = 1,
the 16-row-chunk kernel with a K split, both tiled GEMM kernels with a K split
(all three of those through a workspace) and W8.
"""

import threading

import pytest

import synth
from gpu_harness import gpu_or_skip, linear_fn, repack, to_device

pytestmark = pytest.mark.gpu

# (gemm, bits, M, K, N, G)
CASES = [(False, 4, 1, 4096, 2048, 128), (True, 4, 40, 4096, 512, 128), (True, 4, 130, 4096, 256, 128),
         (True, 8, 300, 1024, 456, 128), (True, 4, 1024, 1024, 8192, 128)]
THREADS = 4
ITERS = 12


def test_threads_on_their_own_streams_match_serial_calls():
    torch, q = gpu_or_skip()
    calls, refs = [], []
    for gemm, bits, M, K, N, G in CASES:
        c = synth.make_inputs(bits, M, K, N, G, seed=(83, bits, M, K))
        d = to_device(c, torch)
        p = repack(c, d, q)
        fn = linear_fn(q, bits, gemm)
        calls.append((fn, d["x"], p, M, K, N, G))
        refs.append(fn(d["x"], p, K, N, G))
    torch.cuda.synchronize()
    with_ws = sum(q.tf_workspace_bytes(bits, gemm, M, K, N, G) > 0 for gemm, bits, M, K, N, G in CASES)
    assert with_ws >= 3, "the cases must exercise the per-stream workspace"

    results, errors = {}, []
    start = threading.Barrier(THREADS, timeout=60)

    def work(tid):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                ys = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0") for _, _, _, M, _, N, _ in calls]
                start.wait()
                for it in range(ITERS):
                    # every thread walks the cases in its own rotating order
                    for j in range(len(calls)):
                        i = (j + tid + it) % len(calls)
                        fn, x, p, M, K, N, G = calls[i]
                        fn(x, p, K, N, G, y=ys[i])
                s.synchronize()
                results[tid] = [y.clone() for y in ys]
                s.synchronize()
        except Exception as exc:  # reported by the main thread
            errors.append(exc)

    print(f"threads {THREADS} x {ITERS} rounds of {len(CASES)} calls", flush=True)
    threads = [threading.Thread(target=work, args=(t,)) for t in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    for tid in range(THREADS):
        for i, (case, y, ref) in enumerate(zip(CASES, results[tid], refs)):
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), f"thread {tid}, case {case}"
