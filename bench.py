"""Benchmark of the fused W4A16 / W8A16 linear layer on one MI355X.

Headline (value): W4A16 GEMV at M=1 over one Llama-style decoder layer's seven
linears (q/o 4096x4096, k/v 4096x1024, gate/up 4096x14336, down 14336x4096,
group 128), as effective HBM GB/s = algorithmic bytes / time.  A step is one
pass over the layer's linears with q/k/v fused into one N=6144 GEMV and
gate/up into one N=28672 GEMV, as serving engines store them (four launches).
The K timed steps are launched eagerly, queued behind filler work so that the
GPU runs them back to back (kernels on one stream run one after another, so
each launch sees its predecessor's results, as in a real decode step); HIP
events on the launch stream bracket them.  HIP-graph replay of the same steps
and the seven separate launches are timed beside it.  Steps rotate over weight
replicas whose total (5 x 113 MB) exceeds twice the 256 MB Infinity Cache, so
every step streams its weights from HBM.  Inputs are resident in HBM before
the timed region starts.

Also reported: the dominant kernel against its roofline (per-launch durations
from HIP events on the launch stream), the W4A16 prefill GEMM at M=2048
(TFLOP/s against the dense bf16 MFMA peak), the CPU oracle on a bounded
sample of the headline workload, and two measured practical roofs: a plain
streaming-read kernel over the same packed buffers in the same launch
pattern, and back-to-back bf16 MFMAs sustained for as long as the GEMM runs.

Algorithmic bytes of one linear: K*N*b/8 codes + (K/G)*N*(b/8 + 2) metadata
+ 2*M*(K + N) activations in and outputs out.  Flops: 2*M*K*N.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_DENSE_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, published
INFINITY_CACHE_BYTES = 256 * 2**20
COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemv_w4a16_layer_m1_counters.json")
GEMM_COUNTERS_FILE = os.path.join(ROOT, "profiles", "gemm_w4a16_m2048_counters.json")
GEMM_SOURCES = ("gemm256.hip", "gemm.hip", "tf_gemm_common.h", "tf_common.h", "tf_launch.h", "tf_operands.h")
GEMM_TRACE_NAME = "gemm256_kernel"


def algorithmic_bytes(bits, M, K, N, G):
    return K * N * bits // 8 + (K // G) * N * (bits // 8 if bits == 8 else 0.5) + (K // G) * N * 2 + 2 * M * (K + N)


GEMV_SOURCES = ("gemv.hip", "tf_common.h", "tf_launch.h", "tf_operands.h")
# the dominant kernel of the headline step as a kernel trace names it: the
# GEMV kernel for W4, one k-tile per group (mode 2), ring depth D, BPW blocks
# per workgroup, plain bf16 store (epilogue 0)
GEMV_TRACE_NAME = "gemv_kernel<4, 2, {depth}, {bpw}, 0>"


def kernel_source_hash(sources=GEMV_SOURCES):
    """Hash of a kernel's sources: stored counters are used only while the
    kernel they were taken on is unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "quantized_linear_layers_awq_amd", "csrc")
    for name in sources:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--replicas", type=int, default=0, help="weight replicas to rotate (0: enough to beat the cache)")
    p.add_argument("--only", choices=["all", "gemv", "gemm", "copy", "configs", "crossover", "energy", "silu"],
                   default="all",
                   help="restrict the run (profiling passes); 'copy' runs the plain-copy calibration kernel")
    p.add_argument("--counters-kernel", default=GEMV_TRACE_NAME.format(depth=4, bpw=1),
                   help="kernel name (as traced) whose dispatches --counters-from averages")
    p.add_argument("--counters-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="no GPU: read four rocprofv3 --pmc output directories (FETCH_SIZE and WRITE_SIZE over "
                        "'--only gemv', then over '--only copy') and write the per-launch HBM traffic file")
    p.add_argument("--gemm-counters-from", nargs=6,
                   metavar=("TRACE", "BUSY", "FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                   help="no GPU: read a --kernel-trace directory and five --pmc directories over '--only gemm' "
                        "(SQ_VALU_MFMA_BUSY_CYCLES with GRBM_GUI_ACTIVE, FETCH_SIZE, WRITE_SIZE) and "
                        "'--only copy' (FETCH_SIZE, WRITE_SIZE), and write the GEMM counter file")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-energy", action="store_true", help="skip the energy-per-call leg")
    p.add_argument("--no-configs", action="store_true", help="skip the per-config throughput table")
    p.add_argument("--no-separate", action="store_true",
                   help="time only the fused four-launch layer (counter passes: every GEMV dispatch is one "
                        "of the four launches the roofline is computed over)")
    p.add_argument("--gemm-iters", type=int, default=50)
    p.add_argument("--crossover-ms", default=None,
                   help="comma-separated M values for '--only crossover' (default: 1 ... 256)")
    return p.parse_args()


def stage_layer(torch, q, synth, M):
    """Seven linears of the decoder layer: packed weights, x and y on the GPU."""
    import numpy as np

    lins = []
    for sid in range(7):
        c = synth.make_case(1, sid, M, keep_codes=False)
        dev = "cuda:0"
        qw = torch.from_numpy(c.qweight.view(np.int32)).to(dev)
        qz = torch.from_numpy(c.qzeros.view(np.int32)).to(dev)
        sc = torch.from_numpy(c.scales.view(np.int16)).to(dev)
        packed = q.tf_repack_w4(qw, qz, sc, c.K, c.N, c.G)
        del qw, qz, sc
        x = torch.from_numpy(c.x.view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((M, c.N), dtype=torch.bfloat16, device=dev)
        lins.append(dict(name=c.name, sid=sid, K=c.K, N=c.N, G=c.G, M=M, packed=packed, x=x, y=y,
                         bytes=algorithmic_bytes(4, M, c.K, c.N, c.G)))
    torch.cuda.synchronize()
    return lins


def cpu_baseline(synth, oracle, M, budget_s=12.0):
    """The oracle, untuned, on the headline workload: whole passes over the
    seven linears (dequant + fp64 linear), as many as fit the time budget."""
    cases = [synth.make_case(1, sid, M, keep_codes=False) for sid in range(7)]
    total_bytes = sum(algorithmic_bytes(4, M, c.K, c.N, c.G) for c in cases)
    passes, t0 = 0, time.perf_counter()
    while True:
        for c in cases:
            oracle.awq_linear(c)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    cores = oracle.num_threads()
    # per core: the 4096 x 4096 linear (config 0) on one thread, about 2 s
    c0 = synth.make_case(0, 0, 1, keep_codes=False)
    c0_bytes = algorithmic_bytes(4, 1, c0.K, c0.N, c0.G)
    oracle.set_num_threads(1)
    try:
        n1, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < 2.0:
            oracle.awq_linear(c0)
            n1 += 1
        el1 = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(cores)
    return dict(value=round(passes * total_bytes / el / 1e9, 3), unit="GB/s", cores=cores,
                kind="oracle",
                sample=f"{passes} full pass(es) over the 7 layer linears at M=1 "
                       f"({passes * total_bytes / 1e6:.0f} MB of algorithmic bytes, {el:.1f} s)",
                per_core=dict(value=round(n1 * c0_bytes / el1 / 1e9, 4), unit="GB/s", cores=1,
                              sample=f"{n1} pass(es) of the 4096x4096 W4 linear at M=1 on one thread ({el1:.1f} s)"))


COPY_BYTES = 1 << 30


def bench_copy(torch):
    """Plain device copy of COPY_BYTES, five times: the calibration kernel whose
    FETCH_SIZE / WRITE_SIZE readings scale the GEMV's counters to bytes."""
    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    return dict(copy_bytes=COPY_BYTES, launches=5)


def _pmc_rows(path):
    """(kernel name, counter name, value) rows of a rocprofv3 counter CSV
    (a file, or a directory searched for *counter_collection.csv)."""
    import csv
    import glob

    files = [path] if os.path.isfile(path) else sorted(
        glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]), r.get("Dispatch_Id"),
                             int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0)))
    return rows


def _per_dispatch_kib(path, counter, match):
    """Mean over matching dispatches of one counter (summed over its
    instances within a dispatch), in the counter's own unit (KiB)."""
    per = {}
    for name, cname, v, did, grid in _pmc_rows(path):
        if cname == counter and match(name, grid):
            per[did] = per.get(did, 0.0) + v
    if not per:
        raise SystemExit(f"no {counter} dispatches matched in {path}")
    return sum(per.values()) / len(per), len(per)


def write_counters(dirs, kernel):
    """Per-launch HBM traffic of the dominant GEMV kernel (its dispatches in
    the layer step) from two --pmc passes, each scaled by the same counter's
    reading on the plain copy kernel."""
    fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    is_gemv = lambda n, grid: kernel in n
    is_copy = lambda n, grid: "copy" in n.lower() and "gemv" not in n
    f_kib, nf = _per_dispatch_kib(fetch_dir, "FETCH_SIZE", is_gemv)
    w_kib, nw = _per_dispatch_kib(write_dir, "WRITE_SIZE", is_gemv)
    cf_kib, _ = _per_dispatch_kib(cfetch_dir, "FETCH_SIZE", is_copy)
    cw_kib, _ = _per_dispatch_kib(cwrite_dir, "WRITE_SIZE", is_copy)
    fetch_scale = COPY_BYTES / (cf_kib * 1024)
    write_scale = COPY_BYTES / (cw_kib * 1024)
    hbm = f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale
    out = dict(kernel_source_hash=kernel_source_hash(), kernel_trace_name=kernel,
               kernel=f"{kernel} (tf_gemv_w4a16): its dispatches in the fused layer step",
               fetch_kib_per_launch=round(f_kib, 1), write_kib_per_launch=round(w_kib, 1),
               dispatches=dict(fetch=nf, write=nw),
               copy_calibration=dict(bytes=COPY_BYTES, fetch_kib=round(cf_kib, 1), write_kib=round(cw_kib, 1),
                                     fetch_scale=round(fetch_scale, 4), write_scale=round(write_scale, 4)),
               hbm_bytes_per_launch=round(hbm))
    with open(COUNTERS_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def _trace_us(path, match):
    """Mean duration (us) and count of the matching dispatches of a rocprofv3
    kernel trace (a file, or a directory searched for *kernel_trace.csv)."""
    import csv
    import glob

    files = [path] if os.path.isfile(path) else sorted(
        glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {path}")
    d = []
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                grid = int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0)
                if match(r["Kernel_Name"], grid):
                    d.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    if not d:
        raise SystemExit(f"no dispatch matched in {path}")
    return sum(d) / len(d), len(d)


def gemm_bench_shapes():
    """(M, K, N, G) of the two prefill shapes the GEMM leg times."""
    return [(2048, 4096, 14336, 128), (2048, 14336, 4096, 128)]


def gemm_grid_threads(q, M, K, N, G):
    """Threads in the 256 x 256 GEMM kernel's grid for a shape (its launch
    plan from tf_gemm_plan; no GPU needed)."""
    m_tiles, wide, narrow, splits, _, _, rows, col_tile = q.tf_gemm_plan(4, M, K, N, G, cus=256)
    if col_tile != 256:
        raise SystemExit(f"shape {M}x{K}x{N} does not run the 256 x 256 kernel")
    return m_tiles * wide * splits * 512


def write_gemm_counters(dirs):
    """MFMA busy, clock and HBM traffic per launch of the 256 x 256 GEMM
    kernel on each prefill shape, from a kernel trace and five --pmc passes
    (the traffic counters scaled by their readings on the plain copy kernel)."""
    import quantized_linear_layers_awq_amd as q

    trace_dir, busy_dir, fetch_dir, write_dir, cfetch_dir, cwrite_dir = dirs
    is_copy = lambda n, grid: "copy" in n.lower() and "gemm" not in n
    cf_kib, _ = _per_dispatch_kib(cfetch_dir, "FETCH_SIZE", is_copy)
    cw_kib, _ = _per_dispatch_kib(cwrite_dir, "WRITE_SIZE", is_copy)
    fetch_scale = COPY_BYTES / (cf_kib * 1024)
    write_scale = COPY_BYTES / (cw_kib * 1024)
    shapes = []
    for M, K, N, G in gemm_bench_shapes():
        threads = gemm_grid_threads(q, M, K, N, G)
        match = lambda n, grid, t=threads: GEMM_TRACE_NAME in n and grid == t
        us, n_trace = _trace_us(trace_dir, match)
        busy, nb = _per_dispatch_kib(busy_dir, "SQ_VALU_MFMA_BUSY_CYCLES", match)
        grbm, _ = _per_dispatch_kib(busy_dir, "GRBM_GUI_ACTIVE", match)
        f_kib, nf = _per_dispatch_kib(fetch_dir, "FETCH_SIZE", match)
        w_kib, nw = _per_dispatch_kib(write_dir, "WRITE_SIZE", match)
        simd_cycles = grbm / 8 * 1024  # GRBM_GUI_ACTIVE sums the 8 XCDs; 256 CUs x 4 SIMDs
        flops = 2.0 * M * K * N
        alg = 2 * M * K + algorithmic_bytes(4, 0, K, N, G) + 2 * M * N
        shapes.append(dict(M=M, K=K, N=N, G=G, grid_threads=threads, trace_us=round(us, 2),
                           trace_tflops=round(flops / (us * 1e-6) / 1e12, 1),
                           clock_ghz=round(grbm / 8 / (us * 1e3), 3), mfma_busy=round(busy / simd_cycles, 4),
                           fetch_kib_per_launch=round(f_kib, 1), write_kib_per_launch=round(w_kib, 1),
                           hbm_bytes_per_launch=round(f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale),
                           algorithmic_bytes=int(alg), dispatches=dict(trace=n_trace, busy=nb, fetch=nf, write=nw)))
    out = dict(kernel_source_hash=kernel_source_hash(GEMM_SOURCES), kernel_trace_name=GEMM_TRACE_NAME,
               kernel=f"{GEMM_TRACE_NAME} (tf_gemm_w4a16), M=2048 prefill shapes",
               shapes=shapes,
               copy_calibration=dict(bytes=COPY_BYTES, fetch_kib=round(cf_kib, 1), write_kib=round(cw_kib, 1),
                                     fetch_scale=round(fetch_scale, 4), write_scale=round(write_scale, 4)))
    with open(GEMM_COUNTERS_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def queue_filler(torch, ms):
    """Enqueue ~ms of GPU work so the launches queued after it run back to back."""
    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda:0")
    reps = max(1, int(ms / 0.6))
    for _ in range(reps):
        a = (a @ a).clamp_(-1, 1)
    return a


def fuse_layer(torch, q, lins):
    """The layer as serving engines lay it out: q, k, v fused into one N=6144
    projection and gate, up into one N=28672 projection (the same weights and
    bytes, four launches instead of seven).  The packed format is block-major
    with self-contained 16-column blocks, so the fused buffer is the
    concatenation of the per-linear buffers; that is checked here against a
    repack of the concatenated AWQ checkpoint."""
    import numpy as np

    import synth

    by = {l["name"].split("_")[2]: l for l in lins}
    groups = [("qkv", ["q", "k", "v"]), ("o", ["o"]), ("gate_up", ["gate", "up"]), ("down", ["down"])]
    fused = []
    for name, parts in groups:
        ls = [by[p] for p in parts]
        K, G, M = ls[0]["K"], ls[0]["G"], ls[0]["M"]
        N = sum(l["N"] for l in ls)
        packed = torch.cat([l["packed"] for l in ls]) if len(ls) > 1 else ls[0]["packed"]
        if len(ls) > 1 and name == "qkv":
            cs = [synth.make_case(1, l["sid"], M, keep_codes=False) for l in ls]
            dev = "cuda:0"
            qw = torch.from_numpy(np.concatenate([c.qweight for c in cs], axis=1).view(np.int32)).to(dev)
            qz = torch.from_numpy(np.concatenate([c.qzeros for c in cs], axis=1).view(np.int32)).to(dev)
            sc = torch.from_numpy(np.concatenate([c.scales for c in cs], axis=1).view(np.int16)).to(dev)
            assert torch.equal(q.tf_repack_w4(qw, qz, sc, K, N, G), packed), "fused repack differs from concatenation"
            del qw, qz, sc
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        fused.append(dict(name=name, K=K, N=N, G=G, M=M, packed=packed, x=ls[0]["x"], y=y,
                          bytes=algorithmic_bytes(4, M, K, N, G)))
    torch.cuda.synchronize()
    return fused


def time_graphs(torch, q, lins, args, R):
    """Graph replays of one pass over `lins`, rotating over R weight replicas;
    returns (ms per pass, eager ms per pass, per-launch mean us)."""
    replicas = [[l["packed"] for l in lins]]
    for _ in range(R - 1):
        replicas.append([p.clone() for p in replicas[0]])
    torch.cuda.synchronize()

    def layer_pass(r):
        for l, p in zip(lins, replicas[r]):
            q.tf_gemv_w4a16(l["x"], p, l["K"], l["N"], l["G"], y=l["y"])

    # eager reference results, then one graph per replica
    layer_pass(0)
    torch.cuda.synchronize()
    ref = [l["y"].clone() for l in lins]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(stream):
        for r in range(R):
            layer_pass(r)  # warm the capture stream before capturing
        torch.cuda.synchronize()
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                layer_pass(r)
            graphs.append(g)
    torch.cuda.synchronize()
    for r in range(R):
        graphs[r].replay()
        torch.cuda.synchronize()
        for l, y0 in zip(lins, ref):
            assert torch.equal(l["y"], y0), "graph replay differs from the eager result"

    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        graphs[i % R].replay()
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # eager step time for reference (host launch overhead included)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    n_eager = min(args.steps, 50)
    for i in range(n_eager):
        layer_pass(i % R)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - h0) * 1e3 / n_eager

    # per-linear launch time: a batch of eager launches of one linear queued
    # behind filler work (so they run back to back), one event pair per batch
    n_prof = min(args.steps, 40)
    keep = queue_filler(torch, ms=0.02 * n_prof * len(lins) + 5)
    evs = []
    for j, l in enumerate(lins):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n_prof):
            q.tf_gemv_w4a16(l["x"], replicas[i % R][j], l["K"], l["N"], l["G"], y=l["y"])
        e1.record()
        evs.append((e0, e1))
    torch.cuda.synchronize()
    del keep
    mean_us = [1e3 * e0.elapsed_time(e1) / n_prof for e0, e1 in evs]

    # the headline: K eager steps queued behind filler work, one event pair
    enq_us = host_us_per_step(layer_pass, R)
    queued_ms = time_queued(torch, lambda i: layer_pass(i % R), args.steps, enqueue_us=enq_us)
    for l, y0 in zip(lins, ref):
        assert torch.equal(l["y"], y0), "queued eager launches differ from the first result"
    # spread: the same queued steps with an event between consecutive steps
    step_pct = percentiles_us(time_queued_steps(torch, lambda i: layer_pass(i % R), args.steps, enq_us))

    # practical roof: a plain streaming read of the same packed buffers, one
    # launch per linear, in the same queued pattern
    sink = torch.zeros(4, dtype=torch.int32, device="cuda:0")

    def read_pass(r):
        for p in replicas[r]:
            q.tf_probe_stream_read(p, sink)

    read_ms = time_queued(torch, lambda i: read_pass(i % R), args.steps, enqueue_us=host_us_per_step(read_pass, R))

    # the GEMV's own code stream without its arithmetic (same blocks, waves,
    # ring depth and closing exchange), per launch and as a queued step
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    plans = [q.tf_gemv_plan(4, 1, l["K"], l["N"], l["G"], cus) for l in lins]

    def block_read(j, p):
        l, pl = lins[j], plans[j]
        q.tf_probe_block_read(4, p, l["K"], l["N"], l["G"], pl["waves"], pl["depth"], sink)

    def block_pass(r):
        for j, p in enumerate(replicas[r]):
            block_read(j, p)

    block_ms = time_queued(torch, lambda i: block_pass(i % R), args.steps,
                           enqueue_us=host_us_per_step(block_pass, R))
    keep = queue_filler(torch, ms=0.02 * n_prof * len(lins) * 2 + 5)
    evs = []
    for j in range(len(lins)):
        for probe in ("read", "block"):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(n_prof):
                if probe == "read":
                    q.tf_probe_stream_read(replicas[i % R][j], sink)
                else:
                    block_read(j, replicas[i % R][j])
            e1.record()
            evs.append((e0, e1))
    torch.cuda.synchronize()
    del keep
    probe_us = [1e3 * e0.elapsed_time(e1) / n_prof for e0, e1 in evs]
    del replicas, graphs
    return dict(graph_ms=ms_step, host_eager_ms=eager_ms, queued_ms=queued_ms, read_roof_ms=read_ms,
                block_read_ms=block_ms, mean_us=mean_us, read_us=probe_us[0::2], block_us=probe_us[1::2],
                step_pct_us=step_pct)


def host_us_per_step(step, R, n=20):
    """Host time to enqueue one step (for sizing the filler in front of a
    queued run)."""
    import torch

    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for i in range(n):
        step(i % R)
    us = (time.perf_counter() - h0) * 1e6 / n
    torch.cuda.synchronize()
    return us


def time_queued(torch, step, steps, enqueue_us):
    """ms per step of `steps` steps launched eagerly behind enough filler work
    that the host has enqueued them all before the GPU reaches them; HIP
    events on the launch stream bracket exactly the steps."""
    torch.cuda.synchronize()
    f0 = torch.cuda.Event(enable_timing=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    h0 = time.perf_counter()
    f0.record()
    keep = queue_filler(torch, ms=1.5 * steps * enqueue_us * 1e-3 + 2)
    e0.record()
    for i in range(steps):
        step(i)
    host_ms = (time.perf_counter() - h0) * 1e3
    e1.record()
    torch.cuda.synchronize()
    del keep
    ms = e0.elapsed_time(e1) / steps
    # the GPU reached the steps after the filler; if the host was still
    # enqueueing them then, the measurement includes host time (it can only
    # err high)
    filler_ms = f0.elapsed_time(e0)
    if host_ms > filler_ms:
        print(f"note: host enqueue ({host_ms:.2f} ms) outlasted the filler ({filler_ms:.2f} ms); the step time "
              f"may include host waits", file=sys.stderr)
    return ms


def percentiles_us(ms_list):
    """p10, p50 (median) and p90 of per-step times given in ms, in us."""
    import numpy as np

    a = np.asarray(ms_list) * 1e3
    return dict(p10=round(float(np.percentile(a, 10)), 3), p50=round(float(np.percentile(a, 50)), 3),
                p90=round(float(np.percentile(a, 90)), 3), n=int(a.size))


def time_queued_steps(torch, step, steps, enqueue_us):
    """Per-step times (ms) of `steps` steps queued as in time_queued, with a
    HIP event on the launch stream between consecutive steps.  The events
    add a little work of their own, so this gives the spread, while
    time_queued (one event pair) gives the mean."""
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    keep = queue_filler(torch, ms=1.5 * steps * enqueue_us * 1e-3 + 2)
    evs[0].record()
    for i in range(steps):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    del keep
    return [a.elapsed_time(b) for a, b in zip(evs[:-1], evs[1:])]


def bench_gemv(torch, q, args):
    import synth

    lins = stage_layer(torch, q, synth, M=1)
    layer_bytes = sum(l["bytes"] for l in lins)
    packed_bytes = sum(l["packed"].numel() for l in lins)
    R = args.replicas or max(2, -(-2 * INFINITY_CACHE_BYTES // packed_bytes) + 1)

    # headline: the fused four-launch layer; beside it the seven separate launches
    fused = fuse_layer(torch, q, lins)
    assert abs(sum(f["bytes"] for f in fused) - layer_bytes) < 2 * 2 * (4096 + 4096 + 14336), "fusion changed the bytes"
    tf_ = time_graphs(torch, q, fused, args, R)
    ms_f, us_f = tf_["queued_ms"], tf_["mean_us"]
    if not args.no_separate:
        ts_ = time_graphs(torch, q, lins, args, R)

    # The roofline's dominant kernel: launches are grouped by the kernel
    # instance they run (the GEMV kernel, its ring depth and blocks per
    # workgroup, from the library's plan), as a kernel trace's statistics
    # group them; the group with the most time per step is the dominant
    # kernel.  Its per-launch durations are the back-to-back batches of one
    # launch each, timed with HIP events on the launch stream (torch's
    # current stream, which the binding launches on).
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    groups = {}
    for f, us in zip(fused, us_f):
        pl = q.tf_gemv_plan(4, 1, f["K"], f["N"], f["G"], cus)
        key = (pl["kernel"], pl["depth"], pl["bpw"])
        g = groups.setdefault(key, dict(names=[], bytes=0.0, us=0.0, n=0))
        g["names"].append(f["name"])
        g["bytes"] += f["bytes"]
        g["us"] += us
        g["n"] += 1
    dom_key, dom = max(groups.items(), key=lambda kv: kv[1]["us"])
    avg_launch_us = dom["us"] / dom["n"]
    achieved = dom["bytes"] / (dom["us"] * 1e-6) / 1e9
    step_achieved = layer_bytes / (ms_f * 1e-3) / 1e9
    read_roof = layer_bytes / (tf_["read_roof_ms"] * 1e-3) / 1e9

    trace_name = GEMV_TRACE_NAME.format(depth=dom_key[1], bpw=dom_key[2])
    traffic = None
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE) as f:
            cnt = json.load(f)
        if cnt.get("kernel_source_hash") == kernel_source_hash() and cnt.get("kernel_trace_name") == trace_name:
            traffic = cnt.get("hbm_bytes_per_launch")

    def rows(ls, t):
        return [dict(name=l["name"].replace("c1_layer_", "").replace("_M1", ""), K=l["K"], N=l["N"],
                     us=round(u, 3), gbs=round(l["bytes"] / (u * 1e-6) / 1e9, 1),
                     read_probe_us=round(ru, 3), block_probe_us=round(bu, 3),
                     vs_read_probe=round(u / ru, 3), vs_block_probe=round(u / bu, 3))
                for l, u, ru, bu in zip(ls, t["mean_us"], t["read_us"], t["block_us"])]

    value = layer_bytes / (ms_f * 1e-3) / 1e9
    gbs = lambda ms: round(layer_bytes / (ms * 1e-3) / 1e9, 1)
    return dict(
        value=value, ms_step=ms_f, replicas=R, layer_bytes=layer_bytes,
        graph_ms=tf_["graph_ms"], graph_gbs=gbs(tf_["graph_ms"]), host_eager_ms=tf_["host_eager_ms"],
        step_pct_us=tf_["step_pct_us"],
        read_roof_gbs=round(read_roof, 1),
        block_probe_gbs=gbs(tf_["block_read_ms"]),
        per_launch=rows(fused, tf_),
        separate=None if args.no_separate else dict(
            ms_per_step=round(ts_["queued_ms"], 5), gbs=gbs(ts_["queued_ms"]),
            graph_ms_per_step=round(ts_["graph_ms"], 5), graph_gbs=gbs(ts_["graph_ms"]),
            per_linear=rows(lins, ts_)),
        roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                      kernel=f"{trace_name} ({' and '.join(dom['names'])} launches)",
                      launches=dom["names"],
                      bytes_per_launch=round(dom["bytes"] / dom["n"]),
                      avg_launch_us=round(avg_launch_us, 3),
                      step_average=dict(achieved=round(step_achieved, 1),
                                        frac=round(step_achieved / HBM_PEAK_GBS, 4),
                                        what="all four launches of the step: layer bytes over step time"),
                      measured_roof=round(read_roof, 1),
                      frac_of_measured_roof=round(step_achieved / read_roof, 4),
                      measured_roof_kind="plain streaming read of the same packed buffers, same queued launches "
                                         "(compared with the step average)"),
    )


def bench_gemm(torch, q, args):
    import numpy as np

    import synth

    shapes = []
    for sid in (0, 1):
        c = synth.make_case(3, sid, 2048, keep_codes=False)
        dev = "cuda:0"
        qw = torch.from_numpy(c.qweight.view(np.int32)).to(dev)
        qz = torch.from_numpy(c.qzeros.view(np.int32)).to(dev)
        sc = torch.from_numpy(c.scales.view(np.int16)).to(dev)
        packed = q.tf_repack_w4(qw, qz, sc, c.K, c.N, c.G)
        x = torch.from_numpy(c.x.view(np.int16)).to(dev).view(torch.bfloat16)
        y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
        shapes.append(dict(M=c.M, K=c.K, N=c.N, G=c.G, packed=packed, x=x, y=y))
    # the GPU's clock ramps up over the first tens of milliseconds of
    # sustained MFMA work (the first 20 launches run up to 25 % slower than
    # the later ones): warm up on both shapes for about 300 ms first
    import time as _time

    t_end = _time.perf_counter() + 0.3
    while _time.perf_counter() < t_end:
        for s in shapes:
            for _ in range(4):
                q.tf_gemm_w4a16(s["x"], s["packed"], s["K"], s["N"], s["G"], y=s["y"])
        torch.cuda.synchronize()
    out = []
    for s in shapes:
        # back-to-back launches between one event pair: throughput per launch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.gemm_iters):
            q.tf_gemm_w4a16(s["x"], s["packed"], s["K"], s["N"], s["G"], y=s["y"])
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / args.gemm_iters
        fl = 2.0 * s["M"] * s["K"] * s["N"]
        # spread: the same back-to-back launches with an event between them
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.gemm_iters + 1)]
        evs[0].record()
        for i in range(args.gemm_iters):
            q.tf_gemm_w4a16(s["x"], s["packed"], s["K"], s["N"], s["G"], y=s["y"])
            evs[i + 1].record()
        torch.cuda.synchronize()
        pct = percentiles_us([a.elapsed_time(b) for a, b in zip(evs[:-1], evs[1:])])
        out.append(dict(M=s["M"], K=s["K"], N=s["N"], us=round(us, 2), tflops=round(fl / (us * 1e-6) / 1e12, 1),
                        launch_pct_us=pct))
    tot_fl = sum(2.0 * o["M"] * o["K"] * o["N"] for o in out)
    tot_us = sum(o["us"] for o in out)
    tfs = tot_fl / (tot_us * 1e-6) / 1e12

    # the vendor library's dense bf16 GEMM (hipBLASLt through
    # torch.nn.functional.linear, weights [N][K] in bf16, nothing to
    # dequantize) on the same shapes, warmed up and timed the same way: what a
    # tuned dense kernel reaches on this GPU at its board power limit
    lib = []
    for s in shapes:
        w = torch.empty((s["N"], s["K"]), dtype=torch.bfloat16, device="cuda:0").normal_(0.0, 0.02)
        t_end = _time.perf_counter() + 0.3
        while _time.perf_counter() < t_end:
            for _ in range(4):
                torch.nn.functional.linear(s["x"], w)
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.gemm_iters):
            torch.nn.functional.linear(s["x"], w)
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / args.gemm_iters
        lib.append(dict(K=s["K"], N=s["N"], us=round(us, 2),
                        tflops=round(2.0 * s["M"] * s["K"] * s["N"] / (us * 1e-6) / 1e12, 1)))
        del w
    lib_tfs = tot_fl / (sum(o["us"] for o in lib) * 1e-6) / 1e12

    # practical roof: back-to-back bf16 MFMAs on every SIMD (two waves each),
    # sustained for about as long as the GEMM launches above
    props = torch.cuda.get_device_properties(0)
    wgs = props.multi_processor_count
    sink = torch.zeros(4, dtype=torch.float32, device="cuda:0")
    iters = 2000
    q.tf_probe_mfma(wgs, iters, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = max(1, int(tot_us * args.gemm_iters / 300.0))
    e0.record()
    fl = 0
    for _ in range(n):
        fl += q.tf_probe_mfma(wgs, iters, sink)
    e1.record()
    torch.cuda.synchronize()
    mfma_roof = fl / (e0.elapsed_time(e1) * 1e-3) / 1e12

    # counters of the same kernel build (MFMA busy, clock, HBM bytes per
    # launch), taken by rocprofv3 passes over this leg and stored with the
    # hash of the kernel's sources; unused once the sources have changed
    counters = None
    if os.path.exists(GEMM_COUNTERS_FILE):
        with open(GEMM_COUNTERS_FILE) as f:
            cnt = json.load(f)
        if cnt.get("kernel_source_hash") == kernel_source_hash(GEMM_SOURCES):
            counters = cnt
    traffic = mfma_busy = clock = None
    if counters:
        sh = counters["shapes"]
        traffic = round(sum(c["hbm_bytes_per_launch"] for c in sh) / len(sh))
        wsum = sum(c["trace_us"] for c in sh)
        mfma_busy = round(sum(c["mfma_busy"] * c["trace_us"] for c in sh) / wsum, 4)
        clock = round(sum(c["clock_ghz"] * c["trace_us"] for c in sh) / wsum, 3)
    return dict(
        metric="W4A16 GEMM M=2048 TFLOP/s", value=round(tfs, 1), unit="TFLOP/s",
        frac_of_peak=round(tfs / BF16_DENSE_PEAK_TFS, 4), shapes=out,
        roofline=dict(bound="mfma", achieved=round(tfs, 1), peak=BF16_DENSE_PEAK_TFS, unit="TFLOP/s",
                      frac=round(tfs / BF16_DENSE_PEAK_TFS, 4), traffic=traffic,
                      kernel="gemm256_kernel (tf_gemm_w4a16; per call, the split-K sum included)",
                      mfma_busy=mfma_busy, clock_ghz=clock,
                      counters=None if counters is None else dict(
                          source=os.path.relpath(GEMM_COUNTERS_FILE, ROOT),
                          what="time-weighted over both shapes; traffic = mean HBM bytes per launch of the kernel",
                          shapes=[dict(K=c["K"], N=c["N"], trace_us=c["trace_us"], mfma_busy=c["mfma_busy"],
                                       clock_ghz=c["clock_ghz"], hbm_bytes_per_launch=c["hbm_bytes_per_launch"],
                                       algorithmic_bytes=c["algorithmic_bytes"]) for c in counters["shapes"]]),
                      measured_roof=round(mfma_roof, 1), frac_of_measured_roof=round(tfs / mfma_roof, 4),
                      measured_roof_kind="back-to-back bf16 32x32x16 MFMAs, 8 waves per CU, sustained "
                                         "as long as the GEMM launches",
                      library_dense_bf16=dict(
                          value=round(lib_tfs, 1), unit="TFLOP/s", frac_of_library=round(tfs / lib_tfs, 4),
                          shapes=lib,
                          what="hipBLASLt dense bf16 GEMM (torch.nn.functional.linear, weights [N][K] bf16, no "
                               "dequantization) on the same shapes, warmed up and timed the same way")),
    )


def bench_configs(torch, q, args):
    """Throughput of every workload configuration at every M it names: GEMV
    launches queued back to back over weight replicas larger than twice the
    Infinity Cache (GB/s of algorithmic bytes), GEMM launches back to back
    (TFLOP/s).  Weights are the seeded synthetic ones; x for a second M of
    the same weights is drawn on the GPU (timing does not depend on it)."""
    import numpy as np

    import synth

    dev = "cuda:0"
    out = []
    for cfg in sorted(synth.CONFIGS):
        spec = synth.CONFIGS[cfg]
        if cfg == 1:
            for M in spec["Ms"]:
                lins = stage_layer(torch, q, synth, M=M)
                fused = fuse_layer(torch, q, lins)
                lb = sum(l["bytes"] for l in lins)
                R = max(2, -(-2 * INFINITY_CACHE_BYTES // sum(f["packed"].numel() for f in fused)) + 1)
                reps = [[f["packed"] for f in fused]] + [[f["packed"].clone() for f in fused] for _ in range(R - 1)]

                def step(i, fused=fused, reps=reps, R=R):
                    for f, p in zip(fused, reps[i % R]):
                        q.tf_gemv_w4a16(f["x"], p, f["K"], f["N"], f["G"], y=f["y"])

                step(0)
                ms = time_queued(torch, step, 100, enqueue_us=host_us_per_step(lambda r: step(r), R))
                out.append(dict(config=cfg, kernel="gemv", bits=4, M=M, shape="decoder layer, 4 launches", G=128,
                                us=round(ms * 1e3, 2), gbs=round(lb / (ms * 1e-3) / 1e9, 1),
                                frac_of_hbm_peak=round(lb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)))
                del lins, fused, reps
            continue
        if cfg == 3:
            continue  # the GEMM leg of the line
        for sid, (name, bits, K, N, G) in enumerate(spec["shapes"]):
            c = synth.make_case(cfg, sid, 1, keep_codes=False)
            qw = torch.from_numpy(c.qweight.view(np.int32) if bits == 4 else c.qweight).to(dev)
            qz = torch.from_numpy(c.qzeros.view(np.int32) if bits == 4 else c.qzeros).to(dev)
            sc = torch.from_numpy(c.scales.view(np.int16)).to(dev)
            repack = q.tf_repack_w4 if bits == 4 else q.tf_repack_w8
            packed = repack(qw, qz, sc, K, N, G)
            del qw, qz, sc, c
            gemv = q.tf_gemv_w4a16 if bits == 4 else q.tf_gemv_w8a16
            gemm = q.tf_gemm_w4a16 if bits == 4 else q.tf_gemm_w8a16
            for M in spec["Ms"]:
                x = torch.randn((M, K), device=dev).to(torch.bfloat16)
                y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                if M <= 16:
                    R = max(2, -(-2 * INFINITY_CACHE_BYTES // packed.numel()) + 1)
                    reps = [packed] + [packed.clone() for _ in range(R - 1)]

                    def step(i, reps=reps, R=R, x=x, y=y, K=K, N=N, G=G, gemv=gemv):
                        gemv(x, reps[i % R], K, N, G, y=y)

                    step(0)
                    ms = time_queued(torch, step, 100, enqueue_us=host_us_per_step(lambda r: step(r), R))
                    b = algorithmic_bytes(bits, M, K, N, G)
                    out.append(dict(config=cfg, kernel="gemv", bits=bits, M=M, shape=f"{K}x{N}", G=G,
                                    us=round(ms * 1e3, 2), gbs=round(b / (ms * 1e-3) / 1e9, 1),
                                    frac_of_hbm_peak=round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)))
                    del reps
                else:
                    for _ in range(2):
                        gemm(x, packed, K, N, G, y=y)
                    torch.cuda.synchronize()
                    n = max(3, min(args.gemm_iters, int(2e-2 / (2.0 * M * K * N / 1e15))))
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(n):
                        gemm(x, packed, K, N, G, y=y)
                    e1.record()
                    torch.cuda.synchronize()
                    us = 1e3 * e0.elapsed_time(e1) / n
                    tfs = 2.0 * M * K * N / (us * 1e-6) / 1e12
                    out.append(dict(config=cfg, kernel="gemm", bits=bits, M=M, shape=f"{K}x{N}", G=G,
                                    us=round(us, 2), tflops=round(tfs, 1),
                                    frac_of_peak=round(tfs / BF16_DENSE_PEAK_TFS, 4)))
                del x, y
            del packed
            torch.cuda.empty_cache()
    return out


CROSSOVER_MS = (1, 2, 4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256)


def bench_crossover(torch, q, args):
    """GEMV against GEMM on the decoder layer (four fused launches, W4, group
    128) at M = 1 ... 256: microseconds per layer pass for each entry point
    that accepts the M (tf_gemm as routed, and up to M = 64 also forced onto
    the tiled GEMM), queued back to back over weight replicas larger than
    twice the Infinity Cache, and which is fastest."""
    import synth

    lins = stage_layer(torch, q, synth, M=1)
    fused = fuse_layer(torch, q, lins)
    del lins
    R = max(2, -(-2 * INFINITY_CACHE_BYTES // sum(f["packed"].numel() for f in fused)) + 1)
    reps = [[f["packed"] for f in fused]] + [[f["packed"].clone() for f in fused] for _ in range(R - 1)]
    flops1 = sum(2.0 * f["K"] * f["N"] for f in fused)
    out = []
    ms_list = [int(v) for v in args.crossover_ms.split(",")] if args.crossover_ms else CROSSOVER_MS
    for M in ms_list:
        xs = [torch.randn((M, f["K"]), device="cuda:0").to(torch.bfloat16) for f in fused]
        ys = [torch.empty((M, f["N"]), dtype=torch.bfloat16, device="cuda:0") for f in fused]
        lb = sum(algorithmic_bytes(4, M, f["K"], f["N"], f["G"]) for f in fused)
        row = dict(M=M, layer_bytes=int(lb))
        cus = torch.cuda.get_device_properties(0).multi_processor_count

        def tiled(x, p, K, N, G, y):  # the same GEMM call forced onto the tiled GEMM
            return q.tf_linear_planned(4, q.TF_OP_GEMM, x, p, K, N, G, cus, q.TF_ROUTE_TILED, y=y)

        kernels = [("gemv", q.tf_gemv_w4a16)] if M <= 16 else []
        kernels.append(("gemm", q.tf_gemm_w4a16))
        if M <= 64:  # the GEMM call runs the GEMV kernel; the tiled GEMM beside it
            kernels.append(("gemm_tiled", tiled))
        for name, fn in kernels:
            def step(i, fn=fn, xs=xs, ys=ys):
                for f, p, x, y in zip(fused, reps[i % R], xs, ys):
                    fn(x, p, f["K"], f["N"], f["G"], y=y)

            step(0)
            ms = time_queued(torch, step, 40, enqueue_us=host_us_per_step(step, R))
            row[name] = dict(us=round(ms * 1e3, 2), gbs=round(lb / (ms * 1e-3) / 1e9, 1),
                             tflops=round(flops1 * M / (ms * 1e-3) / 1e12, 1))
        row["faster"] = min((k for k in ("gemv", "gemm", "gemm_tiled") if k in row), key=lambda k: row[k]["us"])
        out.append(row)
        del xs, ys
    del reps, fused
    torch.cuda.empty_cache()
    return out


def bench_silu(torch, q, args):
    """The decoder layer's fused gate/up projection (W4, K = 4096, N = 2 x
    14336, group 128) followed by silu(gate) * up, at M = 1 ... 16: the GEMV
    then torch's silu and multiply (three launches) against the GEMV with the
    product in its epilogue (one launch), queued back to back over weight
    replicas larger than twice the Infinity Cache; then the same at 2048 rows
    with the GEMM, launched back to back; microseconds per call."""
    import numpy as np

    import synth

    # the layer's gate and up checkpoints side by side, packed both ways: plain
    # (for the GEMV) and with the halves interleaved (for the fused call)
    cs = [synth.make_case(1, sid, 1, keep_codes=False) for sid in (4, 5)]
    assert [c.name.split("_")[2] for c in cs] == ["gate", "up"]
    K, G, N = cs[0].K, cs[0].G, cs[0].N + cs[1].N
    n2 = N // 2
    dev = "cuda:0"
    qw = torch.from_numpy(np.concatenate([c.qweight for c in cs], axis=1).view(np.int32)).to(dev)
    qz = torch.from_numpy(np.concatenate([c.qzeros for c in cs], axis=1).view(np.int32)).to(dev)
    sc = torch.from_numpy(np.concatenate([c.scales for c in cs], axis=1).view(np.int16)).to(dev)
    plain = q.tf_repack_w4(qw, qz, sc, K, N, G)
    paired = q.tf_repack_w4_gate_up(qw, qz, sc, K, N, G)
    del qw, qz, sc, cs
    R = max(2, -(-2 * INFINITY_CACHE_BYTES // plain.numel()) + 1)
    reps = [plain] + [plain.clone() for _ in range(R - 1)]
    preps = [paired] + [paired.clone() for _ in range(R - 1)]
    F = torch.nn.functional
    out = []
    for M in (1, 4, 8, 16):
        x = torch.randn((M, K), device="cuda:0").to(torch.bfloat16)
        yg = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
        o = torch.empty((M, n2), dtype=torch.bfloat16, device="cuda:0")

        def unfused(i):
            q.tf_gemv_w4a16(x, reps[i % R], K, N, G, y=yg)
            torch.mul(F.silu(yg[:, :n2]), yg[:, n2:], out=o)

        def fused(i):
            q.tf_gemv_w4a16_silu_mul(x, preps[i % R], K, N, G, y=o)

        row = dict(M=M)
        for name, step in (("gemv_then_torch_silu_mul", unfused), ("fused_epilogue", fused)):
            step(0)
            ms = time_queued(torch, step, 60, enqueue_us=host_us_per_step(step, R))
            row[name] = dict(us=round(ms * 1e3, 2),
                             gbs=round(algorithmic_bytes(4, M, K, N, G) / (ms * 1e-3) / 1e9, 1))
        out.append(row)
        del x, yg, o
    # prefill: 2048 rows, launches back to back (MFMA-bound, no replicas needed)
    M = 2048
    x = torch.randn((M, K), device="cuda:0").to(torch.bfloat16)
    yg = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    o = torch.empty((M, n2), dtype=torch.bfloat16, device="cuda:0")
    steps = (("gemm_then_torch_silu_mul", lambda: (q.tf_gemm_w4a16(x, plain, K, N, G, y=yg),
                                                   torch.mul(F.silu(yg[:, :n2]), yg[:, n2:], out=o))),
             ("fused_epilogue", lambda: q.tf_gemm_w4a16_silu_mul(x, paired, K, N, G, y=o)))
    row = dict(M=M)
    for name, step in steps:
        for _ in range(3):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            step()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / 10 * 1e3
        row[name] = dict(us=round(us, 2), tflops=round(2.0 * M * K * N / (us * 1e-6) / 1e12, 1))
    out.append(row)
    del x, yg, o, reps, preps, plain, paired
    torch.cuda.empty_cache()
    return out


def bench_energy(torch, q, args, seconds=1.0, max_seconds=8.0):
    """Energy per call from the GPU's energy accumulator (amdsmi), read around
    about `seconds` of calls that keep the GPU busy the whole window: the
    decoder layer's GEMV pass at M=1 as HIP-graph replays of 32 passes each
    (over weight replicas larger than twice the Infinity Cache; eager
    launches from the host would leave the GPU idle between them), and the
    prefill GEMM at M=2048 launched back to back, and for scale the vendor
    library's dense bf16 GEMM of that shape.  HIP events around the
    window give the GPU-busy fraction.  Beside them the idle draw over the
    same time.  Each window lasts at least `seconds` and at least four
    updates of the accumulator (at most `max_seconds`); the figures are board
    energy, idle included."""
    try:
        import amdsmi

        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as exc:  # no SMI access on this machine
        return dict(available=False, reason=f"{type(exc).__name__}: {exc}")

    import synth

    def joules():
        e = amdsmi.amdsmi_get_energy_count(handle)
        return e["energy_accumulator"] * e["counter_resolution"] * 1e-6

    try:  # the board power limit, in microwatts
        cap_w = round(amdsmi.amdsmi_get_power_cap_info(handle)["power_cap"] * 1e-6, 1)
    except Exception:
        cap_w = None

    def clock_mhz():
        try:
            return amdsmi.amdsmi_get_clock_info(handle, amdsmi.AmdSmiClkType.GFX)["clk"]
        except Exception:
            return None

    def sample(edges):
        """Append (time, energy) when the accumulator has moved since the last edge."""
        j = joules()
        if j != edges[-1][1]:
            edges.append((time.perf_counter(), j))

    def edge_watts(edges, t0, t1, j0, j1):
        """Power between the first and the last accumulator update seen, and
        the number of intervals left out.  The accumulator moves in steps
        (about once a millisecond on some boards, about once a second on
        others), so the two end readings of a window can each lag by a whole
        step; between update edges the energy is exact up to the sampling
        interval.  An interval between successive updates whose power is
        negative or above three times the board limit comes from a bad
        reading (one such reading spoils the intervals on both sides of it)
        and is left out of both sums."""
        ups = edges[1:]
        limit = 3.0 * (cap_w or 1400.0)
        good, dropped = [], 0
        for (ta, ja), (tb, jb) in zip(ups, ups[1:]):
            if tb > ta and 0.0 <= (jb - ja) / (tb - ta) <= limit:
                good.append((jb - ja, tb - ta))
            else:
                dropped += 1
        if good:
            return sum(g[0] for g in good) / sum(g[1] for g in good), dropped
        return (j1 - j0) / (t1 - t0), dropped

    def enough(edges, t0):
        elapsed = time.perf_counter() - t0
        return (elapsed >= seconds and len(edges) >= 5) or elapsed >= max_seconds

    def window(run_one, calls_per_run, gpu_ms_per_run):
        run_one(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 0.3:  # settle the clocks
            run_one(n)
            n += 1
        torch.cuda.synchronize()
        # keep about 20 ms of work queued: the host never lets the GPU drain
        ahead = max(2, int(20.0 / gpu_ms_per_run))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        marks, clocks = [], []
        j0, t0 = joules(), time.perf_counter()
        edges = [(t0, j0)]
        t_poll = t0
        e0.record()
        n = 0
        # run until `seconds` have passed and four accumulator updates were
        # seen, so that the power comes from whole update periods
        while not enough(edges, t0):
            run_one(n)
            n += 1
            ev = torch.cuda.Event()
            ev.record()
            marks.append(ev)
            if len(marks) > ahead:
                marks.pop(0).synchronize()
            if time.perf_counter() - t_poll > 0.002:  # energy every 2 ms, clock beside it
                t_poll = time.perf_counter()
                sample(edges)
                if len(clocks) < 4000:
                    mhz = clock_mhz()
                    if mhz is not None:
                        clocks.append(mhz)
        e1.record()
        torch.cuda.synchronize()
        j1, t1 = joules(), time.perf_counter()
        calls = n * calls_per_run
        busy = e0.elapsed_time(e1) * 1e-3 / (t1 - t0)
        watts, dropped = edge_watts(edges, t0, t1, j0, j1)
        joules_window = watts * (t1 - t0)
        return dict(calls=calls, seconds=round(t1 - t0, 3), joules=round(joules_window, 3),
                    watts=round(watts, 1), mj_per_call=round(joules_window / calls * 1e3, 4),
                    energy_updates=len(edges) - 1, intervals_dropped=dropped, gpu_busy_frac=round(min(busy, 1.0), 3),
                    gfx_clock_mhz_median=float(sorted(clocks)[len(clocks) // 2]) if clocks else None)

    torch.cuda.synchronize()
    j0, t0 = joules(), time.perf_counter()
    edges = [(t0, j0)]
    while not enough(edges, t0):
        time.sleep(0.002)
        sample(edges)
    idle_w, _ = edge_watts(edges, t0, time.perf_counter(), j0, joules())

    lins = stage_layer(torch, q, synth, M=1)
    fused = fuse_layer(torch, q, lins)
    del lins
    R = max(2, -(-2 * INFINITY_CACHE_BYTES // sum(f["packed"].numel() for f in fused)) + 1)
    reps = [[f["packed"] for f in fused]] + [[f["packed"].clone() for f in fused] for _ in range(R - 1)]
    passes = 32

    def layer_pass(i):
        for f, p in zip(fused, reps[i % R]):
            q.tf_gemv_w4a16(f["x"], p, f["K"], f["N"], f["G"], y=f["y"])

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        layer_pass(0)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(passes):
                layer_pass(i)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph.replay()
    g0.record()
    graph.replay()
    g1.record()
    torch.cuda.synchronize()
    gemv = window(lambda i: graph.replay(), passes, g0.elapsed_time(g1))
    gemv.update(kernel="gemv W4A16 M=1, decoder layer pass (four launches), HIP-graph replays of "
                       f"{passes} passes", unit="mJ per layer pass")
    del reps, fused, graph

    c = synth.make_case(3, 0, 2048, keep_codes=False)
    import numpy as np

    dev = "cuda:0"
    packed = q.tf_repack_w4(torch.from_numpy(c.qweight.view(np.int32)).to(dev),
                            torch.from_numpy(c.qzeros.view(np.int32)).to(dev),
                            torch.from_numpy(c.scales.view(np.int16)).to(dev), c.K, c.N, c.G)
    x = torch.from_numpy(c.x.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.empty((c.M, c.N), dtype=torch.bfloat16, device=dev)
    gemm = window(lambda i: q.tf_gemm_w4a16(x, packed, c.K, c.N, c.G, y=y), 1, 0.3)
    gemm.update(kernel=f"gemm W4A16 M={c.M} K={c.K} N={c.N}", unit="mJ per GEMM call",
                tflop_per_joule=round(2.0 * c.M * c.K * c.N * gemm["calls"] / 1e12 / gemm["joules"], 3))
    # the same shape as a dense bf16 GEMM in the vendor library, for scale
    del packed
    w = torch.empty((c.N, c.K), dtype=torch.bfloat16, device=dev).normal_(0.0, 0.02)
    lib = window(lambda i: torch.nn.functional.linear(x, w), 1, 0.3)
    lib.update(kernel=f"hipBLASLt dense bf16 GEMM (torch.nn.functional.linear) M={c.M} K={c.K} N={c.N}",
               unit="mJ per GEMM call",
               tflop_per_joule=round(2.0 * c.M * c.K * c.N * lib["calls"] / 1e12 / lib["joules"], 3))
    del w
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:
        pass
    return dict(available=True, idle_watts=round(idle_w, 1), power_cap_watts=cap_w, gemv=gemv, gemm=gemm,
                library_dense_bf16_gemm=lib,
                note="board energy from the amdsmi accumulator, idle draw included")


def main():
    args = parse()
    if args.counters_from:
        write_counters(args.counters_from, args.counters_kernel)
        return
    if args.gemm_counters_from:
        write_gemm_counters(args.gemm_counters_from)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import quantized_linear_layers_awq_amd as q

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(1)
    q.load_library()
    torch.cuda.set_device(0)
    if args.only == "copy":
        print(json.dumps(bench_copy(torch)), flush=True)
        return

    line = {
        "metric": "W4A16 GEMV M=1 effective HBM GB/s; W4A16 GEMM M=2048 TFLOP/s (% of peak)",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "W4A16 GEMV, M=1, one Llama-style decoder layer (q/o 4096x4096, k/v 4096x1024, "
                               "gate/up 4096x14336, down 14336x4096), group 128; q/k/v fused into one N=6144 "
                               "launch and gate/up into one N=28672 launch (four launches per step), launched "
                               "back to back on one stream, weights rotating over replicas larger than twice the "
                               "Infinity Cache",
                   "global_batch": 1, "parallelism": "none (1 GPU)"},
    }
    if args.only in ("all", "gemv"):
        gv = bench_gemv(torch, q, args)
        line["value"] = round(gv["value"], 1)
        line["ms_per_step"] = round(gv["ms_step"], 5)
        line["config"].update(replicas=gv["replicas"], layer_bytes=int(gv["layer_bytes"]))
        line["roofline"] = gv["roofline"]
        line["gemv_detail"] = dict(per_launch=gv["per_launch"],
                                   frac_of_hbm_peak=round(gv["value"] / HBM_PEAK_GBS, 4),
                                   read_roof_gbs=gv["read_roof_gbs"],
                                   frac_of_read_roof=round(gv["value"] / gv["read_roof_gbs"], 4),
                                   block_probe_gbs=gv["block_probe_gbs"],
                                   frac_of_block_probe=round(gv["value"] / gv["block_probe_gbs"], 4),
                                   graph_replay=dict(ms_per_step=round(gv["graph_ms"], 5), gbs=gv["graph_gbs"]),
                                   host_eager_ms_per_step=round(gv["host_eager_ms"], 4),
                                   step_percentiles_us=gv["step_pct_us"],
                                   seven_separate_launches=gv["separate"])
    if args.only in ("all", "gemm"):
        line["gemm"] = bench_gemm(torch, q, args)
    if args.only == "configs" or (args.only == "all" and not args.no_configs):
        line["configs"] = bench_configs(torch, q, args)
    if args.only == "crossover":
        line["crossover"] = bench_crossover(torch, q, args)
    if args.only == "energy" or (args.only == "all" and not args.no_energy):
        line["energy"] = bench_energy(torch, q, args)
    if args.only == "silu":
        line["silu_mul"] = bench_silu(torch, q, args)
    if args.only == "all" and not args.no_cpu:
        import oracle
        import synth

        line["cpu_baseline"] = cpu_baseline(synth, oracle, M=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
