"""The five workloads at full size, in the launch configuration the benchmark
times (same plans, same kernels).

GEMV outputs (M <= 8) are compared element by element over the whole output:
every column of every row, so every workgroup's 16-column block is checked.
GEMM outputs (M = 512, 2048, 4096) are compared over every column of a row
sample that holds the first and last row of every 256-row tile plus a seeded
draw, so every output tile is checked on its edge rows.  The row rms in the
bound is the full row's (all columns are compared).

The headline step runs q/k/v as one N = 6144 launch and gate/up as one
N = 28672 launch over concatenated packed buffers; those launches are
checked here too, and the concatenation is checked byte for byte against the
oracle's repack of the concatenated checkpoint."""

import dataclasses

import numpy as np
import pytest

import oracle
import synth
from gpu_harness import bf16_to_f64, check_linear, gpu_or_skip, linear_fn, sample_indices, to_device, within_tolerance

pytestmark = pytest.mark.gpu


def tile_edge_rows(M, extra=16, tile=256):
    """First and last row of every `tile`-row tile, plus `extra` seeded rows."""
    edges = {r for t in range(0, M, tile) for r in (t, min(t + tile, M) - 1)}
    return np.array(sorted(edges | set(sample_indices(M, extra, seed=M).tolist())))


def _run(config, shape_id, M, gemm, rows=None):
    torch, q = gpu_or_skip()
    c = synth.make_case(config, shape_id, M, keep_codes=False)
    print(f"config {c.name} gemm={gemm} rows={'all' if rows is None else len(rows)} cols=all", flush=True)
    ok, ratio, _ = check_linear(c, torch, q, gemm, rows=rows)
    assert ok, f"{c.name}: worst error / bound = {ratio:.3f}"
    return ratio


def test_c0_gemv_full_output():
    _run(0, 0, 1, gemm=False)


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("shape_id", range(7))
def test_c1_layer_gemv(shape_id, M):
    _run(1, shape_id, M, gemm=False)


FUSED = {"qkv": (0, 1, 2), "gate_up": (4, 5)}


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("name", list(FUSED))
def test_c1_fused_headline_launch(name, M):
    """One launch over the concatenation of the parts' packed buffers (the
    layout the benchmark step uses): every output element against each part's
    oracle on the shared activations, and the concatenated buffer against the
    oracle's repack of the concatenated checkpoint."""
    torch, q = gpu_or_skip()
    parts = [synth.make_case(1, sid, M, keep_codes=False) for sid in FUSED[name]]
    x = parts[0].x
    parts = [dataclasses.replace(c, x=x) for c in parts]
    K, G = parts[0].K, parts[0].G
    N = sum(c.N for c in parts)
    print(f"fused {name} M={M} K={K} N={N}", flush=True)
    packed = torch.cat([q.tf_repack_w4(*(to_device(c, torch)[k] for k in ("qweight", "qzeros", "scales")),
                                       c.K, c.N, c.G) for c in parts])
    want = oracle.repack(4, np.concatenate([c.qweight for c in parts], axis=1),
                         np.concatenate([c.qzeros for c in parts], axis=1),
                         np.concatenate([c.scales for c in parts], axis=1), K, N, G)
    assert np.array_equal(packed.cpu().numpy(), want)
    xd = to_device(parts[0], torch)["x"]
    y = bf16_to_f64(linear_fn(q, 4, False)(xd, packed, K, N, G))
    ref = np.concatenate([oracle.awq_linear(c) for c in parts], axis=1)
    # the bound uses each part's own row rms: the parts are separate linears
    c0 = 0
    for c in parts:
        ok, ratio = within_tolerance(y[:, c0:c0 + c.N], ref[:, c0:c0 + c.N])
        assert ok, f"{name} part at column {c0}: worst error / bound = {ratio:.3f}"
        c0 += c.N


@pytest.mark.parametrize("M", [1, 8])
def test_c2_w8_gemv(M):
    _run(2, 0, M, gemm=False)


def test_c2_w8_gemm_m512():
    _run(2, 0, 512, gemm=True, rows=tile_edge_rows(512))


@pytest.mark.parametrize("shape_id", [0, 1])
def test_c3_prefill_gemm(shape_id):
    _run(3, shape_id, 2048, gemm=True, rows=tile_edge_rows(2048))


@pytest.mark.parametrize("shape_id", [0, 1])
def test_c4_large_gemv(shape_id):
    _run(4, shape_id, 1, gemm=False)


@pytest.mark.parametrize("shape_id", [0, 1])
def test_c4_large_gemm(shape_id):
    _run(4, shape_id, 4096, gemm=True, rows=tile_edge_rows(4096, extra=8))
