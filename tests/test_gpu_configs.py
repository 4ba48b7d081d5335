"""The five workloads at full size, in the launch configuration the benchmark
times (same plans, same kernels).  Large outputs are compared on sampled rows
and columns that the oracle computes one by one; the row rms in the bound is
then taken over the sampled columns (columns are i.i.d., so it estimates the
full-row rms).  Edges are always sampled (first and last row and column)."""

import numpy as np
import pytest

import synth
from gpu_harness import check_linear, gpu_or_skip, sample_indices

pytestmark = pytest.mark.gpu


def _run(config, shape_id, M, gemm, n_rows=None, n_cols=None):
    torch, q = gpu_or_skip()
    c = synth.make_case(config, shape_id, M, keep_codes=False)
    print(f"config {c.name} gemm={gemm}", flush=True)
    rows = None if n_rows is None else sample_indices(c.M, n_rows, seed=M)
    cols = None if n_cols is None else sample_indices(c.N, n_cols, seed=c.N)
    ok, ratio, _ = check_linear(c, torch, q, gemm, rows=rows, cols=cols)
    assert ok, f"{c.name}: worst error / bound = {ratio:.3f}"
    return ratio


def test_c0_gemv_full_output():
    _run(0, 0, 1, gemm=False)


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("shape_id", range(7))
def test_c1_layer_gemv(shape_id, M):
    _run(1, shape_id, M, gemm=False, n_cols=1024)


@pytest.mark.parametrize("M", [1, 8])
def test_c2_w8_gemv(M):
    _run(2, 0, M, gemm=False, n_cols=1024)


def test_c2_w8_gemm_m512():
    _run(2, 0, 512, gemm=True, n_rows=64, n_cols=512)


@pytest.mark.parametrize("shape_id", [0, 1])
def test_c3_prefill_gemm(shape_id):
    _run(3, shape_id, 2048, gemm=True, n_rows=64, n_cols=512)


@pytest.mark.parametrize("shape_id", [0, 1])
def test_c4_large_gemv(shape_id):
    _run(4, shape_id, 1, gemm=False, n_cols=1024)


@pytest.mark.parametrize("shape_id", [0, 1])
def test_c4_large_gemm(shape_id):
    _run(4, shape_id, 4096, gemm=True, n_rows=32, n_cols=256)
