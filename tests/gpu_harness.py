"""Helpers of the GPU parity tests: move a synth.Case to the device, run the
HIP path through the binding, and compare with the oracle.

Tolerance (fp32 accumulation, bf16 or fp16 output):
    |y - y_ref| <= 1e-2 * max(|y_ref|, rms(y_ref row))  for every element.
A case whose dtype is "f16" (fp16 x and scales) runs the *_f16 entry points.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle


def gpu_or_skip():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import quantized_linear_layers_awq_amd as q

    q.load_library()  # raises when the HIP library is missing: no silent fallback
    return torch, q


def to_device(case, torch, dev="cuda:0"):
    qw = case.qweight.view(np.int32) if case.bits == 4 else case.qweight
    qz = case.qzeros.view(np.int32) if case.bits == 4 else case.qzeros
    return dict(
        qweight=torch.from_numpy(np.ascontiguousarray(qw)).to(dev),
        qzeros=torch.from_numpy(np.ascontiguousarray(qz)).to(dev),
        scales=torch.from_numpy(case.scales.view(np.int16)).to(dev),
        x=torch.from_numpy(case.x.view(np.int16)).to(dev).view(
            torch.float16 if getattr(case, "dtype", "bf16") == "f16" else torch.bfloat16),
    )


def repack(case, d, q):
    fn = q.tf_repack_w4 if case.bits == 4 else q.tf_repack_w8
    return fn(d["qweight"], d["qzeros"], d["scales"], case.K, case.N, case.G)


def linear_fn(q, bits, gemm):
    return {(4, False): q.tf_gemv_w4a16, (8, False): q.tf_gemv_w8a16,
            (4, True): q.tf_gemm_w4a16, (8, True): q.tf_gemm_w8a16}[(bits, gemm)]


def bf16_to_f64(t):
    """bf16 or fp16 device tensor -> float64 numpy (exact)."""
    return t.float().cpu().numpy().astype(np.float64)


def bf16_bits(t):
    """bf16 device tensor -> uint16 bit patterns (numpy)."""
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def within_tolerance(y, ref, rms=None):
    """Elementwise bound; returns (ok, worst ratio of error to its bound)."""
    if rms is None:
        rms = np.sqrt(np.mean(ref**2, axis=1, keepdims=True))
    bound = 1e-2 * np.maximum(np.abs(ref), rms)
    err = np.abs(y - ref)
    ratio = float(np.max(err / np.where(bound > 0, bound, np.inf))) if err.size else 0.0
    ok = bool(np.all(err <= bound))
    return ok, ratio


def sample_indices(n, count, seed):
    if n <= count:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(n, size=count, replace=False))
    # always include both ends (first tile, ragged last tile)
    return np.unique(np.concatenate([[0, n - 1], idx]))


def device_cus(torch):
    return torch.cuda.get_device_properties(0).multi_processor_count


def run_linear(q, bits, op, x, packed, K, N, G, cus=0, route=0, y=None, torch=None):
    """One call of the linear op (q.TF_OP_*) through the C ABI: the product
    entry point when cus == 0 and route == 0 (automatic), else
    tf_linear_planned with those plan inputs (cus 0: the device's count)."""
    if cus == 0 and route == 0:
        fn = {q.TF_OP_GEMV: linear_fn(q, bits, False), q.TF_OP_GEMM: linear_fn(q, bits, True),
              q.TF_OP_GEMV_SILU_MUL: q.tf_gemv_w4a16_silu_mul if bits == 4 else q.tf_gemv_w8a16_silu_mul,
              q.TF_OP_GEMM_SILU_MUL: q.tf_gemm_w4a16_silu_mul if bits == 4 else q.tf_gemm_w8a16_silu_mul,
              q.TF_OP_GEMV_F16: q.tf_gemv_w4a16_f16 if bits == 4 else q.tf_gemv_w8a16_f16,
              q.TF_OP_GEMM_F16: q.tf_gemm_w4a16_f16 if bits == 4 else q.tf_gemm_w8a16_f16}[op]
        return fn(x, packed, K, N, G, y=y)
    if cus == 0:
        import torch as _torch

        cus = device_cus(torch or _torch)
    return q.tf_linear_planned(bits, op, x, packed, K, N, G, cus, route, y=y)


def linear_op(q, case, gemm):
    """The TF_OP_* of a plain linear call on the case (its dtype picks the
    bf16 or the fp16 entry points)."""
    if getattr(case, "dtype", "bf16") == "f16":
        return q.TF_OP_GEMM_F16 if gemm else q.TF_OP_GEMV_F16
    return q.TF_OP_GEMM if gemm else q.TF_OP_GEMV


def check_linear(case, torch, q, gemm, rows=None, cols=None, packed=None, d=None, cus=0, route=0):
    """Run the HIP path on the whole case, compare the chosen rows/columns.
    cus / route: the plan inputs (0, 0: the product call as routed)."""
    d = d or to_device(case, torch)
    packed = packed if packed is not None else repack(case, d, q)
    op = linear_op(q, case, gemm)
    y = run_linear(q, case.bits, op, d["x"], packed, case.K, case.N, case.G, cus=cus, route=route, torch=torch)
    torch.cuda.synchronize()
    yh = bf16_to_f64(y)
    ref = oracle.awq_linear(case, cols=cols, rows=rows)
    sub = yh if rows is None else yh[np.asarray(rows)]
    sub = sub if cols is None else sub[:, np.asarray(cols)]
    ok, ratio = within_tolerance(sub, ref)
    return ok, ratio, y


def split_cus(q, bits, M, K, N, G):
    """A compute-unit count for which the 256 x 128 tiled GEMM's plan has
    both 128- and 64-column tiles and does not split K, or None if no count
    gives one (run it with route TF_ROUTE_TILED128)."""
    mt = -(-M // 256)
    tiles = mt * -(-N // 128)
    for cus in range(2, tiles + 1):
        _, wide, narrow, splits, _, _, _, _ = q.tf_gemm_plan(bits, M, K, N, G, cus, q.TF_ROUTE_TILED128)
        if wide and narrow and splits == 1:
            return cus
    return None


def splitk_cus(q, bits, M, K, N, G, route=None):
    """A compute-unit count for which the tiled GEMM's plan (route: default
    TF_ROUTE_TILED) splits K, or None."""
    route = q.TF_ROUTE_TILED if route is None else route
    for cus in (256, 1024, 4096, 1 << 20):
        if q.tf_gemm_plan(bits, M, K, N, G, cus, route)[3] > 1:
            return cus
    return None
