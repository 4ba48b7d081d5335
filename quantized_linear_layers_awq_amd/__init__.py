"""Fused W4A16 / W8A16 linear layer for AMD MI355X (gfx950).

Thin binding over ``libtilefuse.so`` (C ABI declared in ``include/tilefuse.h``).
Each ``tf_*`` function here has the name of the C entry point it calls and
only marshals arguments: torch supplies device memory and the current
stream, every step of the computation runs in the HIP kernels.  There is no
CPU fallback: without the built library every call raises.
"""

from __future__ import annotations

from ._binding import (  # noqa: F401
    TF_ERRORS,
    TileFuseError,
    library_path,
    load_library,
    TF_OP_GEMM,
    TF_OP_GEMM_F16,
    TF_OP_GEMM_SILU_MUL,
    TF_OP_GEMV,
    TF_OP_GEMV_F16,
    TF_OP_GEMV_SILU_MUL,
    TF_ROUTE_AUTO,
    TF_ROUTE_GEMV,
    TF_ROUTE_TILED,
    TF_ROUTE_TILED128,
    tf_dequant_gemv_w4_f32,
    tf_dequant_gemv_w8_f32,
    tf_dequant_w4_f32,
    tf_dequant_w8_f32,
    tf_format_version,
    tf_gemm_plan,
    tf_gemv_plan,
    tf_gemm_w4a16,
    tf_gemm_w4a16_f16,
    tf_gemm_w4a16_noalloc,
    tf_gemm_w4a16_silu_mul,
    tf_gemm_w8a16,
    tf_gemm_w8a16_f16,
    tf_gemm_w8a16_silu_mul,
    tf_gemv_w4a16,
    tf_gemv_w4a16_f16,
    tf_gemv_w4a16_silu_mul,
    tf_gemv_w8a16,
    tf_gemv_w8a16_f16,
    tf_gemv_w8a16_silu_mul,
    tf_linear_planned,
    tf_packed_bytes_w4,
    tf_packed_bytes_w8,
    tf_probe_block_read,
    tf_probe_mfma,
    tf_probe_stream_read,
    tf_repack_w4,
    tf_repack_w4_gate_up,
    tf_repack_w8,
    tf_repack_w8_gate_up,
    tf_status_string,
    tf_workspace_bytes,
    tf_workspace_bytes_planned,
)

__all__ = [n for n in dir() if n.startswith(("tf_", "TF_"))] + ["TileFuseError", "load_library"]
