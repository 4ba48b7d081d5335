"""ctypes marshalling for libtilefuse.so (argument handling only).

Torch tensors are passed as raw device pointers plus sizes; the stream is
torch's current stream on the tensor's device.  Outputs and the split-K
workspace are allocated with torch.  The C library validates every argument
before touching the GPU and returns a status; a non-zero status raises
:class:`TileFuseError`.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtilefuse.so")

TF_ERRORS = {
    0: "TF_OK", 1: "TF_ERR_NULL", 2: "TF_ERR_SHAPE", 3: "TF_ERR_GROUP", 4: "TF_ERR_ALIGN",
    5: "TF_ERR_BUFFER_TOO_SMALL", 6: "TF_ERR_UNSUPPORTED", 7: "TF_ERR_HIP",
}


class TileFuseError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        self.name = TF_ERRORS.get(status, f"status {status}")
        super().__init__(f"{where}: {tf_status_string(status)}")


_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libtilefuse.so (built in-tree); raise if it was never built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with quantized_linear_layers_awq_amd.build.build()")
        L = ctypes.CDLL(_LIB_PATH)
        P, I64, SZ, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        L.tf_status_string.argtypes = [I]
        L.tf_status_string.restype = ctypes.c_char_p
        L.tf_format_version.restype = I
        for n in ("tf_packed_bytes_w4", "tf_packed_bytes_w8"):
            getattr(L, n).argtypes = [I64, I64, I64]
            getattr(L, n).restype = SZ
        for n in ("tf_repack_w4", "tf_repack_w8", "tf_repack_w4_gate_up", "tf_repack_w8_gate_up"):
            getattr(L, n).argtypes = [P, P, P, I64, I64, I64, P, SZ, P]
            getattr(L, n).restype = I
        L.tf_workspace_bytes.argtypes = [I, I, I64, I64, I64, I64]
        L.tf_workspace_bytes.restype = SZ
        for n in ("tf_gemv_w4a16", "tf_gemv_w8a16", "tf_gemm_w4a16", "tf_gemm_w8a16",
                  "tf_gemv_w4a16_f16", "tf_gemv_w8a16_f16", "tf_gemm_w4a16_f16", "tf_gemm_w8a16_f16"):
            getattr(L, n).argtypes = [P, P, SZ, P, I64, I64, I64, I64, P, SZ, P]
            getattr(L, n).restype = I
        for n in ("tf_gemv_w4a16_silu_mul", "tf_gemv_w8a16_silu_mul", "tf_gemm_w4a16_silu_mul", "tf_gemm_w8a16_silu_mul"):
            getattr(L, n).argtypes = [P, P, SZ, P, I64, I64, I64, I64, P, SZ, P]
            getattr(L, n).restype = I
        for n in ("tf_dequant_w4_f32", "tf_dequant_w8_f32", "tf_dequant_gemv_w4_f32", "tf_dequant_gemv_w8_f32"):
            getattr(L, n).argtypes = [P, SZ, P, I64, I64, I64, P]
            getattr(L, n).restype = I
        L.tf_gemm_w4a16_noalloc.argtypes = [P, P, SZ, P, I64, I64, I64, I64, P]
        L.tf_gemm_w4a16_noalloc.restype = I
        L.tf_linear_planned.argtypes = [I, I, P, P, SZ, P, I64, I64, I64, I64, P, SZ, I, I, P]
        L.tf_linear_planned.restype = I
        L.tf_workspace_bytes_planned.argtypes = [I, I, I64, I64, I64, I64, I, I]
        L.tf_workspace_bytes_planned.restype = SZ
        L.tf_gemm_plan.argtypes = [I, I64, I64, I64, I64, I, I, ctypes.POINTER(I64)]
        L.tf_gemm_plan.restype = I
        L.tf_gemv_plan.argtypes = [I, I64, I64, I64, I64, I, ctypes.POINTER(I64)]
        L.tf_gemv_plan.restype = I
        L.tf_probe_stream_read.argtypes = [P, SZ, P, P]
        L.tf_probe_stream_read.restype = I
        L.tf_probe_mfma.argtypes = [I, I, P, ctypes.POINTER(I64), P]
        L.tf_probe_mfma.restype = I
        L.tf_probe_block_read.argtypes = [I, P, SZ, I64, I64, I64, I, I, P, P]
        L.tf_probe_block_read.restype = I
        _lib = L
        return _lib


def _check(status: int, where: str):
    if status != 0:
        raise TileFuseError(status, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor, stream) -> int:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, name: str, nbytes_per_elem: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if nbytes_per_elem is not None and t.element_size() != nbytes_per_elem:
        raise ValueError(f"{name} must have {nbytes_per_elem}-byte elements (got {t.dtype})")


def tf_status_string(status: int) -> str:
    return load_library().tf_status_string(int(status)).decode()


def tf_format_version() -> int:
    return int(load_library().tf_format_version())


def tf_packed_bytes_w4(K: int, N: int, G: int) -> int:
    return int(load_library().tf_packed_bytes_w4(K, N, G))


def tf_packed_bytes_w8(K: int, N: int, G: int) -> int:
    return int(load_library().tf_packed_bytes_w8(K, N, G))


def tf_workspace_bytes(bits: int, is_gemm: bool, M: int, K: int, N: int, G: int) -> int:
    return int(load_library().tf_workspace_bytes(bits, int(bool(is_gemm)), M, K, N, G))


def _repack(bits, fn, qweight, qzeros, scales, K, N, G, packed, stream):
    L = load_library()
    elem = 4 if bits == 4 else 1
    _need(qweight, "qweight", elem)
    if qzeros is not None:  # None: symmetric quantization (zero point 2^(bits-1))
        _need(qzeros, "qzeros", elem)
    _need(scales, "scales", 2)
    nbytes = (L.tf_packed_bytes_w4 if bits == 4 else L.tf_packed_bytes_w8)(K, N, G)
    if packed is None:
        packed = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=qweight.device)
    _need(packed, "packed", 1)
    if qweight.numel() * elem < (K * N * bits) // 8 or scales.numel() * G < K * N:
        raise ValueError(f"{fn}: qweight/scales hold fewer elements than (K, N, G) need")
    _check(getattr(L, fn)(_ptr(qweight), _ptr(qzeros), _ptr(scales), K, N, G, _ptr(packed),
                          packed.numel(), _stream(packed, stream)), fn)
    return packed


def tf_repack_w4(qweight, qzeros, scales, K, N, G, packed=None, stream=None):
    """AWQ W4 checkpoint (int32 [K][N/8], int32 [K/G][N/8] or None for
    symmetric zero points of 8, bf16 [K/G][N]) -> packed uint8."""
    return _repack(4, "tf_repack_w4", qweight, qzeros, scales, K, N, G, packed, stream)


def tf_repack_w4_gate_up(qweight, qzeros, scales, K, N, G, packed=None, stream=None):
    """AWQ W4 checkpoint of a [gate | up] layer (N columns, gate first) ->
    packed uint8 for tf_gemv_w4a16_silu_mul."""
    return _repack(4, "tf_repack_w4_gate_up", qweight, qzeros, scales, K, N, G, packed, stream)


def tf_repack_w8_gate_up(qweight, zeros, scales, K, N, G, packed=None, stream=None):
    return _repack(8, "tf_repack_w8_gate_up", qweight, zeros, scales, K, N, G, packed, stream)


def tf_repack_w8(qweight, zeros, scales, K, N, G, packed=None, stream=None):
    """W8 checkpoint (uint8 [K][N], uint8 [K/G][N] or None for symmetric
    zero points of 128, bf16 [K/G][N]) -> packed uint8."""
    return _repack(8, "tf_repack_w8", qweight, zeros, scales, K, N, G, packed, stream)


# Split-K workspaces, one per (device, stream), grown on demand.  A split
# launch writes every partial sum it later adds up, so what a buffer holds
# between calls does not matter; calls on one stream run in order, so one
# buffer per stream is never used by two calls at once.  A buffer that a
# larger one replaces is kept, never freed: a HIP graph captured on that
# stream still writes and reads it on every replay.
_workspaces: dict = {}
_retired: list = []


def _workspace(device: torch.device, stream_handle: int, nbytes: int):
    if nbytes == 0:
        return None
    key = (device.index, stream_handle)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _retired.append(ws)
        # allocated on the launch stream, so that torch orders the memory's
        # first use after the work already queued there
        with torch.cuda.stream(torch.cuda.ExternalStream(stream_handle, device=device)):
            ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


TF_OP_GEMV, TF_OP_GEMM, TF_OP_GEMV_SILU_MUL, TF_OP_GEMM_SILU_MUL, TF_OP_GEMV_F16, TF_OP_GEMM_F16 = 0, 1, 2, 3, 4, 5
_GEMM_OPS = (TF_OP_GEMM, TF_OP_GEMM_SILU_MUL, TF_OP_GEMM_F16)
_F16_OPS = (TF_OP_GEMV_F16, TF_OP_GEMM_F16)
TF_ROUTE_AUTO, TF_ROUTE_TILED, TF_ROUTE_GEMV, TF_ROUTE_TILED128 = 0, 1, 2, 3


def _call(bits, op, fn, x, packed, K, N, G, y, workspace, stream, plan=None):
    """One linear call through entry point `fn`; plan = (cus, route) calls
    tf_linear_planned with those plan inputs instead."""
    L = load_library()
    _need(x, "x", 2)
    _need(packed, "packed", 1)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"{fn}: x must be [M][K] with K={K}")
    M = x.shape[0]
    n_out = N // 2 if op in (TF_OP_GEMV_SILU_MUL, TF_OP_GEMM_SILU_MUL) else N
    if y is None:
        y = torch.empty((M, n_out), dtype=torch.float16 if op in _F16_OPS else torch.bfloat16, device=x.device)
    _need(y, "y", 2)
    if y.numel() < M * n_out:
        raise ValueError(f"{fn}: y holds fewer than {M * n_out} elements")
    sh = _stream(x, stream)
    if plan is None:
        need = int(L.tf_workspace_bytes(bits, int(op in _GEMM_OPS), M, K, N, G))
    else:
        need = int(L.tf_workspace_bytes_planned(bits, op, M, K, N, G, int(plan[0]), int(plan[1])))
    if workspace is None:
        workspace = _workspace(x.device, sh, need)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (_ptr(workspace), workspace.numel() * workspace.element_size())
    if plan is None:
        st = getattr(L, fn)(_ptr(x), _ptr(packed), packed.numel(), _ptr(y), M, K, N, G, ws_ptr, ws_bytes, sh)
    else:
        st = L.tf_linear_planned(bits, op, _ptr(x), _ptr(packed), packed.numel(), _ptr(y), M, K, N, G, ws_ptr,
                                 ws_bytes, int(plan[0]), int(plan[1]), sh)
    _check(st, fn if plan is None else f"tf_linear_planned({fn})")
    return y


def _linear(bits, is_gemm, fn, x, packed, K, N, G, y, workspace, stream):
    return _call(bits, TF_OP_GEMM if is_gemm else TF_OP_GEMV, fn, x, packed, K, N, G, y, workspace, stream)


def tf_gemv_w4a16(x, packed, K, N, G, y=None, workspace=None, stream=None):
    """y[M][N] (bf16) for x [M][K] bf16, 1 <= M <= 16, W4 packed weights."""
    return _linear(4, False, "tf_gemv_w4a16", x, packed, K, N, G, y, workspace, stream)


def tf_gemv_w8a16(x, packed, K, N, G, y=None, workspace=None, stream=None):
    return _linear(8, False, "tf_gemv_w8a16", x, packed, K, N, G, y, workspace, stream)


def tf_gemm_w4a16(x, packed, K, N, G, y=None, workspace=None, stream=None):
    """y[M][N] (bf16) for x [M][K] bf16, any M, W4 packed weights."""
    return _linear(4, True, "tf_gemm_w4a16", x, packed, K, N, G, y, workspace, stream)


def tf_gemm_w4a16_noalloc(x, packed, K, N, G, y=None, stream=None):
    """tf_gemm_w4a16 without a workspace: split-K partial sums go to the
    library's fixed per-GPU device array (calls that overlap on one GPU race
    on it).  Allocates nothing but y when y is None."""
    L = load_library()
    _need(x, "x", 2)
    _need(packed, "packed", 1)
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"tf_gemm_w4a16_noalloc: x must be [M][K] with K={K}")
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", 2)
    if y.numel() < M * N:
        raise ValueError("tf_gemm_w4a16_noalloc: y holds fewer than M*N elements")
    _check(L.tf_gemm_w4a16_noalloc(_ptr(x), _ptr(packed), packed.numel(), _ptr(y), M, K, N, G, _stream(x, stream)),
           "tf_gemm_w4a16_noalloc")
    return y


def tf_gemm_w8a16(x, packed, K, N, G, y=None, workspace=None, stream=None):
    return _linear(8, True, "tf_gemm_w8a16", x, packed, K, N, G, y, workspace, stream)


def tf_gemv_w4a16_f16(x, packed, K, N, G, y=None, workspace=None, stream=None):
    """tf_gemv_w4a16 for fp16 checkpoints: x [M][K] fp16, packed from fp16
    scales, y [M][N] fp16."""
    return _call(4, TF_OP_GEMV_F16, "tf_gemv_w4a16_f16", x, packed, K, N, G, y, workspace, stream)


def tf_gemv_w8a16_f16(x, packed, K, N, G, y=None, workspace=None, stream=None):
    return _call(8, TF_OP_GEMV_F16, "tf_gemv_w8a16_f16", x, packed, K, N, G, y, workspace, stream)


def tf_gemm_w4a16_f16(x, packed, K, N, G, y=None, workspace=None, stream=None):
    """tf_gemm_w4a16 for fp16 checkpoints: x [M][K] fp16, packed from fp16
    scales, y [M][N] fp16."""
    return _call(4, TF_OP_GEMM_F16, "tf_gemm_w4a16_f16", x, packed, K, N, G, y, workspace, stream)


def tf_gemm_w8a16_f16(x, packed, K, N, G, y=None, workspace=None, stream=None):
    return _call(8, TF_OP_GEMM_F16, "tf_gemm_w8a16_f16", x, packed, K, N, G, y, workspace, stream)


def _silu_mul(bits, fn, x, packed, K, N, G, y, workspace, stream, is_gemm=False):
    op = TF_OP_GEMM_SILU_MUL if is_gemm else TF_OP_GEMV_SILU_MUL
    return _call(bits, op, fn, x, packed, K, N, G, y, workspace, stream)


def tf_gemm_w4a16_silu_mul(x, packed, K, N, G, y=None, workspace=None, stream=None):
    """y[M][N/2] = silu(x Wg) * (x Wu) (bf16) for a W4 [gate | up] layer of N
    columns packed by tf_repack_w4_gate_up, x [M][K] bf16, any M."""
    return _silu_mul(4, "tf_gemm_w4a16_silu_mul", x, packed, K, N, G, y, workspace, stream, is_gemm=True)


def tf_gemm_w8a16_silu_mul(x, packed, K, N, G, y=None, workspace=None, stream=None):
    return _silu_mul(8, "tf_gemm_w8a16_silu_mul", x, packed, K, N, G, y, workspace, stream, is_gemm=True)


def tf_gemv_w4a16_silu_mul(x, packed, K, N, G, y=None, workspace=None, stream=None):
    """y[M][N/2] = silu(x Wg) * (x Wu) (bf16) for a W4 [gate | up] layer of N
    columns packed by tf_repack_w4_gate_up, x [M][K] bf16, 1 <= M <= 16."""
    return _silu_mul(4, "tf_gemv_w4a16_silu_mul", x, packed, K, N, G, y, workspace, stream)


def tf_gemv_w8a16_silu_mul(x, packed, K, N, G, y=None, workspace=None, stream=None):
    return _silu_mul(8, "tf_gemv_w8a16_silu_mul", x, packed, K, N, G, y, workspace, stream)


def _dequant(fn, packed, K, N, G, w, stream):
    L = load_library()
    _need(packed, "packed", 1)
    if w is None:
        w = torch.empty((K, N), dtype=torch.float32, device=packed.device)
    _need(w, "w", 4)
    if w.numel() < K * N:
        raise ValueError(f"{fn}: w holds fewer than K*N elements")
    _check(getattr(L, fn)(_ptr(packed), packed.numel(), _ptr(w), K, N, G, _stream(packed, stream)), fn)
    return w


def tf_dequant_w4_f32(packed, K, N, G, w=None, stream=None):
    """Test hook: fp32 dequantized weights [K][N] from a W4 packed buffer,
    decoded by the GEMM's operand builder."""
    return _dequant("tf_dequant_w4_f32", packed, K, N, G, w, stream)


def tf_dequant_w8_f32(packed, K, N, G, w=None, stream=None):
    return _dequant("tf_dequant_w8_f32", packed, K, N, G, w, stream)


def tf_dequant_gemv_w4_f32(packed, K, N, G, w=None, stream=None):
    """Test hook: the same weights decoded by the GEMV kernels' operand
    builders (128 + q and 128 + z, their difference times s)."""
    return _dequant("tf_dequant_gemv_w4_f32", packed, K, N, G, w, stream)


def tf_dequant_gemv_w8_f32(packed, K, N, G, w=None, stream=None):
    return _dequant("tf_dequant_gemv_w8_f32", packed, K, N, G, w, stream)


_OP_FN = {(4, TF_OP_GEMV): "tf_gemv_w4a16", (8, TF_OP_GEMV): "tf_gemv_w8a16", (4, TF_OP_GEMM): "tf_gemm_w4a16",
          (8, TF_OP_GEMM): "tf_gemm_w8a16", (4, TF_OP_GEMV_SILU_MUL): "tf_gemv_w4a16_silu_mul",
          (8, TF_OP_GEMV_SILU_MUL): "tf_gemv_w8a16_silu_mul", (4, TF_OP_GEMM_SILU_MUL): "tf_gemm_w4a16_silu_mul",
          (8, TF_OP_GEMM_SILU_MUL): "tf_gemm_w8a16_silu_mul", (4, TF_OP_GEMV_F16): "tf_gemv_w4a16_f16",
          (8, TF_OP_GEMV_F16): "tf_gemv_w8a16_f16", (4, TF_OP_GEMM_F16): "tf_gemm_w4a16_f16",
          (8, TF_OP_GEMM_F16): "tf_gemm_w8a16_f16"}


def tf_linear_planned(bits, op, x, packed, K, N, G, cus, route=TF_ROUTE_AUTO, y=None, workspace=None, stream=None):
    """Test hook: the linear call `op` (TF_OP_*) planned for `cus` compute
    units and kernel route `route` (TF_ROUTE_*), with the workspace that plan
    needs; same validation and kernels as the product entry point."""
    return _call(bits, op, _OP_FN[(bits, op)], x, packed, K, N, G, y, workspace, stream, plan=(cus, route))


def tf_workspace_bytes_planned(bits, op, M, K, N, G, cus, route=TF_ROUTE_AUTO) -> int:
    return int(load_library().tf_workspace_bytes_planned(bits, op, M, K, N, G, cus, route))


def tf_gemm_plan(bits: int, M: int, K: int, N: int, G: int, cus: int, route: int = TF_ROUTE_AUTO) -> tuple[int, ...]:
    """Test hook: (row tiles, wide column tiles, 64-column tiles, K ranges,
    k-tiles per range, 1 if the call runs the GEMV kernels else 0, rows per
    row tile, columns per wide tile (256 or 128)) of a GEMM call's launch
    plan on a device of `cus` compute units with kernel route `route` (host
    only)."""
    L = load_library()
    out = (ctypes.c_int64 * 8)()
    _check(L.tf_gemm_plan(bits, M, K, N, G, cus, route, out), "tf_gemm_plan")
    return tuple(int(v) for v in out)


GEMV_PLAN_FIELDS = ("kernel", "waves", "bpw", "splits", "split_tiles", "chunk_tiles", "depth", "row_chunks", "lds",
                    "lds_limit", "x_capacity", "rec_capacity", "meta_cap", "xpitch")


def tf_gemv_plan(bits: int, M: int, K: int, N: int, G: int, cus: int) -> dict:
    """Test hook: the GEMV kernels' launch plan for M <= 64 rows on `cus`
    compute units (host only), as a dict over GEMV_PLAN_FIELDS."""
    L = load_library()
    out = (ctypes.c_int64 * 14)()
    _check(L.tf_gemv_plan(bits, M, K, N, G, cus, out), "tf_gemv_plan")
    return dict(zip(GEMV_PLAN_FIELDS, (int(v) for v in out)))


def tf_probe_stream_read(buf, sink, stream=None):
    """Measurement probe: one launch reading every byte of `buf` (a CUDA tensor
    whose size is a multiple of 16 bytes) once; `sink` is a small int32 CUDA
    tensor the kernel may write."""
    L = load_library()
    nbytes = buf.numel() * buf.element_size()
    _check(L.tf_probe_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(buf, stream)), "tf_probe_stream_read")


def tf_probe_block_read(bits, packed, K, N, G, waves, depth, sink, stream=None):
    """Measurement probe: the GEMV's code stream over `packed` (a CUDA uint8
    tensor in the pre-tiled layout of (bits, K, N, G)) without its
    arithmetic, `waves` waves per 16-column block and `depth` tiles in
    flight per wave; `sink` is a small int32 CUDA tensor the kernel may
    write."""
    L = load_library()
    nbytes = packed.numel() * packed.element_size()
    _check(L.tf_probe_block_read(int(bits), _ptr(packed), nbytes, int(K), int(N), int(G), int(waves), int(depth),
                                 _ptr(sink), _stream(packed, stream)), "tf_probe_block_read")


def tf_probe_mfma(workgroups, iters, sink, stream=None) -> int:
    """Measurement probe: one launch of back-to-back bf16 MFMAs; returns its
    flop count.  `sink` is a small float32 CUDA tensor the kernel may write."""
    L = load_library()
    flops = ctypes.c_int64(0)
    _check(L.tf_probe_mfma(int(workgroups), int(iters), _ptr(sink), ctypes.byref(flops), _stream(sink, stream)),
           "tf_probe_mfma")
    return int(flops.value)
