"""CPU oracle for the fused W4A16 / W8A16 linear layer (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``; never by the product package.  It
shares no code with the HIP library.

The arithmetic lives in ``oracle.c`` (plain C, fp32 dequant, fp64 sums in k
order); this module only marshals numpy arrays.  See that file's header for
what each step computes and which passage of the TileFuse summary it
follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (host only)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_unpack_w4.argtypes = [P, I64, I64, P]
        L.oracle_pack_w4.argtypes = [P, I64, I64, P]
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_round_bf16.argtypes = [P, I64, P]
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_round_f16.argtypes = [P, I64, P]
        L.oracle_dequant_w4.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, P, I64, P]
        L.oracle_dequant_w8.argtypes = [P, P, P, ctypes.c_int, I64, I64, I64, P, I64, P]
        L.oracle_linear.argtypes = [P, ctypes.c_int, I64, I64, P, I64, P]
        L.oracle_silu_mul.argtypes = [P, P, I64, P]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        L.oracle_packed_bytes.argtypes = [ctypes.c_int, I64, I64, I64]
        L.oracle_packed_bytes.restype = ctypes.c_size_t
        L.oracle_repack.argtypes = [ctypes.c_int, P, P, P, I64, I64, I64, P]
        L.oracle_repack.restype = ctypes.c_int
        L.oracle_unrepack.argtypes = [ctypes.c_int, P, I64, I64, I64, P, P, P]
        L.oracle_unrepack.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_num_threads(n: int) -> None:
    """Threads the oracle's later parallel loops use."""
    lib().oracle_set_num_threads(int(n))


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def unpack_w4(words) -> np.ndarray:
    """AWQ words [R][C/8] -> 4-bit codes [R][C] (uint8)."""
    words = _c(words, np.uint32)
    R, C8 = words.shape
    out = np.empty((R, C8 * 8), dtype=np.uint8)
    lib().oracle_unpack_w4(_p(words), R, C8 * 8, _p(out))
    return out


def pack_w4(codes) -> np.ndarray:
    """4-bit codes [R][C] -> AWQ words [R][C/8] (the oracle's own packer)."""
    codes = _c(codes, np.uint8)
    R, C = codes.shape
    out = np.empty((R, C // 8), dtype=np.uint32)
    lib().oracle_pack_w4(_p(codes), R, C, _p(out))
    return out


def bf16_to_f32(bits) -> np.ndarray:
    bits = _c(bits, np.uint16)
    f = np.vectorize(lambda b: lib().oracle_bf16_to_f32(int(b)), otypes=[np.float32])
    return f(bits) if bits.size else bits.astype(np.float32)


def f64_to_bf16(y) -> np.ndarray:
    """Round fp64 values to bf16 bits (nearest, ties to even) in one step."""
    y = _c(y, np.float64)
    out = np.empty(y.shape, dtype=np.uint16)
    lib().oracle_round_bf16(_p(y), y.size, _p(out))
    return out


FORMATS = {"bf16": 0, "f16": 1}


def _fmt(dtype: str) -> int:
    if dtype not in FORMATS:
        raise ValueError(f"dtype must be one of {sorted(FORMATS)}")
    return FORMATS[dtype]


def f16_to_f32(bits) -> np.ndarray:
    """Widen fp16 bit patterns to float32 (exact)."""
    bits = _c(bits, np.uint16)
    f = np.vectorize(lambda b: lib().oracle_f16_to_f32(int(b)), otypes=[np.float32])
    return f(bits) if bits.size else bits.astype(np.float32)


def f64_to_f16(y) -> np.ndarray:
    """Round fp64 values to fp16 bits (nearest, ties to even, overflow to
    infinity) in one step."""
    y = _c(y, np.float64)
    out = np.empty(y.shape, dtype=np.uint16)
    lib().oracle_round_f16(_p(y), y.size, _p(out))
    return out


def dequant(bits, qweight, qzeros, scales, K, N, G, cols=None, dtype="bf16") -> np.ndarray:
    """Dequantized fp32 weights w[K][len(cols)] (all N columns when cols is
    None); scales are bf16 or fp16 bit patterns (dtype)."""
    fmt = _fmt(dtype)
    sc = _c(scales, np.uint16)
    if cols is None:
        cp, ncols = None, N
    else:
        cols = _c(cols, np.int64)
        if cols.size and (cols.min() < 0 or cols.max() >= N):
            raise ValueError("column index out of range")
        cp, ncols = _p(cols), cols.size
    w = np.empty((K, ncols), dtype=np.float32)
    if bits == 4:
        qw, qz = _c(qweight, np.uint32), _c(qzeros, np.uint32)
        assert qw.shape == (K, N // 8) and qz.shape == (K // G, N // 8)
        lib().oracle_dequant_w4(_p(qw), _p(qz), _p(sc), fmt, K, N, G, cp, ncols, _p(w))
    elif bits == 8:
        qw, qz = _c(qweight, np.uint8), _c(qzeros, np.uint8)
        assert qw.shape == (K, N) and qz.shape == (K // G, N)
        lib().oracle_dequant_w8(_p(qw), _p(qz), _p(sc), fmt, K, N, G, cp, ncols, _p(w))
    else:
        raise ValueError("bits must be 4 or 8")
    assert sc.shape == (K // G, N)
    return w


def linear(x_bits, w, dtype="bf16") -> np.ndarray:
    """y64[M][N] = sum_k x[m][k] * w[k][n] in fp64, k ascending; x holds bf16
    or fp16 bit patterns (dtype)."""
    fmt = _fmt(dtype)
    x = _c(x_bits, np.uint16)
    w = _c(w, np.float32)
    M, K = x.shape
    assert w.shape[0] == K
    N = w.shape[1]
    y = np.empty((M, N), dtype=np.float64)
    lib().oracle_linear(_p(x), fmt, M, K, _p(w), N, _p(y))
    return y


def awq_linear(case, cols=None, rows=None) -> np.ndarray:
    """Reference output of a synth.Case: fp64 y for the chosen rows/columns
    (x and scales in the case's dtype, bf16 or fp16)."""
    dtype = getattr(case, "dtype", "bf16")
    w = dequant(case.bits, case.qweight, case.qzeros, case.scales, case.K, case.N, case.G, cols, dtype=dtype)
    x = case.x if rows is None else case.x[np.asarray(rows)]
    return linear(x, w, dtype=dtype)


def silu_mul(g, u) -> np.ndarray:
    """silu(g) * u elementwise in fp64 (g and u fp64 arrays of one shape)."""
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    if g.shape != u.shape:
        raise ValueError("g and u differ in shape")
    out = np.empty(g.shape, dtype=np.float64)
    lib().oracle_silu_mul(_p(g), _p(u), g.size, _p(out))
    return out


def awq_linear_silu_mul(case, cols=None, rows=None) -> np.ndarray:
    """Reference output of a synth.Case holding a [gate | up] layer (N even):
    fp64 silu(y[:, n]) * y[:, N/2 + n] for the chosen rows and n < N/2."""
    half = case.N // 2
    cols = np.arange(half) if cols is None else np.asarray(cols, dtype=np.int64)
    y = awq_linear(case, cols=np.concatenate([cols, cols + half]), rows=rows)
    return silu_mul(y[:, : cols.size], y[:, cols.size :])


def packed_bytes(bits, K, N, G) -> int:
    return int(lib().oracle_packed_bytes(bits, K, N, G))


def repack(bits, qweight, qzeros, scales, K, N, G) -> np.ndarray:
    """Reference interleaved pre-tiled buffer (uint8) for the checkpoint inputs."""
    nbytes = packed_bytes(bits, K, N, G)
    if nbytes == 0:
        raise ValueError("invalid (bits, K, N, G)")
    dt = np.uint32 if bits == 4 else np.uint8
    qw, qz, sc = _c(qweight, dt), _c(qzeros, dt), _c(scales, np.uint16)
    out = np.empty(nbytes, dtype=np.uint8)
    rc = lib().oracle_repack(bits, _p(qw), _p(qz), _p(sc), K, N, G, _p(out))
    if rc:
        raise ValueError("oracle_repack rejected the shape")
    return out


def gate_up_order(N) -> np.ndarray:
    """Checkpoint column of each packed column of a [gate | up] layer (N / 2
    a multiple of 8) packed for the SiLU-product GEMV: in 16-column block j,
    columns 0..7 take gate columns 8j..8j+7 and columns 8..15 take up columns
    N/2 + 8j .. N/2 + 8j + 7."""
    if N % 16:
        raise ValueError("N / 2 must be a multiple of 8")
    order = []
    for j in range(N // 16):
        order += [8 * j + c for c in range(8)]
        order += [N // 2 + 8 * j + c for c in range(8)]
    return np.array(order, dtype=np.int64)


def repack_gate_up(bits, qweight, qzeros, scales, K, N, G) -> np.ndarray:
    """Reference buffer for a [gate | up] checkpoint packed for the
    SiLU-product GEMV: the plain layout of the checkpoint with its columns in
    :func:`gate_up_order`.  W4 words hold runs of 8 columns, and the order
    moves whole runs, so whole words move."""
    order = gate_up_order(N)
    if bits == 4:
        words = order[::8] // 8
        qw, qz = np.asarray(qweight)[:, words], np.asarray(qzeros)[:, words]
    else:
        qw, qz = np.asarray(qweight)[:, order], np.asarray(qzeros)[:, order]
    return repack(bits, qw, qz, np.asarray(scales)[:, order], K, N, G)


def unrepack(bits, packed, K, N, G):
    """Inverse of :func:`repack`: (codes [K][N], zeros [K/G][N], scale bits [K/G][N])."""
    packed = _c(packed, np.uint8)
    if packed.size < packed_bytes(bits, K, N, G):
        raise ValueError("packed buffer too small")
    codes = np.empty((K, N), dtype=np.uint8)
    zeros = np.empty((K // G, N), dtype=np.uint8)
    scales = np.empty((K // G, N), dtype=np.uint16)
    rc = lib().oracle_unrepack(bits, _p(packed), K, N, G, _p(codes), _p(zeros), _p(scales))
    if rc:
        raise ValueError("oracle_unrepack rejected the shape")
    return codes, zeros, scales
