"""Seeded synthetic AWQ-style inputs (W4A16 / W8A16).

Value distributions and shapes follow the evaluated workloads of the
TileFuse pages: Llama-style decoder linears (hidden 4096, GQA 32 query / 8
key-value heads of 128, FFN 14336), a 2048-token prefill, and the large
(up to 32K) dimensions the interleaved pre-tiling is said to support
(TileFuse summary, "Results" and Methodology section 2 "Interleaved
pre-tiling").  No trained checkpoint exists here; these draws stand in for
one.

Storage formats produced (the inputs of the linear layer):

* W4 codes: uint32 ``qweight[K][N/8]``; word ``(k, c)`` holds columns
  ``8c .. 8c+7`` of row ``k``, nibble ``i`` (bits ``4i .. 4i+3``) holding
  column ``8c + AWQ_COLUMN_AT_NIBBLE[i]``.  Zero points use the same packing
  on ``qzeros[K/G][N/8]``.  This is the interleaved nibble order of the
  common AWQ GEMM checkpoint layout.
* W8 codes: uint8 ``qweight[K][N]``, zero points uint8 ``zeros[K/G][N]``.
* scales: bf16 bit patterns (uint16) ``[K/G][N]``; group ``g`` covers rows
  ``g*G .. g*G+G-1`` of one output column (per-channel metadata is G = K).
* activations x: bf16 bit patterns (uint16) ``[M][K]``.

With ``dtype="f16"`` the scales and activations are drawn from the same
distributions and stored as IEEE fp16 bit patterns instead (the format of
many AWQ checkpoints); ``Case.dtype`` records which.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 20260611

# Nibble i of a packed W4 word holds column 8c + AWQ_COLUMN_AT_NIBBLE[i].
AWQ_COLUMN_AT_NIBBLE = (0, 2, 4, 6, 1, 3, 5, 7)


def f32_to_bf16_bits(a) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits.

    Inputs are finite by construction; NaN is mapped to the quiet NaN 0x7FC0.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = r.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def f32_to_f16_bits(a) -> np.ndarray:
    """Round float32 values to IEEE fp16 (numpy's conversion: nearest, ties
    to even); return uint16 bits."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32)).astype(np.float16).view(np.uint16)


def to_half_bits(a, dtype) -> np.ndarray:
    """float32 values -> bit patterns of the 16-bit format dtype ("bf16" or "f16")."""
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    if dtype == "f16":
        return f32_to_f16_bits(a)
    raise ValueError("dtype must be 'bf16' or 'f16'")


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def pack_awq_w4(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes ``[R][C]`` (C % 8 == 0) into AWQ words ``[R][C/8]``."""
    codes = np.asarray(codes)
    R, C = codes.shape
    if C % 8:
        raise ValueError("W4 packing needs a column count divisible by 8")
    if codes.size and int(codes.max()) > 15:
        raise ValueError("W4 codes must lie in [0, 15]")
    c8 = codes.reshape(R, C // 8, 8).astype(np.uint32)
    words = np.zeros((R, C // 8), dtype=np.uint32)
    for i, col in enumerate(AWQ_COLUMN_AT_NIBBLE):
        words |= c8[:, :, col] << np.uint32(4 * i)
    return words


@dataclass
class Case:
    """One set of layer inputs, already in checkpoint storage format."""

    bits: int
    M: int
    K: int
    N: int
    G: int
    qweight: np.ndarray
    qzeros: np.ndarray
    scales: np.ndarray
    x: np.ndarray
    codes: np.ndarray | None = None
    zeros: np.ndarray | None = None
    name: str = ""
    meta: dict = field(default_factory=dict)
    dtype: str = "bf16"  # format of scales and x: "bf16" or "f16"


def pack_case(bits, codes, zeros, scales_bits, x_bits, G, name="", keep_codes=True, dtype="bf16") -> Case:
    """Wrap drawn (or hand-made) codes/zeros/scales/x into a :class:`Case`."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    zeros = np.ascontiguousarray(zeros, dtype=np.uint8)
    K, N = codes.shape
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    M = x_bits.shape[0]
    if x_bits.shape[1] != K or zeros.shape != (K // G, N) or K % G:
        raise ValueError("inconsistent case shapes")
    if bits == 4:
        qweight, qzeros = pack_awq_w4(codes), pack_awq_w4(zeros)
    elif bits == 8:
        qweight, qzeros = codes, zeros
    else:
        raise ValueError("bits must be 4 or 8")
    return Case(bits=bits, M=M, K=K, N=N, G=G, qweight=qweight, qzeros=qzeros,
                scales=np.ascontiguousarray(scales_bits, dtype=np.uint16), x=x_bits,
                codes=codes if keep_codes else None, zeros=zeros if keep_codes else None,
                name=name, dtype=dtype)


# Value distributions per weight width: code range, zero range (inclusive),
# and scale = a + c*|N(0,1)|.
DIST = {
    4: dict(zero_lo=0, zero_hi=15, scale_a=0.002, scale_c=0.01),
    8: dict(zero_lo=112, zero_hi=143, scale_a=0.0005, scale_c=0.002),
}


def draw_weights(rng, bits, K, N, G, dtype="bf16"):
    """Draw codes [K][N], zeros [K/G][N] and scales [K/G][N] (bit patterns of
    dtype), in that order."""
    d = DIST[bits]
    codes = rng.integers(0, 1 << bits, size=(K, N), dtype=np.uint8)
    zeros = rng.integers(d["zero_lo"], d["zero_hi"] + 1, size=(K // G, N), dtype=np.uint8)
    z = rng.standard_normal(size=(K // G, N), dtype=np.float32)
    scales = np.float32(d["scale_a"]) + np.float32(d["scale_c"]) * np.abs(z)
    return codes, zeros, to_half_bits(scales, dtype)


def draw_x(rng, M, K, outlier_frac=0.0, outlier_gain=20.0, dtype="bf16"):
    """Draw activations N(0,1); optionally scale round(frac*K) channels by gain."""
    x = rng.standard_normal(size=(M, K), dtype=np.float32)
    if outlier_frac > 0:
        n_out = int(round(outlier_frac * K))
        ch = rng.choice(K, size=n_out, replace=False)
        x[:, ch] *= np.float32(outlier_gain)
    return to_half_bits(x, dtype)


def make_inputs(bits, M, K, N, G, seed, outlier_frac=0.0, keep_codes=True, name="", dtype="bf16") -> Case:
    """Draw a full case from ``seed`` (a tuple of ints).

    Weights come from ``SeedSequence(seed)`` and activations from
    ``SeedSequence(seed + (M,))``, so cases that differ only in M share weights.
    """
    seed = tuple(int(s) for s in seed)
    wrng = np.random.default_rng(np.random.SeedSequence(list(seed)))
    codes, zeros, scales = draw_weights(wrng, bits, K, N, G, dtype=dtype)
    xrng = np.random.default_rng(np.random.SeedSequence(list(seed) + [M]))
    x = draw_x(xrng, M, K, outlier_frac, dtype=dtype)
    return pack_case(bits, codes, zeros, scales, x, G, name=name, keep_codes=keep_codes, dtype=dtype)


# Llama-style decoder layer linears: (name, K, N).
LAYER = (
    ("q", 4096, 4096),
    ("k", 4096, 1024),
    ("v", 4096, 1024),
    ("o", 4096, 4096),
    ("gate", 4096, 14336),
    ("up", 4096, 14336),
    ("down", 14336, 4096),
)


def layer_shapes():
    return LAYER


# The five workloads: per config a list of shapes (name, bits, K, N, G) and the
# M values each is run at, plus the activation outlier fraction.
CONFIGS = {
    0: dict(desc="W4A16 GEMV, M=1, 4096x4096, group 128",
            shapes=[("w4_4096x4096", 4, 4096, 4096, 128)], Ms=(1,), outlier=0.0),
    1: dict(desc="W4A16 GEMV over one Llama-style decoder layer, group 128",
            shapes=[(f"layer_{n}", 4, K, N, 128) for n, K, N in LAYER], Ms=(1, 4, 8), outlier=0.0),
    2: dict(desc="W8A16 per-channel, 8192x8192",
            shapes=[("w8_8192x8192", 8, 8192, 8192, 8192)], Ms=(1, 8, 512), outlier=0.0),
    3: dict(desc="W4A16 prefill GEMM, M=2048, group 128, 1% outlier channels x20",
            shapes=[("w4_4096x14336", 4, 4096, 14336, 128), ("w4_14336x4096", 4, 14336, 4096, 128)],
            Ms=(2048,), outlier=0.01),
    4: dict(desc="W4A16 large dimensions, group 128",
            shapes=[("w4_8192x32768", 4, 8192, 32768, 128), ("w4_28672x8192", 4, 28672, 8192, 128)],
            Ms=(1, 4096), outlier=0.0),
}


def make_case(config: int, shape_id: int, M: int, keep_codes=True, replica: int | None = None,
              dtype: str = "bf16") -> Case:
    """Inputs of one workload shape, seeded by (root, config, shape_id[, replica])."""
    cfg = CONFIGS[config]
    name, bits, K, N, G = cfg["shapes"][shape_id]
    seed = (SEED_ROOT, config, shape_id) + (() if replica is None else (replica,))
    c = make_inputs(bits, M, K, N, G, seed, outlier_frac=cfg["outlier"], keep_codes=keep_codes,
                    name=f"c{config}_{name}_M{M}" + ("" if dtype == "bf16" else f"_{dtype}"), dtype=dtype)
    c.meta.update(config=config, shape_id=shape_id)
    return c
