"""Seeded synthetic inputs for the fused W4A16 / W8A16 linear layer.

This package produces the inputs that both the HIP path and the CPU oracle
consume: integer codes packed in the AWQ checkpoint layout, zero points,
bf16 (or fp16) scales and activations.  It holds none of the layer's arithmetic
(no unpacking, no dequantization, no products); it only draws random values
and writes them in the storage formats a quantized checkpoint uses.
"""

from .gen import (  # noqa: F401
    AWQ_COLUMN_AT_NIBBLE,
    CONFIGS,
    Case,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    f32_to_f16_bits,
    layer_shapes,
    make_case,
    make_inputs,
    pack_case,
    pack_awq_w4,
)
