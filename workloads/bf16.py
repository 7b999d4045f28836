"""bfloat16 encoding helpers for the synthetic input generators.

Inputs are produced as float32 and stored as bfloat16 bit patterns (uint16)
so that the CPU oracle and the GPU path consume exactly the same bits.
Rounding is round-to-nearest-even on the float32 bit pattern; NaN stays NaN.
"""

import numpy as np


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (nearest-even), returned as uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # Round to nearest even: add 0x7FFF plus the lowest kept mantissa bit.
    lsb = (u >> 16) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b):
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x):
    """Round float32 values to the nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))
