"""fp32 <-> bfloat16 conversion (bfloat16 = the upper 16 bits of an IEEE-754
binary32).  Rounding is round-to-nearest, ties-to-even; NaN stays NaN."""
from __future__ import annotations

import numpy as np


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16, returned as uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    nan = np.isnan(x)
    bits = r.astype(np.uint16)
    if nan.any():
        bits = np.where(nan, np.uint16(0x7FC0), bits)
    return bits


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (returned as float32)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))
