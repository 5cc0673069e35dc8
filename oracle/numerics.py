"""Bit-level conversions between bf16 / fp16 patterns and numpy floats.

bf16 -> fp32 is exact (a bf16 pattern is the top half of an fp32 pattern).
fp32 -> fp16 uses numpy's conversion, which rounds to nearest, ties to even;
tests pin it against exact rational rounding.
"""

from __future__ import annotations

import numpy as np


def bf16_to_f32(bits) -> np.ndarray:
    """uint16 bf16 patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_f16_bits(x) -> np.ndarray:
    """float32 -> fp16 bit patterns, round to nearest even."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def f16_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)
