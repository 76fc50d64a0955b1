"""Exact widening of 16-bit storage patterns to float64.

Every fp16 and bf16 value is exactly representable in float64, so these
conversions lose nothing.  bf16 is the high half of an IEEE binary32, so a
16-bit left shift gives the binary32 pattern.
"""

from __future__ import annotations

import numpy as np


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    raise ValueError(dtype)
