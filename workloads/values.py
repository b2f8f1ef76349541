"""Seeded random values and their storage encodings.

Values are standard normal float32 from numpy's PCG64 ``default_rng`` (the
decode configurations draw q, K and V from N(0, 1)).  bf16 storage is the upper
half of the float32 bit pattern after round-to-nearest-even; arrays of bf16 are
carried as uint16 bit patterns so that no library's bf16 type is involved.
"""
from __future__ import annotations

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)   # quiet NaN, used to poison unused cache slots
E4M3_NAN_CODE = np.uint8(0x7F)      # S.1111.111 with S = 0: NaN in OCP E4M3FN
F32_NAN = np.float32(np.nan)


def standard_normal_f32(seed, shape) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even) and return the uint16 bit patterns.

    NaN inputs become the quiet NaN with the input's sign.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        sign = ((u >> np.uint32(16)) & np.uint32(0x8000)).astype(np.uint16)
        rounded = np.where(nan, sign | BF16_NAN_BITS, rounded)
    return rounded


def bf16_bits_to_f32_exact(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
