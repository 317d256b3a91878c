"""Storage-format helpers of the oracle: 16-bit activation and scale bit patterns to fp64.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> exact fp64 values (numpy's half conversion is exact)."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exact fp64 values.  bf16 is the top half of an fp32 word."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def x_bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return f16_bits_to_f64(bits)
    if dtype == "bf16":
        return bf16_bits_to_f64(bits)
    raise ValueError(f"unknown activation dtype {dtype!r}")


def f32_to_bf16_rne_bits(v: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16, nearest even on the 16 dropped bits; return the bits.

    Written out on the integer pattern: add 0x7FFF plus the lowest kept bit, then truncate.  A
    value exactly halfway between two bf16 neighbours moves to the one whose last bit is 0.
    """
    v = np.ascontiguousarray(v, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("bf16 rounding of a non-finite value")
    u = v.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
