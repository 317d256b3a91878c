"""Symmetric INT4 (+8 zero point, one bf16 scale per 128-column group) of the oracle.

Test infrastructure only (see the package docstring).

Sources:
  * My Triton Kernel Ties bitsandbytes, section "The kernels": the stored nibble carries a +8
    zero point; packing without it destroyed every positive weight.
  * LLM Compressor 0.14, section "The problem GPTQ solves" and "Details worth knowing": the grid
    is a fixed multiple of one scale per group, round-to-nearest with a clip, and INT rounding is
    ``rint`` (round half to even).
  * The group size (128 along K) and the bf16 scale come from the workload definition.

Readings where the pages are silent (each listed in the design notes):
  * scale s = bf16_RNE(fp32(absmax / 7)): symmetric, the absmax lands on code +-7 and never clips.
  * code q = clamp(rint(w / s), -8, 7) with the quotient taken against the *rounded* s, so that
    weights on the grid round-trip exactly; the stored nibble is q + 8.
  * A group whose scale is 0 (absmax 0, or absmax / 7 rounding to 0 in bf16) stores scale 0 and
    nibble 8 everywhere.
  * Nibble order within a byte is the NF4 one: element 2i in the high nibble.
  * Non-finite weights are rejected.
"""
from __future__ import annotations

import numpy as np

from .bits import bf16_bits_to_f64, f32_to_bf16_rne_bits

INT4_GROUP = 128


def quantize_int4(w: np.ndarray):
    """Quantize fp32 ``w[N, K]``; returns ``(packed uint8[N, K/2], scale_bits uint16[N, K/128])``."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    if n < 1 or k < 1 or k % INT4_GROUP:
        raise ValueError(f"K must be a positive multiple of {INT4_GROUP}")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    groups = w.reshape(n, k // INT4_GROUP, INT4_GROUP)
    absmax = np.abs(groups).max(axis=2)  # fp32, exact
    s32 = absmax / np.float32(7.0)  # IEEE fp32 division, round to nearest even
    s_bits = f32_to_bf16_rne_bits(s32)
    s64 = bf16_bits_to_f64(s_bits)[..., None]
    safe = np.where(s64 > 0.0, s64, 1.0)
    q = np.clip(np.rint(groups.astype(np.float64) / safe), -8, 7)
    nib = (q + 8).astype(np.uint8)
    nib[np.broadcast_to(s64 == 0.0, nib.shape)] = 8
    nib = nib.reshape(n, k)
    packed = ((nib[:, 0::2] << 4) | nib[:, 1::2]).astype(np.uint8)
    return packed, s_bits


def dequant_int4(packed: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """fp64 [N, K] decoded weights: (nibble - 8) * scale of the nibble's group (exact)."""
    from .gemv import unpack_nibbles

    nib = unpack_nibbles(packed).astype(np.float64)
    n, k = nib.shape
    s = np.repeat(bf16_bits_to_f64(scale_bits), INT4_GROUP, axis=1)
    if s.shape != (n, k):
        raise ValueError("scale shape does not match [N, K/128]")
    return (nib - 8.0) * s
