"""Asymmetric INT4 (unsigned codes 0..15 with a per-group zero point, one bf16 scale per 128-column
group) of the oracle.

Test infrastructure only (see the package docstring).

Sources:
  * LLM Compressor 0.14: GPTQ's 15x speedup is one fused loop, section "The fused kernel": a code
    is the clamped, rounded sum of the scale quotient and the zero point, and it is decoded
    from the same scale and zero point; section "Details worth knowing": INT rounding is ``rint``
    (round half to even); section "What those numbers leave out": INT4 is tested symmetric and
    asymmetric, grouped.
  * Group size 128 along K and the bf16 scale are the symmetric INT4 format's (the workload's).

Readings where the pages are silent (each listed in the design notes):
  * Range of a group: lo = min(min w, 0), hi = max(max w, 0), so that 0 is always in range.
  * Scale s = bf16_RNE(fp32(fp32(hi - lo) / 15)): the range spread over the 16 unsigned codes.
  * Zero point z = clamp(rint(-lo / s), 0, 15), the quotient in fp64 against the rounded s.
  * Code q = rint(clamp(w / s + z, 0, 15)) in that order, w / s in fp64 against the rounded s;
    the decoded weight is (q - z) * s, so weights on the grid round-trip exactly.
  * A group whose scale is 0 (hi - lo = 0, or the quotient rounding to 0 in bf16) stores scale 0,
    zero point 0 and nibble 0 everywhere.
  * Storage: the nibble is q itself (element 2i in the high nibble, as NF4); per group one 32-bit
    word with the bf16 scale bits in bits 0-15 and z in bits 16-19 (bits 20-31 zero).
  * Non-finite weights are rejected.
"""
from __future__ import annotations

import numpy as np

from .bits import bf16_bits_to_f64, f32_to_bf16_rne_bits

INT4A_GROUP = 128


def int4_asym_scale_zero(lo: np.ndarray, hi: np.ndarray):
    """Scale bf16 bits and zero point of groups with range [lo, hi] (fp32, lo <= 0 <= hi)."""
    lo = np.asarray(lo, dtype=np.float32)
    hi = np.asarray(hi, dtype=np.float32)
    s32 = (hi - lo) / np.float32(15.0)  # two IEEE fp32 operations, round to nearest even
    s_bits = f32_to_bf16_rne_bits(np.asarray(s32, dtype=np.float32))
    s64 = bf16_bits_to_f64(s_bits)
    safe = np.where(s64 > 0.0, s64, 1.0)
    z = np.clip(np.rint(-lo.astype(np.float64) / safe), 0, 15)
    z = np.where(s64 > 0.0, z, 0.0)
    return s_bits, z.astype(np.uint32)


def quantize_int4_asym(w: np.ndarray):
    """Quantize fp32 ``w[N, K]``; returns ``(packed uint8[N, K/2], words uint32[N, K/128])`` with
    word = bf16 scale bits | zero point << 16."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    if n < 1 or k < 1 or k % INT4A_GROUP:
        raise ValueError(f"K must be a positive multiple of {INT4A_GROUP}")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    groups = w.reshape(n, k // INT4A_GROUP, INT4A_GROUP)
    lo = np.minimum(groups.min(axis=2), np.float32(0.0))
    hi = np.maximum(groups.max(axis=2), np.float32(0.0))
    s_bits, z = int4_asym_scale_zero(lo, hi)
    s64 = bf16_bits_to_f64(s_bits)[..., None]
    safe = np.where(s64 > 0.0, s64, 1.0)
    # w / s + z, clamped to the code range, then rounded half to even
    v = groups.astype(np.float64) / safe + z[..., None].astype(np.float64)
    q = np.rint(np.clip(v, 0.0, 15.0))
    q[np.broadcast_to(s64 == 0.0, q.shape)] = 0
    nib = q.astype(np.uint8).reshape(n, k)
    packed = ((nib[:, 0::2] << 4) | nib[:, 1::2]).astype(np.uint8)
    words = s_bits.astype(np.uint32) | (z << 16)
    return packed, words


def dequant_int4_asym(packed: np.ndarray, words: np.ndarray) -> np.ndarray:
    """fp64 [N, K] decoded weights: (nibble - z) * s of the nibble's group (exact)."""
    from .gemv import unpack_nibbles

    nib = unpack_nibbles(packed).astype(np.float64)
    n, k = nib.shape
    words = np.asarray(words, dtype=np.uint32)
    if words.shape != (n, k // INT4A_GROUP):
        raise ValueError("scale shape does not match [N, K/128]")
    s = np.repeat(bf16_bits_to_f64((words & 0xFFFF).astype(np.uint16)), INT4A_GROUP, axis=1)
    z = np.repeat(((words >> 16) & 0xF).astype(np.float64), INT4A_GROUP, axis=1)
    return (nib - z) * s
