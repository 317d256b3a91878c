"""FP4 (E2M1) codes through a 16-entry table, one fp32 scale per 64-weight block, of the oracle.

Test infrastructure only (see the package docstring).

Sources:
  * LLM Compressor 0.14: GPTQ's 15x speedup is one fused loop, section "Details worth knowing"
    (rounding per format): FP4 rounds onto the magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6} by
    comparisons against fixed thresholds whose <= and < alternate, so that a value exactly
    between two magnitudes goes to the even code.
  * My Triton Kernel Ties bitsandbytes, section "The kernels": the fused kernel named for FP4
    decodes through a 16-entry fp32 codebook, code[nibble] times the block's scale, the same
    unpack path as NF4.

Readings where the pages are silent (each listed in the design notes):
  * Nibble layout: bit 3 is the sign, bits 0-2 index the magnitude grid above (E2M1), so the
    16-entry table is [+grid, -grid]; entry 8 is -0.0.
  * Blocks of 64 along K with one fp32 scale per block, as NF4; the scale is s = fp32(absmax / 6),
    so the block's largest magnitude lands on 6, the top of the grid.
  * Magnitude index: the ladder applied to |w| / s, the quotient in fp64 against the rounded s
    (thresholds 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5: a value on 0.25, 1.25, 2.5 or 5 stays below,
    one on 0.75, 1.75 or 3.5 goes above: the even code in both cases); sign bit = (w < 0).
  * A block whose scale is 0 stores scale 0 and nibble 0 everywhere.
  * Nibble order within a byte is the NF4 one: element 2i in the high nibble.
  * Non-finite weights are rejected.
"""
from __future__ import annotations

import numpy as np

FP4_BLOCK = 64
FP4_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
# (threshold, a value on it stays below): alternating <= and <, ties to the even index
FP4_LADDER = ((0.25, True), (0.75, False), (1.25, True), (1.75, False), (2.5, True), (3.5, False),
              (5.0, True))


def fp4_codebook() -> np.ndarray:
    """The 16 table entries as fp32: nibbles 0-7 the magnitude grid, 8-15 its negatives."""
    g = np.array(FP4_GRID, dtype=np.float32)
    return np.concatenate([g, -g]).astype(np.float32)


def fp4_magnitude_index(y: np.ndarray) -> np.ndarray:
    """Ladder index 0..7 of magnitudes y >= 0 (fp64): one step past each threshold crossed."""
    y = np.asarray(y, dtype=np.float64)
    idx = np.zeros(y.shape, dtype=np.uint8)
    for t, stays_below in FP4_LADDER:
        idx += ((y > t) if stays_below else (y >= t)).astype(np.uint8)
    return idx


def quantize_fp4(w: np.ndarray):
    """Quantize fp32 ``w[N, K]`` to FP4.

    Returns ``(packed uint8[N, K/2], scale float32[N, K/64])``.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    if n < 1 or k < 1 or k % FP4_BLOCK:
        raise ValueError(f"K must be a positive multiple of {FP4_BLOCK}")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    blocks = w.reshape(n, k // FP4_BLOCK, FP4_BLOCK)
    absmax = np.abs(blocks).max(axis=2)  # fp32, exact
    s32 = absmax / np.float32(6.0)  # IEEE fp32 division, round to nearest even
    s64 = s32.astype(np.float64)[..., None]
    safe = np.where(s64 > 0.0, s64, 1.0)
    mag = fp4_magnitude_index(np.abs(blocks.astype(np.float64)) / safe)
    nib = (mag | np.where(blocks < 0.0, 8, 0).astype(np.uint8)).astype(np.uint8)
    nib[np.broadcast_to(s64 == 0.0, nib.shape)] = 0
    nib = nib.reshape(n, k)
    packed = ((nib[:, 0::2] << 4) | nib[:, 1::2]).astype(np.uint8)
    return packed, s32.astype(np.float32)


def dequant_fp4(packed: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp64 [N, K] decoded weights: table[nibble] * scale of the nibble's block (exact)."""
    from .gemv import unpack_nibbles

    idx = unpack_nibbles(packed)
    n, k = idx.shape
    code = fp4_codebook().astype(np.float64)
    s = np.repeat(np.asarray(scale, dtype=np.float32).astype(np.float64), FP4_BLOCK, axis=1)
    if s.shape != (n, k):
        raise ValueError("scale shape does not match [N, K/64]")
    return code[idx] * s
