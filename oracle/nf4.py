"""NF4 codebook, blockwise-absmax quantizer and dequantizer of the oracle.

Test infrastructure only (see the package docstring).

Source: LLM Quantization on RTX 4060: Where 4-bit Decode Falls Behind FP16.
  * section "Standard Expectation from Quantization": NF4 is a nonlinear 4-bit format for
    normally distributed weights with 16 unevenly spaced code points; blocks of 64 weights share
    one FP32 absmax scale; two 4-bit values are packed per uint8.
  * section "Kernel Implementation": the high nibble ``(p >> 4) & 0xF`` pairs with input element
    2i and the low nibble ``p & 0xF`` with 2i+1; the block index of a byte is
    ``row * (K / 64) + (2 * byte) // 64``; the decoded weight is ``code[nibble] * absmax``.

Readings where the page is silent (each listed in the design notes):
  * The 16 code values are not printed.  They are the standard NormalFloat construction:
    delta = ((1 - 1/30) + (1 - 1/32)) / 2; eight positive codes Phi^-1(p) at nine evenly spaced
    p from delta down to 1/2 with the 1/2 end dropped; seven negative codes -Phi^-1(p) at eight
    evenly spaced p from delta down to 1/2 with the 1/2 end dropped; an exact 0; sorted, divided
    by Phi^-1(delta) and rounded to fp32.
  * Index choice: the nearest code to the exact ratio w / absmax; a ratio exactly on the midpoint
    of two codes takes the lower index.
  * A block whose absmax is 0 stores absmax 0 and index 7 (the 0.0 code) everywhere.
  * Non-finite weights are rejected.
"""
from __future__ import annotations

from statistics import NormalDist

import numpy as np

NF4_BLOCK = 64


def nf4_codebook() -> np.ndarray:
    """The 16 NF4 code points, ascending, as fp32 (construction in the module docstring)."""
    nd = NormalDist()
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    pos_p = np.linspace(delta, 0.5, 9)[:-1]
    neg_p = np.linspace(delta, 0.5, 8)[:-1]
    values = [nd.inv_cdf(float(p)) for p in pos_p]
    values += [-nd.inv_cdf(float(p)) for p in neg_p]
    values.append(0.0)
    values.sort()
    top = nd.inv_cdf(delta)
    return np.array([v / top for v in values], dtype=np.float32)


def nf4_midpoints(code: np.ndarray | None = None) -> np.ndarray:
    """fp64 midpoints between neighbouring codes; exact, since each is (a + b) / 2 of two fp32."""
    c = (nf4_codebook() if code is None else code).astype(np.float64)
    return (c[:-1] + c[1:]) / 2.0


def quantize_nf4(w: np.ndarray):
    """Quantize fp32 ``w[N, K]`` to NF4.

    Returns ``(packed uint8[N, K/2], absmax float32[N, K/64])``.

    Steps per row and 64-block: absmax A = max |w| (exact in fp32); index = number of midpoints
    strictly below the ratio w / A, the ratio taken as an fp64 quotient (the fp64 quotient of two
    fp32 values lands on the same side of every midpoint as the exact ratio, and lands exactly on
    a midpoint only when the exact ratio does); pack element 2i into the high nibble.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    if n < 1 or k < 1 or k % NF4_BLOCK:
        raise ValueError(f"K must be a positive multiple of {NF4_BLOCK}")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    blocks = w.reshape(n, k // NF4_BLOCK, NF4_BLOCK)
    absmax = np.abs(blocks).max(axis=2)  # fp32, exact
    a64 = absmax.astype(np.float64)[..., None]
    safe = np.where(a64 > 0.0, a64, 1.0)
    ratio = blocks.astype(np.float64) / safe
    mids = nf4_midpoints()
    idx = np.zeros(blocks.shape, dtype=np.uint8)
    for m in mids:
        idx += (ratio > m).astype(np.uint8)
    idx[np.broadcast_to(a64 == 0.0, idx.shape)] = 7
    idx = idx.reshape(n, k)
    packed = ((idx[:, 0::2] << 4) | idx[:, 1::2]).astype(np.uint8)
    return packed, absmax.astype(np.float32)


def dequant_nf4(packed: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """fp64 [N, K] decoded weights: code[nibble] * absmax of the nibble's block (exact)."""
    from .gemv import unpack_nibbles

    idx = unpack_nibbles(packed)
    n, k = idx.shape
    code = nf4_codebook().astype(np.float64)
    a = np.repeat(np.asarray(absmax, dtype=np.float32).astype(np.float64), NF4_BLOCK, axis=1)
    if a.shape != (n, k):
        raise ValueError("absmax shape does not match [N, K/64]")
    return code[idx] * a
