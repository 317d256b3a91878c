"""2:4 structured sparsity (two kept 16-bit values of every four weights, plus position codes) of
the oracle.

Test infrastructure only (see the package docstring).

Source: Do Quantization and Sparsity make LLM Inference Faster?, sections "Library 2:4 sparsity:
fewer values, but too much overhead" and "Custom CUDA 2:4 GEMV" with its optional kernel
walk-through:
  * each group of four weights keeps two values, with a small code giving the two positions;
    values and codes together are 56.25% of the dense fp16 bytes;
  * per row the kept values are stored consecutively, two per group (K/2 16-bit values), and each
    group has a 4-bit code whose low two bits are the first kept position and next two bits the
    second; two codes share a byte, the even group in the low nibble (K/8 bytes per row);
  * the product multiplies each kept value by the activation at its recorded position and sums;
    the removed weights are never rebuilt.

Readings where the pages are silent (each listed in the design notes):
  * Which two are kept: the two largest magnitudes of the group (magnitude pruning); between
    equal magnitudes the lower position wins.  The two kept positions are stored in ascending
    order (first < second).
  * Values are the kept fp32 weights rounded to nearest even to the activation's 16-bit type
    (fp16 as on the page, or bf16).
  * Output y in fp32 (the page's kernel writes fp16); the reference is the plain product with the
    decoded dense matrix (zeros at the removed positions).
  * K a multiple of 32 (whole 16-byte value chunks per lane in the kernel; the page's shapes are).
"""
from __future__ import annotations

import numpy as np

from .bits import f32_to_bf16_rne_bits


def _to16(v: np.ndarray, xdt: str) -> np.ndarray:
    v = np.asarray(v, dtype=np.float32)
    if xdt == "f16":
        return v.astype(np.float16).view(np.uint16)
    return f32_to_bf16_rne_bits(v)


def _from16(bits: np.ndarray, xdt: str) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if xdt == "f16":
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def keep_positions(w: np.ndarray):
    """Positions (p0 < p1) of the two largest magnitudes in every group of four along K, ties to
    the lower position.  w [N, K] -> two int arrays [N, K/4]."""
    a = np.abs(np.asarray(w, dtype=np.float32)).reshape(w.shape[0], -1, 4)
    # rank positions by (-|w|, position): a stable sort on -|w| keeps lower positions first
    order = np.argsort(-a, axis=2, kind="stable")
    two = np.sort(order[:, :, :2], axis=2)
    return two[:, :, 0], two[:, :, 1]


def compress_2to4(w: np.ndarray, xdt: str = "f16"):
    """fp32 w [N, K] -> (values uint16 [N, K/2] (16-bit bits), meta uint8 [N, K/8])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N, K]")
    n, k = w.shape
    if n < 1 or k < 32 or k % 32:
        raise ValueError("K must be a positive multiple of 32")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    p0, p1 = keep_positions(w)
    g = w.reshape(n, k // 4, 4)
    v0 = np.take_along_axis(g, p0[..., None], axis=2)[..., 0]
    v1 = np.take_along_axis(g, p1[..., None], axis=2)[..., 0]
    values = np.stack([v0, v1], axis=2).reshape(n, k // 2)
    code = (p0 | (p1 << 2)).astype(np.uint8)            # one 4-bit code per group
    meta = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)  # even group: low nibble
    return _to16(values, xdt), meta


def dense_from_2to4(values: np.ndarray, meta: np.ndarray, xdt: str = "f16") -> np.ndarray:
    """fp64 [N, K]: the kept values at their recorded positions, zeros elsewhere (exact)."""
    values = np.asarray(values, dtype=np.uint16)
    meta = np.asarray(meta, dtype=np.uint8)
    n, half = values.shape
    k = 2 * half
    if meta.shape != (n, k // 8):
        raise ValueError("meta must be [N, K/8]")
    code = np.empty((n, k // 4), dtype=np.uint8)
    code[:, 0::2] = meta & 0x0F
    code[:, 1::2] = meta >> 4
    v = _from16(values, xdt).reshape(n, k // 4, 2)
    out = np.zeros((n, k // 4, 4))
    rows = np.arange(n)[:, None]
    grp = np.arange(k // 4)[None, :]
    # the second kept value goes in last, so a (malformed) code with equal positions keeps it
    out[rows, grp, code & 3] = v[..., 0]
    out[rows, grp, (code >> 2) & 3] = v[..., 1]
    return out.reshape(n, k)


def sparse_bytes(n: int, k: int) -> int:
    """Stored bytes of an N x K matrix: K/2 16-bit values and K/8 metadata bytes per row."""
    return n * (k // 2) * 2 + n * (k // 8)
