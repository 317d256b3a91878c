"""Reference GEMV / small-batch GEMM of the oracle and its acceptance bound.

Test infrastructure only (see the package docstring).

Source: LLM Quantization on RTX 4060: Where 4-bit Decode Falls Behind FP16, section "Kernel
Implementation": an output row is the dot product of the decoded weight row with the activation
row, and the kernel there keeps its running sums in fp32, since a dot product 1536 terms long loses
too much in a 16-bit accumulator; fusing the dequantization into the product moves where the
decode happens, not what is summed.  So the reference is
the plain definition y[b, n] = sum_k x[b, k] * W_hat[n, k], taken here in fp64 on the exact
decoded weights and the exact activation values.

Acceptance (the pages give no tolerance): |y - y_ref| <= 2e-3 * T + 1e-5 per element, with
T[b, n] = sum_k |x[b, k] * W_hat[n, k]|.  Any summation order inside that bound is correct, so
results of different GPU paths need not be bitwise equal to each other.
"""
from __future__ import annotations

import numpy as np

from .bits import x_bits_to_f64

REL_TOL = 2e-3
ABS_TOL = 1e-5


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """uint8 [N, K/2] -> uint8 [N, K] of 4-bit indices; element 2i is the high nibble."""
    p = np.ascontiguousarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p >> 4
    out[:, 1::2] = p & 0x0F
    return out


def dequant(fmt: str, packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Decoded fp64 weights for ``fmt`` in {"nf4", "int4", "int4a", "fp4"}."""
    if fmt == "nf4":
        from .nf4 import dequant_nf4

        return dequant_nf4(packed, scales)
    if fmt == "int4":
        from .int4 import dequant_int4

        return dequant_int4(packed, scales)
    if fmt == "int4a":
        from .int4_asym import dequant_int4_asym

        return dequant_int4_asym(packed, scales)
    if fmt == "fp4":
        from .fp4 import dequant_fp4

        return dequant_fp4(packed, scales)
    raise ValueError(f"unknown weight format {fmt!r}")


def gemv_reference(x_bits: np.ndarray, x_dtype: str, w_hat: np.ndarray):
    """Return ``(y_ref, T)``, both fp64 [B, N], for activation bits ``x_bits[B, K]``."""
    x = x_bits_to_f64(np.atleast_2d(x_bits), x_dtype)
    w = np.asarray(w_hat, dtype=np.float64)
    if x.shape[1] != w.shape[1]:
        raise ValueError("x and W_hat disagree on K")
    y = x @ w.T
    t = np.abs(x) @ np.abs(w).T
    return y, t


def violation_ratio(y, y_ref, t) -> float:
    """max over elements of |y - y_ref| / (2e-3 T + 1e-5); the result passes iff this is <= 1."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    bound = REL_TOL * np.asarray(t, dtype=np.float64) + ABS_TOL
    return float(np.max(np.abs(y - y_ref) / bound)) if y.size else 0.0


def accept(y, y_ref, t) -> bool:
    return violation_ratio(y, y_ref, t) <= 1.0
