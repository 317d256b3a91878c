"""GPTQ's column loop with lazy blocks, of the oracle.

Test infrastructure only (see the package docstring).

Source: LLM Compressor 0.14: GPTQ's 15x speedup is one fused loop.
  * "The problem GPTQ solves": a layer W [rows x cols] is quantized onto a grid fixed beforehand
    (a scale per row or per group), choosing grid points so as to keep the layer's output on the
    calibration inputs X; the data enters only through H = X X^T.
  * "One weight at a time: the Optimal Brain Surgeon update": rounding one weight, the other
    weights not yet quantized absorb the error along the column of the inverse Hessian, divided by
    its diagonal entry; the inverse then loses that row and column by one step of Gaussian
    elimination.
  * "Three changes that make it fast": one column order (left to right) for every row; the rows of
    the eliminated inverses are the rows of U, the upper Cholesky factor of H^-1, so column j's
    step is e = (w_j - q_j) / U_jj and w_{j+1:} -= e U_{j, j+1:}; lazy blocks of B columns apply
    those updates inside the block, collect the block's errors in E [rows x B], and then update
    the columns to the right once, W[:, i2:] -= E U[i1:i2, i2:]; dampening adds 1% of the mean
    diagonal to H, dead channels get diagonal 1 and zero weights.
  * "The fused kernel": one program per row tile walks the block's columns; each column is
    quantized (scale quotient plus zero point, clamped and rounded, then dequantized), its error
    e = (w - q) / U_jj is kept with q, and e U_j,: comes off the columns to its right.  "Details worth knowing": INT rounding is rint, and the
    kernel avoids fused multiply-adds so that it matches the unfused eager loop bit for bit.

Readings where the pages are silent (each listed in the design notes):
  * The grid is given per row and group: scale s[r, g] and zero point z[r, g] (fp), integer range
    [qmin, qmax]; group g of column j is j // group.  q = rint(clamp(w / s + z, qmin, qmax)),
    q_hat = (q - z) * s; the stored code is q - qmin.  A group with s == 0 takes w / s as 0.
  * ``dtype`` fixes the arithmetic of the column loop: float64 for the algorithm-level checks,
    float32 for parity with the GPU kernels, which take every rounding decision in fp32 with the
    same order of operations (each product rounded, then the subtraction; no fused multiply-add).
  * The lazy update's sum over the block's columns runs in column order:
    t = sum_{c = i1 .. i2-1} E[:, c] U[c, i2:] (each product rounded, then added), W -= t.
"""
from __future__ import annotations

import numpy as np


def dampen(h: np.ndarray, percdamp: float = 0.01):
    """H plus percdamp times its mean diagonal on the diagonal; dead channels (diagonal 0) get
    diagonal 1.  Returns (H_damped, dead mask)."""
    h = np.array(h, dtype=np.float64, copy=True)
    dead = np.diag(h) == 0
    h[dead, dead] = 1.0
    h[np.diag_indices_from(h)] += percdamp * np.mean(np.diag(h))
    return h, dead


def inv_chol_upper(h: np.ndarray, percdamp: float = 0.01):
    """U, the upper Cholesky factor of the inverse of the dampened H (H^-1 = U^T U), in fp64.
    Raises numpy.linalg.LinAlgError when the dampened H is not positive definite."""
    hd, _ = dampen(h, percdamp)
    lower = np.linalg.cholesky(hd)                # H = L L^T
    linv = np.linalg.inv(lower)
    hinv = linv.T @ linv                           # H^-1 = L^-T L^-1
    return np.linalg.cholesky(hinv).T              # upper: H^-1 = U^T U


def quantize_column(w, s, z, qmin, qmax, dtype):
    """q = rint(clamp(w / s + z, qmin, qmax)) and q_hat = (q - z) s, every step in ``dtype``.
    Returns (q_hat, code) with code = q - qmin."""
    w = np.asarray(w, dtype=dtype)
    s = np.asarray(s, dtype=dtype)
    z = np.asarray(z, dtype=dtype)
    safe = np.where(s != 0, s, dtype(1))
    v = np.where(s != 0, w / safe, dtype(0))
    v = v + z
    v = np.minimum(np.maximum(v, dtype(qmin)), dtype(qmax))
    q = np.rint(v)
    q_hat = (q - z) * s
    return q_hat.astype(dtype), (q - qmin).astype(np.int64)


def gptq(w, u, scale, zero, qmin, qmax, group=None, block=128, dtype=np.float64, dead=None):
    """Quantize W [rows x cols] column by column with error feedback through U (upper, cols x cols),
    lazy blocks of ``block`` columns.  scale, zero: [rows, cols // group] (group defaults to cols:
    one grid per row).  Returns dict(q_hat, codes, err, w_final) where err[:, j] is column j's
    e = (w_j - q_j) / U_jj and w_final the weights after every update."""
    dtype = np.dtype(dtype).type
    w = np.array(w, dtype=dtype, copy=True)
    u = np.asarray(u, dtype=dtype)
    rows, cols = w.shape
    group = cols if group is None else group
    scale = np.asarray(scale, dtype=dtype).reshape(rows, -1)
    zero = np.asarray(zero, dtype=dtype).reshape(rows, -1)
    if scale.shape[1] != cols // group or cols % group:
        raise ValueError("scale / zero must be [rows, cols // group]")
    if dead is not None:
        w[:, dead] = 0
    q_hat = np.zeros_like(w)
    codes = np.zeros((rows, cols), dtype=np.int64)
    err = np.zeros_like(w)
    for i1 in range(0, cols, block):
        i2 = min(i1 + block, cols)
        for j in range(i1, i2):
            g = j // group
            q_hat[:, j], codes[:, j] = quantize_column(w[:, j], scale[:, g], zero[:, g], qmin, qmax,
                                                       dtype)
            e = (w[:, j] - q_hat[:, j]) / u[j, j]
            err[:, j] = e
            # rank-one update of the block's columns to the right (product rounded, then the
            # subtraction)
            w[:, j + 1:i2] = w[:, j + 1:i2] - np.outer(e, u[j, j + 1:i2])
        if i2 < cols:
            t = np.zeros((rows, cols - i2), dtype=dtype)
            for c in range(i1, i2):
                t = t + np.outer(err[:, c], u[c, i2:])
            w[:, i2:] = w[:, i2:] - t
    return {"q_hat": q_hat, "codes": codes, "err": err, "w_final": w}


def rtn(w, scale, zero, qmin, qmax, group=None, dtype=np.float64):
    """Round to nearest on the same grid (no error feedback): GPTQ with a diagonal H."""
    w = np.asarray(w, dtype=dtype)
    rows, cols = w.shape
    group = cols if group is None else group
    scale = np.asarray(scale, dtype=dtype).reshape(rows, -1)
    zero = np.asarray(zero, dtype=dtype).reshape(rows, -1)
    g = np.arange(cols) // group
    return quantize_column(w, scale[:, g], zero[:, g], qmin, qmax, np.dtype(dtype).type)


def proxy_loss(w, q_hat, h):
    """The objective GPTQ minimizes: sum over rows of delta H delta^T, delta = w - q_hat."""
    d = np.asarray(w, dtype=np.float64) - np.asarray(q_hat, dtype=np.float64)
    return float(np.einsum("ri,ij,rj->", d, np.asarray(h, dtype=np.float64), d))
