"""GPTQ's column loop with lazy blocks, of the oracle.

Test infrastructure only (see the package docstring).

Source: LLM Compressor 0.14: GPTQ's 15x speedup is one fused loop.
  * "The problem GPTQ solves": a layer W [rows x cols] is rounded onto a grid fixed beforehand (a
    scale per row or per group) so as to keep the layer's output on calibration inputs X; the data
    enters only through H = X X^T.
  * "One weight at a time: the Optimal Brain Surgeon update": after one weight is rounded, the
    weights not yet rounded absorb its error along that weight's row of the inverse Hessian,
    divided by the row's diagonal entry, and the inverse loses that row and column by one step of
    Gaussian elimination.
  * "Three changes that make it fast": every row takes the columns in one order (left to right);
    the successive eliminated inverses' rows, divided by the square root of their diagonal, are
    the rows of U, the upper triangular factor with H^-1 = U^T U, so column j's error is
    (w_j - q_j) / U_jj and column c > j takes that error times U_jc off its weight; within a lazy
    block those updates are applied one column at a time, and each block's errors reach the
    columns to its right in one accumulated update; dampening adds 1% of the mean diagonal to H,
    and dead channels (diagonal 0) get diagonal 1 and zero weights.
  * "The fused kernel" gives the order of one column's steps (scale quotient, zero point, clamp,
    rounding, dequantization, error); "Details worth knowing": integer rounding is rint, and the
    fused kernel avoids fused multiply-adds so that its bits match the unfused loop.

Readings where the pages are silent (each listed in the design notes):
  * The grid is given per row and group: scale s[r, g] and zero point z[r, g] (fp), integer range
    [qmin, qmax]; column j belongs to group j // group.  q = rint(clamp(w / s + z, qmin, qmax)),
    q_hat = (q - z) * s; the stored code is q - qmin.  A group with s == 0 takes w / s as 0.
  * ``dtype`` fixes the arithmetic: float64 for the algorithm-level checks, float32 for parity
    with the GPU kernels, which round every product before subtracting it (no fused multiply-add).
  * Order of the subtractions reaching column c (inside block k): first one correction per earlier
    block, in block order, each the sum over that block's columns in column order (every product
    rounded, the sum started from +0 and rounded after each addition); then the corrections of
    block k's earlier columns one at a time, in column order.

Structure: ``inverse_factor`` builds U by the Gaussian elimination the OBS section describes;
``grid_point`` is one quantization step; ``gptq`` walks the blocks, solving each block column by
column from the left (each column gathers the corrections of the block's earlier columns just before
it is rounded) and then handing the block's accumulated correction to every column to its right.
"""
from __future__ import annotations

import numpy as np


def dampened(h: np.ndarray, damp: float = 0.01):
    """(H with dead channels set to diagonal 1 and ``damp`` times the mean diagonal added to the
    diagonal, dead-channel mask), fp64."""
    hd = np.array(h, dtype=np.float64, copy=True)
    diag = np.diagonal(hd).copy()
    dead = diag == 0
    diag[dead] = 1.0
    diag = diag + damp * float(np.mean(diag))
    np.fill_diagonal(hd, diag)
    return hd, dead


def inverse_factor(h: np.ndarray, damp: float = 0.01) -> np.ndarray:
    """U [cols x cols], upper triangular with H_d^-1 = U^T U (H_d = the dampened H), built as the
    OBS section states it: row j of U is row j of the inverse after eliminating columns 0..j-1,
    from column j on, divided by the square root of its diagonal entry.  fp64.  Raises
    numpy.linalg.LinAlgError when H_d is not positive definite (its smallest eigenvalue at most
    cols * eps times its largest) or an eliminated diagonal is not positive."""
    hd, _ = dampened(h, damp)
    eig = np.linalg.eigvalsh(hd)
    if not eig[0] > hd.shape[0] * np.finfo(np.float64).eps * eig[-1]:
        raise np.linalg.LinAlgError("dampened H is not positive definite")
    cur = np.linalg.inv(hd)
    n = cur.shape[0]
    out = np.zeros_like(cur)
    for j in range(n):
        pivot = cur[j, j]
        if not pivot > 0:
            raise np.linalg.LinAlgError(f"eliminated inverse not positive definite at column {j}")
        out[j, j:] = cur[j, j:] / np.sqrt(pivot)
        # drop column j from the inverse: one step of Gaussian elimination
        cur = cur - np.outer(cur[:, j], cur[j, :]) / pivot
    return out


def grid_point(w, s, z, qmin, qmax, dtype):
    """One quantization step in ``dtype``: v = w / s (0 where s == 0), v + z, clamped to
    [qmin, qmax], rounded half to even; q_hat = (q - z) * s.  Returns (q_hat, code = q - qmin)."""
    w = np.asarray(w, dtype=dtype)
    s = np.asarray(s, dtype=dtype)
    z = np.asarray(z, dtype=dtype)
    ratio = np.divide(w, s, out=np.zeros_like(w), where=(s != 0))
    shifted = np.clip(ratio + z, dtype(qmin), dtype(qmax))
    q = np.rint(shifted)
    q_hat = (q - z) * s
    return q_hat.astype(dtype), (q - qmin).astype(np.int64)


def gptq(w, u, scale, zero, qmin, qmax, group=None, block=128, dtype=np.float64, dead=None):
    """Round W [rows x cols] column by column with error feedback through U (upper, cols x cols),
    in lazy blocks of ``block`` columns.  scale, zero: [rows, cols // group] (group defaults to
    cols: one grid per row).  Returns dict(q_hat, codes, err, w_final): err[:, j] = (v_j - q_hat_j)
    / U_jj where v_j is column j as it stands when it is rounded, and w_final[:, j] = v_j."""
    dt = np.dtype(dtype).type
    cur = np.array(w, dtype=dt, copy=True)  # columns not yet rounded receive corrections here
    u = np.asarray(u, dtype=dt)
    rows, cols = cur.shape
    group = cols if group is None else group
    if cols % group:
        raise ValueError("cols must be a multiple of group")
    scale = np.asarray(scale, dtype=dt).reshape(rows, -1)
    zero = np.asarray(zero, dtype=dt).reshape(rows, -1)
    if scale.shape[1] != cols // group or zero.shape != scale.shape:
        raise ValueError("scale / zero must be [rows, cols // group]")
    if dead is not None:
        cur[:, np.asarray(dead, dtype=bool)] = 0
    q_hat = np.zeros_like(cur)
    codes = np.zeros((rows, cols), dtype=np.int64)
    err = np.zeros_like(cur)

    for start in range(0, cols, block):
        stop = min(start + block, cols)
        # inside the block: each column takes the corrections of the block's earlier columns, one
        # at a time in column order, then is rounded and yields its own error
        for c in range(start, stop):
            v = cur[:, c]
            for prev in range(start, c):
                v = v - err[:, prev] * u[prev, c]
            cur[:, c] = v
            gi = c // group
            q_hat[:, c], codes[:, c] = grid_point(v, scale[:, gi], zero[:, gi], qmin, qmax, dt)
            err[:, c] = (v - q_hat[:, c]) / u[c, c]
        # the block's correction of every column to its right, summed over the block's columns
        # in column order from +0, subtracted once
        if stop < cols:
            corr = np.zeros((rows, cols - stop), dtype=dt)
            for prev in range(start, stop):
                corr = corr + err[:, prev:prev + 1] * u[prev:prev + 1, stop:]
            cur[:, stop:] = cur[:, stop:] - corr
    return {"q_hat": q_hat, "codes": codes, "err": err, "w_final": cur}


def rtn(w, scale, zero, qmin, qmax, group=None, dtype=np.float64):
    """Round to nearest on the same grid (no error feedback): GPTQ with a diagonal H."""
    w = np.asarray(w, dtype=dtype)
    rows, cols = w.shape
    group = cols if group is None else group
    scale = np.asarray(scale, dtype=dtype).reshape(rows, -1)
    zero = np.asarray(zero, dtype=dtype).reshape(rows, -1)
    gi = np.arange(cols) // group
    return grid_point(w, scale[:, gi], zero[:, gi], qmin, qmax, np.dtype(dtype).type)


def proxy_loss(w, q_hat, h):
    """The objective GPTQ minimizes: sum over rows of delta H delta^T, delta = w - q_hat."""
    d = np.asarray(w, dtype=np.float64) - np.asarray(q_hat, dtype=np.float64)
    return float(np.einsum("ri,ij,rj->", d, np.asarray(h, dtype=np.float64), d))
