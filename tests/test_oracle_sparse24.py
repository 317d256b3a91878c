"""Pins of the oracle's 2:4 sparse format (CPU only): the byte count the page prints (56.25% of
dense fp16), the kept positions against a brute-force count of stronger neighbours, the metadata
layout the page's kernel reads (even group in the low nibble, first position in the low two bits),
exact round trips of weights that are already 2:4 sparse, and the product computed group by group
from the stored values and codes, the way the page's kernel walks them."""
import numpy as np
import pytest

from oracle import sparse24 as S
from oracle.gemv import gemv_reference


def test_bytes_are_56_25_percent_of_dense_fp16():
    # Do Quantization and Sparsity make LLM Inference Faster?, "Library 2:4 sparsity"
    for n, k in [(1536, 1536), (256, 1536), (8960, 1536), (1536, 8960), (151936, 1536)]:
        assert S.sparse_bytes(n, k) / (n * k * 2) == 0.5625
    v, m = S.compress_2to4(np.ones((3, 64), dtype=np.float32))
    assert v.nbytes + m.nbytes == 0.5625 * 3 * 64 * 2


def _brute_keep(w):
    """Kept iff fewer than two others in the group beat it (larger magnitude, or equal magnitude
    at a lower position)."""
    n, k = w.shape
    keep = np.zeros((n, k), dtype=bool)
    for r in range(n):
        for g in range(k // 4):
            a = [abs(float(w[r, 4 * g + i])) for i in range(4)]
            for i in range(4):
                beaten = sum(1 for j in range(4) if j != i and (a[j] > a[i] or (a[j] == a[i] and j < i)))
                keep[r, 4 * g + i] = beaten < 2
    return keep


@pytest.mark.parametrize("seed", [0, 1])
def test_kept_positions_brute_force(seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((6, 64)).astype(np.float32)
    # plenty of ties: magnitudes from a small set, random signs
    w[3:] = (rng.integers(0, 3, (3, 64)) * rng.choice([-1, 1], (3, 64))).astype(np.float32)
    v, m = S.compress_2to4(w)
    dense = S.dense_from_2to4(v, m)
    keep = _brute_keep(w)
    assert np.array_equal(dense != 0, keep & (w != 0))
    expect = np.where(keep, w.astype(np.float16).astype(np.float64), 0.0)
    assert np.array_equal(dense, expect)


def test_metadata_layout():
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0:4] = [0.0, 5.0, 0.0, -7.0]   # group 0 keeps positions 1, 3 -> code 1 | 3 << 2 = 0xD
    w[0, 4:8] = [9.0, 0.0, 8.0, 0.0]    # group 1 keeps 0, 2 -> code 0 | 2 << 2 = 0x8
    w[0, 8:12] = [1.0, 1.0, 1.0, 1.0]   # all tied: positions 0, 1 -> code 0x4
    v, m = S.compress_2to4(w)
    assert m[0, 0] == 0xD | (0x8 << 4)
    assert m[0, 1] & 0xF == 0x4
    assert v[0, :6].view(np.float16).tolist() == [5.0, -7.0, 9.0, 8.0, 1.0, 1.0]


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_round_trip_of_2to4_weights(xdt):
    rng = np.random.default_rng(3)
    w = rng.integers(-64, 64, (5, 128)).astype(np.float32) / 8  # exact in both 16-bit types
    g = w.reshape(5, 32, 4)
    for r in range(5):
        for j in range(32):
            g[r, j, rng.choice(4, 2, replace=False)] = 0  # two zeros per group
    v, m = S.compress_2to4(w, xdt)
    assert np.array_equal(S.dense_from_2to4(v, m, xdt), w.astype(np.float64))


def test_product_group_by_group():
    """y from the stored values and codes, walking each group's two kept values against the
    activations at their positions, equals x times the decoded dense matrix."""
    rng = np.random.default_rng(4)
    w = rng.standard_normal((7, 96)).astype(np.float32)
    xb = rng.standard_normal((2, 96)).astype(np.float16).view(np.uint16)
    v, m = S.compress_2to4(w)
    x = xb.view(np.float16).astype(np.float64)
    vals = v.view(np.float16).astype(np.float64)
    y = np.zeros((2, 7))
    for r in range(7):
        for g in range(96 // 4):
            code = (m[r, g >> 1] >> 4) if (g & 1) else (m[r, g >> 1] & 0x0F)
            i0, i1 = code & 3, (code >> 2) & 3
            y[:, r] += vals[r, 2 * g] * x[:, 4 * g + i0] + vals[r, 2 * g + 1] * x[:, 4 * g + i1]
    ref, _ = gemv_reference(xb, "f16", S.dense_from_2to4(v, m))
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        S.compress_2to4(np.zeros((2, 48), dtype=np.float32))
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 3] = np.inf
    with pytest.raises(ValueError):
        S.compress_2to4(w)
