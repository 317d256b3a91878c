"""Pins of the oracle's NF4 codebook, quantizer and dequantizer (CPU only).

What the pages fix (LLM Quantization on RTX 4060, sections "Standard Expectation from
Quantization" and "Kernel Implementation"): 16 unevenly spaced codes for normally distributed
weights, blocks of 64 with one fp32 absmax, high nibble = even element, decoded weight =
code * absmax.  Everything else is pinned by mathematics: the forward normal CDF, exact rational
arithmetic, and closed-form reconstructions.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import nearest_index


def _phi(z: float) -> float:
    return 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))


def test_codebook_shape_and_anchors():
    c = oracle.nf4_codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert np.all(np.diff(c.astype(np.float64)) > 0)
    assert c[0] == -1.0 and c[7] == 0.0 and c[15] == 1.0
    assert int((c < 0).sum()) == 7 and int((c > 0).sum()) == 8


def test_codebook_is_unevenly_spaced():
    gaps = np.diff(nf4 := oracle.nf4_codebook().astype(np.float64))
    assert gaps.max() / gaps.min() > 2.5  # dense near 0, sparse in the tails
    assert np.argmin(gaps) in (7, 6)  # the smallest gap sits at the zero code


def test_codebook_quantiles_by_forward_cdf():
    """Apply the forward normal CDF (math.erf, not the inverse routine the oracle uses) to the
    codes: positive codes sit at 8 evenly spaced probabilities ending at delta, negative codes
    at 7 evenly spaced probabilities, both stepping towards 1/2."""
    c = oracle.nf4_codebook().astype(np.float64)
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    # Scale z such that Phi(z) = delta, found by bisection on the forward CDF.
    lo, hi = 0.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _phi(mid) < delta:
            lo = mid
        else:
            hi = mid
    z = 0.5 * (lo + hi)
    pos = [_phi(v * z) for v in c[8:]]  # ascending
    neg = [_phi(-v * z) for v in c[:7]]  # descending codes -> ascending probabilities
    step_pos = (delta - 0.5) / 8
    step_neg = (delta - 0.5) / 7
    for j, p in enumerate(pos):
        assert abs(p - (0.5 + (j + 1) * step_pos)) < 5e-7, (j, p)
    for j, p in enumerate(neg):
        assert abs(p - (delta - j * step_neg)) < 5e-7, (j, p)


def test_codebook_two_inverse_cdf_routines_agree():
    scipy_stats = pytest.importorskip("scipy.stats")
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    pos = scipy_stats.norm.ppf(np.linspace(delta, 0.5, 9)[:-1])
    neg = -scipy_stats.norm.ppf(np.linspace(delta, 0.5, 8)[:-1])
    alt = (np.sort(np.concatenate([pos, neg, [0.0]])) / scipy_stats.norm.ppf(delta)).astype(np.float32)
    ulps = np.abs(alt.view(np.int32).astype(np.int64) - oracle.nf4_codebook().view(np.int32))
    assert ulps.max() <= 1


def test_codebook_half_precision_error():
    c = oracle.nf4_codebook()
    nz = c[c != 0].astype(np.float64)
    rel16 = np.abs(nz.astype(np.float16).astype(np.float64) - nz) / np.abs(nz)
    assert rel16.max() <= 3.3e-4  # fp16 codes stay well inside a 2e-3 relative bound


def test_midpoints_exact():
    c = oracle.nf4_codebook()
    m = oracle.nf4_midpoints()
    for i in range(15):
        assert Fraction(m[i]) == (Fraction(float(c[i])) + Fraction(float(c[i + 1]))) / 2


def _brute_nf4(w: np.ndarray):
    """Exact-rational NF4 quantizer: nearest code by distance (a different formulation from the
    oracle's midpoint count), ties to the lower index."""
    codes = [float(v) for v in oracle.nf4_codebook()]
    n, k = w.shape
    idx = np.zeros((n, k), dtype=np.uint8)
    absmax = np.zeros((n, k // 64), dtype=np.float32)
    for r in range(n):
        for b in range(k // 64):
            blk = [Fraction(float(v)) for v in w[r, b * 64:(b + 1) * 64]]
            a = max(abs(v) for v in blk)
            absmax[r, b] = float(a)
            for j, v in enumerate(blk):
                idx[r, b * 64 + j] = 7 if a == 0 else nearest_index(v / a, codes)
    packed = (idx[:, 0::2] << 4) | idx[:, 1::2]
    return packed.astype(np.uint8), absmax


@pytest.mark.parametrize("seed,n,k", [(0, 3, 64), (1, 2, 128), (2, 4, 256), (3, 1, 192)])
def test_nf4_brute_force_tiny(seed, n, k):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[0, :8] = 0.0  # a few exact zeros in a non-zero block
    p, a = oracle.quantize_nf4(w)
    bp, ba = _brute_nf4(w)
    assert np.array_equal(p, bp)
    assert np.array_equal(a.view(np.uint32), ba.view(np.uint32))


def test_nf4_ties_go_to_lower_index():
    c = oracle.nf4_codebook()
    m = oracle.nf4_midpoints()
    tested = 0
    for i, mi in enumerate(m):
        if float(np.float32(mi)) != mi:
            continue  # midpoint not representable as an fp32 weight
        w = np.zeros((1, 64), dtype=np.float32)
        w[0, 0] = 1.0  # absmax = 1 exactly
        w[0, 1] = mi
        w[0, 2] = np.nextafter(np.float32(mi), np.float32(2))
        p, _ = oracle.quantize_nf4(w)
        idx = oracle.unpack_nibbles(p)[0]
        assert idx[1] == i, (i, idx[1])
        assert idx[2] == i + 1
        tested += 1
    assert tested >= 3


def test_nf4_absmax_element_and_constant_blocks():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((4, 128)) * 0.02).astype(np.float32)
    w[1, 64:] = 0.03  # constant positive block -> all 15
    w[2, :64] = -0.5  # constant negative block -> all 0
    p, a = oracle.quantize_nf4(w)
    idx = oracle.unpack_nibbles(p)
    assert np.all(idx[1, 64:] == 15) and np.all(idx[2, :64] == 0)
    for r in range(4):
        for b in range(2):
            blk = w[r, b * 64:(b + 1) * 64]
            j = int(np.argmax(np.abs(blk)))
            assert a[r, b] == np.abs(blk).max()
            assert idx[r, b * 64 + j] == (15 if blk[j] > 0 else 0)


def test_nf4_power_of_two_scaling_invariance():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((3, 256)) * 0.02).astype(np.float32)
    p0, a0 = oracle.quantize_nf4(w)
    for e in (-7, 3, 20):
        p1, a1 = oracle.quantize_nf4(w * np.float32(2.0 ** e))
        assert np.array_equal(p0, p1)
        assert np.array_equal(a1, a0 * np.float32(2.0 ** e))


def test_nf4_exact_reconstruction_on_code_points():
    """W built as code[j] * A with A a power of two per block and +-A present: every nibble is j
    and the decoded weights equal W exactly."""
    rng = np.random.default_rng(8)
    c = oracle.nf4_codebook()
    n, k = 5, 320
    j = rng.integers(0, 16, size=(n, k))
    j[:, 0::64] = 15  # every block holds +A ...
    j[:, 1::64] = 0  # ... and -A
    exps = rng.integers(-12, 4, size=(n, k // 64))
    a = np.repeat((2.0 ** exps).astype(np.float32), 64, axis=1)
    w = (c[j] * a).astype(np.float32)
    p, absmax = oracle.quantize_nf4(w)
    assert np.array_equal(oracle.unpack_nibbles(p), j.astype(np.uint8))
    assert np.array_equal(absmax, (2.0 ** exps).astype(np.float32))
    assert np.array_equal(oracle.dequant_nf4(p, absmax), w.astype(np.float64))


def test_nf4_nibble_order_high_is_even_element():
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 0] = 1.0  # code 15
    w[0, 1] = -1.0  # code 0
    w[0, 3] = -1.0  # element 3: low nibble of byte 1
    p, _ = oracle.quantize_nf4(w)
    assert p[0, 0] == 0xF0
    assert p[0, 1] == 0x70


def test_nf4_zero_block_and_negative_zero():
    w = np.zeros((2, 128), dtype=np.float32)
    w[1, :64] = -0.0
    w[1, 64] = 0.25
    w[1, 65] = -0.0
    p, a = oracle.quantize_nf4(w)
    idx = oracle.unpack_nibbles(p)
    assert np.all(idx[0] == 7) and np.all(a[0] == 0)
    assert np.all(idx[1, :64] == 7) and a[1, 0] == 0
    assert idx[1, 65] == 7 and a[1, 1] == np.float32(0.25)


def test_nf4_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_nf4(np.full((1, 64), np.nan, dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_nf4(np.full((1, 64), np.inf, dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_nf4(np.zeros((1, 96), dtype=np.float32))


def test_nf4_dequant_uses_each_blocks_own_scale():
    w = np.zeros((2, 128), dtype=np.float32)
    w[0, :64] = 1.0
    w[0, 64:] = 4.0
    w[1, :64] = -2.0
    w[1, 64:] = 0.5
    p, a = oracle.quantize_nf4(w)
    assert np.array_equal(oracle.dequant_nf4(p, a), w.astype(np.float64))
