"""Pins of the oracle's asymmetric INT4 quantizer (CPU only).

What the pages fix: a code is the scale quotient plus the zero point, clamped and rounded (LLM
Compressor 0.14, section "The fused kernel"), integer rounding is rint, ties to even
(same page, "Details worth knowing"), and INT4 comes symmetric and asymmetric, grouped (same page,
"What those numbers leave out").  The rest is pinned by an exact-rational re-derivation that picks
the nearest grid point by distance (a different formulation from the oracle's divide-add-round),
grids that must round-trip, and the special groups.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import to_bf16, to_f32


def _brute(w: np.ndarray):
    """Exact rationals: range with 0, scale through fp32 and bf16, zero point, and each code as
    the grid point (c - z) s nearest to w by distance, equal distances to the even c."""
    n, k = w.shape
    nib = np.zeros((n, k), dtype=np.uint8)
    scale = np.zeros((n, k // 128))
    zero = np.zeros((n, k // 128), dtype=np.int64)
    for r in range(n):
        for g in range(k // 128):
            grp = [Fraction(float(v)) for v in w[r, g * 128:(g + 1) * 128]]
            lo, hi = min(min(grp), Fraction(0)), max(max(grp), Fraction(0))
            s = to_bf16(to_f32(to_f32(hi - lo) / 15))
            z = 0 if s == 0 else max(0, min(15, round(-lo / s)))  # Fraction round: ties to even
            scale[r, g], zero[r, g] = float(s), z
            for j, v in enumerate(grp):
                if s == 0:
                    c = 0
                else:
                    d = [abs(v - (c - z) * s) for c in range(16)]
                    best = min(d)
                    cands = [c for c in range(16) if d[c] == best]
                    even = [c for c in cands if c % 2 == 0]
                    c = even[0] if even else cands[0]
                nib[r, g * 128 + j] = c
    packed = (nib[:, 0::2] << 4) | nib[:, 1::2]
    return packed.astype(np.uint8), scale, zero


def _fields(words):
    s = oracle.bf16_bits_to_f64((words & 0xFFFF).astype(np.uint16))
    return s, (words >> 16).astype(np.int64)


@pytest.mark.parametrize("seed,n,k,shift", [(0, 2, 128, 0.0), (1, 3, 256, 0.01), (2, 1, 384, -0.03),
                                            (3, 2, 128, 0.05)])
def test_brute_force_tiny(seed, n, k, shift):
    """Gaussian groups, centred and shifted (shifted groups have zero points far from 8)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02 + shift).astype(np.float32)
    p, words = oracle.quantize_int4_asym(w)
    bp, bs, bz = _brute(w)
    s, z = _fields(words)
    assert np.array_equal(s, bs)
    assert np.array_equal(z, bz)
    assert np.array_equal(p, bp)
    assert np.all(words >> 20 == 0)


def test_grid_round_trip_and_zero_point():
    """Weights on a grid (c - z) s with both end codes present recover s, z and every code."""
    s, z = 2.0 ** -6, 5
    codes = np.arange(128) % 16
    w = ((codes - z) * s).astype(np.float32)[None, :]
    p, words = oracle.quantize_int4_asym(w)
    got_s, got_z = _fields(words)
    assert got_s[0, 0] == s and got_z[0, 0] == z
    assert np.array_equal(oracle.unpack_nibbles(p)[0], codes)
    assert np.array_equal(oracle.dequant_int4_asym(p, words), w.astype(np.float64))


def test_ties_round_to_even():
    s, z = 2.0 ** -4, 3
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 0] = (15 - z) * s  # hi: the top code
    w[0, 1] = -z * s        # lo: code 0
    halves = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 4.5])
    w[0, 2:2 + len(halves)] = halves * s
    p, words = oracle.quantize_int4_asym(w)
    got_s, got_z = _fields(words)
    assert got_s[0, 0] == s and got_z[0, 0] == z
    nib = oracle.unpack_nibbles(p)[0, 2:2 + len(halves)]
    v = halves + z  # 3.5 4.5 5.5 6.5 2.5 1.5 0.5 7.5 -> even neighbours
    assert nib.tolist() == [4, 4, 6, 6, 2, 2, 0, 8]
    assert np.all(nib == np.rint(v))
    # the zero point's own tie: range [-2.5 s, 12.5 s] spans exactly 15 s, -lo / s = 2.5 -> 2,
    # and [-3.5 s, 11.5 s] gives 3.5 -> 4
    w = np.zeros((2, 128), dtype=np.float32)
    w[0, 0], w[0, 1] = -2.5 * s, 12.5 * s
    w[1, 0], w[1, 1] = -3.5 * s, 11.5 * s
    _, words = oracle.quantize_int4_asym(w)
    got_s, got_z = _fields(words)
    assert np.all(got_s == s) and got_z[:, 0].tolist() == [2, 4]


def test_special_groups():
    w = np.zeros((4, 256), dtype=np.float32)
    rng = np.random.default_rng(4)
    w[1] = np.abs(rng.standard_normal(256)).astype(np.float32) * 0.1 + 0.01   # all positive
    w[2] = -np.abs(rng.standard_normal(256)).astype(np.float32) * 0.1 - 0.01  # all negative
    w[3] = rng.standard_normal(256).astype(np.float32) * 0.05
    w[3, 7] = 0.0
    w[3, 200] = -0.0
    p, words = oracle.quantize_int4_asym(w)
    s, z = _fields(words)
    assert np.all(words[0] == 0) and np.all(p[0] == 0)      # zero group: s = 0, z = 0, codes 0
    assert np.all(z[1] == 0)                                 # lo = 0
    assert np.all(z[2] == 15)                                # hi = 0
    nib = oracle.unpack_nibbles(p)
    assert nib[3, 7] == z[3, 0] and nib[3, 200] == z[3, 1]   # 0 decodes to exactly 0
    wh = oracle.dequant_int4_asym(p, words)
    assert wh[3, 7] == 0.0 and wh[3, 200] == 0.0
    # error at most about half a step (the bf16 scale and the rounded zero point can pull the
    # top or bottom code inside the range by a little more)
    err = np.abs(wh - w.astype(np.float64))
    step = np.repeat(s, 128, axis=1)
    assert np.all(err <= 0.6 * step + 1e-30)


def test_symmetric_grid_gives_zero_point_eight():
    """A group whose range is [-8 s, 7 s] gets z = 8: the asymmetric code equals the symmetric
    format's stored nibble q + 8 (same scale rule aside)."""
    s = 2.0 ** -5
    q = (np.arange(128) % 16) - 8
    w = (q * s).astype(np.float32)[None, :]
    p, words = oracle.quantize_int4_asym(w)
    got_s, got_z = _fields(words)
    assert got_s[0, 0] == s and got_z[0, 0] == 8
    assert np.array_equal(oracle.unpack_nibbles(p)[0], q + 8)


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_int4_asym(np.zeros((2, 64), dtype=np.float32))
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.quantize_int4_asym(w)
    with pytest.raises(ValueError):
        oracle.dequant_int4_asym(np.zeros((1, 64), np.uint8), np.zeros((1, 2), np.uint32))
