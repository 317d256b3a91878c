"""Pins of the oracle's symmetric INT4 quantizer (CPU only).

What the pages fix: a +8 zero point, without which every positive weight is destroyed (My Triton
Kernel Ties bitsandbytes, section "The kernels"); integer rounding with rint, i.e. ties to even
(LLM Compressor 0.14, section "Details worth knowing").  The rest is pinned by an exact-rational
re-derivation and by grids that must round-trip.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests.exact import to_bf16, to_f32


def test_bf16_rne_special_values():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, 0.0],
                 dtype=np.float32)
    got = oracle.bf16_bits_to_f64(oracle.f32_to_bf16_rne_bits(v))
    assert got.tolist() == [1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 0.0]


def test_bf16_rne_matches_exact_rounding():
    rng = np.random.default_rng(11)
    v = np.concatenate([rng.standard_normal(2000).astype(np.float32) * 1e-3,
                        np.float32(2.0 ** -133) * rng.integers(1, 300, 50).astype(np.float32)])
    got = oracle.bf16_bits_to_f64(oracle.f32_to_bf16_rne_bits(v))
    want = [float(to_bf16(Fraction(float(t)))) for t in v]
    assert got.tolist() == want


def _brute_int4(w: np.ndarray):
    n, k = w.shape
    nib = np.zeros((n, k), dtype=np.uint8)
    scale = np.zeros((n, k // 128))
    for r in range(n):
        for g in range(k // 128):
            grp = [Fraction(float(v)) for v in w[r, g * 128:(g + 1) * 128]]
            a = max(abs(v) for v in grp)
            s = to_bf16(to_f32(a / 7))
            scale[r, g] = float(s)
            for j, v in enumerate(grp):
                if s == 0:
                    q = 0
                else:
                    q = max(-8, min(7, round(v / s)))  # Fraction.__round__: ties to even
                nib[r, g * 128 + j] = q + 8
    packed = (nib[:, 0::2] << 4) | nib[:, 1::2]
    return packed.astype(np.uint8), scale


@pytest.mark.parametrize("seed,n,k", [(0, 2, 128), (1, 3, 256), (2, 1, 384)])
def test_int4_brute_force_tiny(seed, n, k):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    p, s_bits = oracle.quantize_int4(w)
    bp, bs = _brute_int4(w)
    assert np.array_equal(p, bp)
    assert np.array_equal(oracle.bf16_bits_to_f64(s_bits), bs)


def test_int4_grid_round_trip_plus_eight():
    """W = q * 2^e with +-7 * 2^e present in every group: s = 2^e exactly, nibble = q + 8,
    positive weights -> 9..15, negative -> 1..7, zero -> 8, and W_hat == W."""
    rng = np.random.default_rng(3)
    n, k = 4, 512
    q = rng.integers(-7, 8, size=(n, k))
    q[:, 0::128] = 7
    q[:, 1::128] = -7
    e = rng.integers(-10, 2, size=(n, k // 128))
    s = np.repeat(2.0 ** e, 128, axis=1)
    w = (q * s).astype(np.float32)
    p, s_bits = oracle.quantize_int4(w)
    nib = oracle.unpack_nibbles(p).astype(np.int64)
    assert np.array_equal(nib, q + 8)
    assert np.all(nib[w > 0] >= 9) and np.all(nib[w < 0] <= 7) and np.all(nib[w == 0] == 8)
    assert np.array_equal(oracle.bf16_bits_to_f64(s_bits), 2.0 ** e)
    assert np.array_equal(oracle.dequant_int4(p, s_bits), w.astype(np.float64))


def test_int4_ties_round_to_even():
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 0] = 7.0  # s = 1 exactly
    halves = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, -3.5, 6.5, -6.5]
    w[0, 1:1 + len(halves)] = halves
    p, s_bits = oracle.quantize_int4(w)
    assert oracle.bf16_bits_to_f64(s_bits)[0, 0] == 1.0
    q = oracle.unpack_nibbles(p)[0, 1:1 + len(halves)].astype(int) - 8
    assert q.tolist() == [0, 2, 2, 4, 0, -2, -2, -4, 6, -6]


def test_int4_zero_and_underflowing_groups():
    w = np.zeros((1, 256), dtype=np.float32)
    w[0, 128] = np.float32(2.0 ** -140)  # absmax / 7 rounds to 0 in bf16
    w[0, 129] = -np.float32(2.0 ** -141)
    p, s_bits = oracle.quantize_int4(w)
    assert np.all(s_bits == 0)
    assert np.all(oracle.unpack_nibbles(p) == 8)


def test_int4_nibble_order_matches_nf4():
    w = np.zeros((1, 128), dtype=np.float32)
    w[0, 0] = 7.0
    w[0, 1] = -7.0
    p, _ = oracle.quantize_int4(w)
    assert p[0, 0] == 0xF1  # element 0 -> high nibble (7 + 8), element 1 -> low nibble (-7 + 8)


def test_int4_clamp_never_engages_with_absmax_over_7():
    rng = np.random.default_rng(9)
    w = (rng.standard_normal((64, 1024)) * 0.02).astype(np.float32)
    p, _ = oracle.quantize_int4(w)
    nib = oracle.unpack_nibbles(p)
    assert nib.min() >= 1 and nib.max() <= 15


def test_int4_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_int4(np.full((1, 128), np.inf, dtype=np.float32))
    with pytest.raises(ValueError):
        oracle.quantize_int4(np.zeros((1, 64), dtype=np.float32))
