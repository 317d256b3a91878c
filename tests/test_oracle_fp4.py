"""Pins of the oracle's FP4 (E2M1) format against what the pages and arithmetic fix: the grid
{0, 0.5, 1, 1.5, 2, 3, 4, 6} with a sign bit, the ladder that sends ties to the even code (LLM
Compressor 0.14, section "Details worth knowing"), nearest-grid-point rounding checked by brute
force, the absmax / 6 block scale, exact round trips on the grid, and the nibble order."""
import numpy as np
import pytest

import oracle


def test_codebook_is_the_signed_e2m1_grid():
    c = oracle.fp4_codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert list(c[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert np.array_equal(c[8:], -c[:8]) and np.signbit(c[8])
    # E2M1 read from the bits of each nibble: sign, two exponent bits with bias 1, one mantissa
    # bit, exponent 0 subnormal (0.m x 2^0)
    for n in range(16):
        sign, e, m = n >> 3, (n >> 1) & 3, n & 1
        mag = m * 0.5 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert c[n] == (-mag if sign else mag) and bool(np.signbit(c[n])) == bool(sign)
    # every entry is exact in fp16 and in bf16 (two significant bits at most)
    assert np.array_equal(c.astype(np.float16).astype(np.float32), c)
    assert np.array_equal((c.view(np.uint32) & 0xFFFF0000).view(np.float32), c)


def _brute_index(y):
    """Nearest grid magnitude by exhaustive search; equal distances go to the even index."""
    grid = np.array(oracle.FP4_GRID)
    out = []
    for v in np.ravel(y):
        d = np.abs(grid - v)
        best = np.flatnonzero(d == d.min())
        even = [i for i in best if i % 2 == 0]
        out.append(even[0] if even else best[0])
    return np.array(out, dtype=np.uint8).reshape(np.shape(y))


def test_ladder_ties_go_to_the_even_code():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    assert list(oracle.fp4_magnitude_index(mids)) == [0, 2, 2, 4, 4, 6, 6]
    assert list(oracle.fp4_magnitude_index(np.array(oracle.FP4_GRID))) == list(range(8))


def test_ladder_is_nearest_grid_point_brute_force():
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.uniform(0.0, 7.0, 20000), np.array(oracle.FP4_GRID),
                        [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0],
                        np.nextafter([0.25, 0.75, 5.0], 0.0), np.nextafter([0.25, 0.75, 5.0], 9.0)])
    assert np.array_equal(oracle.fp4_magnitude_index(y), _brute_index(y))


def test_scale_is_absmax_over_six_and_the_max_lands_on_six():
    rng = np.random.default_rng(1)
    w = (rng.standard_normal((8, 256)) * 0.03).astype(np.float32)
    packed, s = oracle.quantize_fp4(w)
    absmax = np.abs(w.reshape(8, 4, 64)).max(axis=2)
    assert np.array_equal(s, (absmax / np.float32(6.0)).astype(np.float32))
    nib = oracle.unpack_nibbles(packed).reshape(8, 4, 64)
    at_max = np.abs(w.reshape(8, 4, 64)) == absmax[..., None]
    assert np.all((nib[at_max] & 7) == 7)


def test_round_trip_on_the_grid_and_error_bound():
    s = np.float32(0.125)  # a power of two: grid * s and absmax / 6 are exact
    grid = np.array(oracle.FP4_GRID, dtype=np.float32)
    row = np.concatenate([grid, -grid] * 4) * s
    row[0] = 6 * s  # the block's absmax is 6 s
    w = np.tile(row, (3, 1)).astype(np.float32)
    packed, sc = oracle.quantize_fp4(w)
    assert np.all(sc == s)
    assert np.array_equal(oracle.dequant_fp4(packed, sc), w.astype(np.float64))
    rng = np.random.default_rng(2)
    w = rng.uniform(-1, 1, (16, 128)).astype(np.float32)
    packed, sc = oracle.quantize_fp4(w)
    err = np.abs(oracle.dequant_fp4(packed, sc) - w)
    bound = np.repeat(sc.astype(np.float64), 64, axis=1)  # half the widest gap (4 -> 6) is 1 * s
    assert np.all(err <= bound * (1 + 1e-6))


def test_zero_blocks_signs_and_nibble_order():
    w = np.zeros((2, 128), dtype=np.float32)
    w[1, 64:] = np.linspace(-1, 1, 64, dtype=np.float32)
    w[1, 64] = -1e-9  # rounds to magnitude 0 with the sign bit: nibble 8
    w[1, 65] = 1.0
    packed, sc = oracle.quantize_fp4(w)
    assert sc[0, 0] == 0 and sc[0, 1] == 0 and sc[1, 0] == 0
    assert np.all(packed[0] == 0) and np.all(packed[1, :32] == 0)
    nib = oracle.unpack_nibbles(packed)
    assert nib[1, 64] == 8 and nib[1, 65] == 7
    assert np.all((nib[1, 64:] >= 8) == (w[1, 64:] < 0))
    # element 2i is the high nibble
    assert packed[1, 32] == (nib[1, 64] << 4 | nib[1, 65])


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.quantize_fp4(np.zeros((2, 96), dtype=np.float32))
    w = np.zeros((1, 64), dtype=np.float32)
    w[0, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_fp4(w)
