"""Pins of the oracle's reference GEMV and acceptance bound (CPU only).

The reference is the plain definition y[b, n] = sum_k x[b, k] W_hat[n, k] (LLM Quantization on
RTX 4060, section "Kernel Implementation").  It is pinned by exact rational sums on tiny inputs,
by one-hot and zero inputs, and by power-of-two diagonal weights whose product is exact.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth_inputs


def _exact_y(x64, w64):
    b, k = x64.shape
    n = w64.shape[0]
    y = np.zeros((b, n))
    t = np.zeros((b, n))
    for i in range(b):
        xs = [Fraction(float(v)) for v in x64[i]]
        for r in range(n):
            terms = [xs[j] * Fraction(float(w64[r, j])) for j in range(k)]
            y[i, r] = float(sum(terms))
            t[i, r] = float(sum(abs(v) for v in terms))
    return y, t


@pytest.mark.parametrize("fmt,xd,n,k,b", [("nf4", "f16", 3, 128, 2), ("nf4", "bf16", 4, 64, 3),
                                         ("int4", "bf16", 2, 256, 3), ("int4", "f16", 3, 128, 1)])
def test_reference_against_exact_sum(fmt, xd, n, k, b):
    w = synth_inputs.weights(n, k, seed=n * 100 + k)
    x = synth_inputs.activations(b, k, xd, seed=b)
    q = oracle.quantize_nf4(w) if fmt == "nf4" else oracle.quantize_int4(w)
    w_hat = oracle.dequant(fmt, *q)
    y, t = oracle.gemv_reference(x, xd, w_hat)
    ye, te = _exact_y(oracle.x_bits_to_f64(x, xd), w_hat)
    assert np.all(np.abs(y - ye) <= k * 2.0 ** -52 * te + 1e-300)
    assert np.allclose(t, te, rtol=k * 2.0 ** -52, atol=0)
    assert y.shape == (b, n)  # a transposed operand would change the shape or the values


def test_reference_one_hot_and_zero():
    w = synth_inputs.weights(6, 192, seed=4)
    w_hat = oracle.dequant("nf4", *oracle.quantize_nf4(w))
    k = 37
    x = np.zeros((1, 192), dtype=np.uint16)
    x[0, k] = 0x3C00  # fp16 1.0
    y, t = oracle.gemv_reference(x, "f16", w_hat)
    assert np.array_equal(y[0], w_hat[:, k])
    y0, t0 = oracle.gemv_reference(np.zeros((2, 192), dtype=np.uint16), "bf16", w_hat)
    assert np.all(y0 == 0) and np.all(t0 == 0)


def test_reference_power_of_two_diagonal():
    """K = N = 128, W = 2^-3 I in NF4 (every block holds A = 2^-3 on its diagonal, code 15) and
    W = 7 * 2^-3 I in INT4: y = x * diag exactly."""
    n = 128
    x = synth_inputs.activations(2, n, "bf16", seed=12)
    x64 = oracle.x_bits_to_f64(x, "bf16")
    w = np.eye(n, dtype=np.float32) * np.float32(0.125)
    w_hat = oracle.dequant("nf4", *oracle.quantize_nf4(w))
    y, _ = oracle.gemv_reference(x, "bf16", w_hat)
    assert np.array_equal(y, x64 * 0.125)
    w = np.eye(n, dtype=np.float32) * np.float32(7 * 0.125)
    w_hat = oracle.dequant("int4", *oracle.quantize_int4(w))
    y, _ = oracle.gemv_reference(x, "bf16", w_hat)
    assert np.array_equal(y, x64 * 0.875)


def test_accept_bound():
    y_ref = np.array([[1.0, -2.0]])
    t = np.array([[10.0, 10.0]])
    assert oracle.accept(y_ref + 0.019, y_ref, t)
    assert not oracle.accept(y_ref + np.array([[0.0, 0.021]]), y_ref, t)
    assert not oracle.accept(np.array([[np.nan, -2.0]]), y_ref, t)


def test_x_bits_conversion():
    assert oracle.f16_bits_to_f64(np.array([0x3C00, 0xC000, 0x0001], dtype=np.uint16)).tolist() == \
        [1.0, -2.0, 2.0 ** -24]
    assert oracle.bf16_bits_to_f64(np.array([0x3F80, 0xC040, 0x0001], dtype=np.uint16)).tolist() == \
        [1.0, -3.0, 2.0 ** -133]
