"""GPU quantizers against the oracle, bit for bit (packed nibbles and scales)."""
import numpy as np
import pytest

import oracle
import synth_inputs
from tests import gpu_util as g

pytestmark = pytest.mark.gpu

FMTS = ["nf4_f16", "int4_f16", "fp4_f16", "int4a_f16"]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k,seed", [(256, 1536, 0), (37, 384, 1), (1, 128, 2), (1536, 8960, 3),
                                      (129, 8192, 4)])
def test_quantize_bitexact_gaussian(fmt, n, k, seed):
    w = synth_inputs.weights(n, k, seed=seed)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    g.assert_quant_equal(fmt, p, s, *g.oracle_quantize(fmt, w))


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_edge_values(fmt):
    """Zero blocks, -0.0, denormals, huge magnitudes, constant blocks, exact ties (NF4, INT4 and
    FP4 midpoints; asymmetric INT4 codes and zero points), one-signed groups."""
    rng = np.random.default_rng(21)
    w = (rng.standard_normal((12, 256)) * 0.02).astype(np.float32)
    w[0] = 0.0
    w[1, :128] = -0.0
    w[2] = rng.standard_normal(256).astype(np.float32) * np.float32(1e-39)  # fp32 denormals
    w[3] = rng.standard_normal(256).astype(np.float32) * np.float32(1e37)
    w[4] = np.float32(0.75)
    w[5, ::2] = np.float32(2.0 ** -140)
    w[5, 1::2] = -np.float32(2.0 ** -141)
    # NF4 ties: absmax 1 and representable midpoints; INT4 ties: s = 1 and half-integers
    mids = [m for m in oracle.nf4_midpoints() if float(np.float32(m)) == m]
    w[6] = 0.0
    w[6, 0] = 1.0
    w[6, 1:1 + len(mids)] = mids
    w[6, 128] = 7.0
    w[6, 129:137] = [0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 6.5]
    w[7] = rng.integers(-7, 8, 256).astype(np.float32) * np.float32(2.0 ** -5)
    w[7, ::128] = 7 * 2.0 ** -5
    # FP4 ties: absmax 6 gives s = 1, so the ladder's midpoints are exact ties; absmax 3 gives
    # s = 0.5 and the same ties at half the size
    w[8] = 0.0
    w[8, 0] = 6.0
    w[8, 1:8] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    w[8, 8:15] = [-0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0]
    w[8, 64] = -3.0
    w[8, 65:72] = [0.125, 0.375, 0.625, 0.875, 1.25, 1.75, 2.5]
    # asymmetric INT4: all-positive and all-negative groups (zero points 0 and 15), and zero-point
    # ties: ranges [-2.5 s, 12.5 s] and [-3.5 s, 11.5 s] with s = 2^-4
    w[9, :128] = np.abs(w[9, :128]) + np.float32(0.01)
    w[9, 128:] = -np.abs(w[9, 128:]) - np.float32(0.01)
    w[10] = 0.0
    w[10, 0], w[10, 1], w[10, 2:10] = -2.5 / 16, 12.5 / 16, np.arange(8) / 16 + 1 / 32
    w[10, 128], w[10, 129], w[10, 130:138] = -3.5 / 16, 11.5 / 16, -np.arange(8) / 16 - 1 / 32
    w = np.ascontiguousarray(w)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    g.assert_quant_equal(fmt, p, s, *g.oracle_quantize(fmt, w))


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_rejects_nonfinite(fmt):
    import bit_weight_only_w4_amd as w4

    for bad in (np.nan, np.inf, -np.inf):
        w = synth_inputs.weights(4, 256, seed=5)
        w[2, 77] = bad
        with pytest.raises(w4.W4ValueError) as e:
            g.gpu_quantize(fmt, g.to_dev_f32(w))
        assert e.value.status == -5
    # the error word is cleared by the next call
    w = synth_inputs.weights(4, 256, seed=5)
    g.gpu_quantize(fmt, g.to_dev_f32(w))


def test_quantize_lm_head_sampled_rows():
    """Full 151936 x 1536 matrix quantized on the GPU; 96 sampled rows compared bit for bit."""
    n, k = synth_inputs.QWEN15_LM_HEAD[1:]
    w = synth_inputs.weights(n, k, seed=999)
    wd = g.to_dev_f32(w)
    rows = np.sort(np.random.default_rng(1).choice(n, 94, replace=False))
    rows = np.concatenate([[0], rows, [n - 1]])
    for fmt in FMTS:
        p, s = g.gpu_quantize(fmt, wd)
        g.assert_quant_equal(fmt, p, s, *g.oracle_quantize(fmt, w[rows]), rows=rows)
