"""Asymmetric INT4 with zero points far from 8: weights shifted to one side of 0, so that the
zero-point term -(z - 8) * s * sum(x) of every kernel carries most of the result.  Each path
against the oracle's fp64 reference (per element, 2e-3 T + 1e-5), after a bit-exact check of the
GPU quantizer."""
import numpy as np
import pytest

import synth_inputs
from tests import gpu_util as g

pytestmark = pytest.mark.gpu

FMTS = ["int4a_f16", "int4a_bf16"]


def _case(fmt, n, k, b, seed, shift):
    w = synth_inputs.weights(n, k, sigma=0.02, seed=seed) + np.float32(shift)
    w = np.ascontiguousarray(w, dtype=np.float32)
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=seed + 7)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    g.assert_quant_equal(fmt, p, s, pr, sr)
    z = (sr >> 16) & 15
    return x, g.to_dev_x(x, g.XDT[fmt]), p, s, pr, sr, z


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("shift", [0.03, -0.05, 0.2])
@pytest.mark.parametrize("path,n,k,b", [("gemv", 300, 1536, 1), ("gemv", 129, 8960, 3),
                                        ("gemv", 70, 384, 8), ("mfma", 130, 1536, 16),
                                        ("mfma", 77, 2048, 64), ("tiled", 300, 1536, 200),
                                        ("tiled", 129, 640, 128), ("twopass", 90, 1536, 5)])
def test_shifted_weights_every_path(fmt, shift, path, n, k, b):
    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr, z = _case(fmt, n, k, b, seed=n + k + b, shift=shift)
    # the shift moves the zero points to one end of the code range
    assert (np.mean(z) < 5) if shift > 0 else (np.mean(z) > 10)
    ws = None
    if path == "twopass":
        import torch

        ws = torch.empty(w4.workspace_bytes(fmt, n, k, b, "twopass"), dtype=torch.uint8,
                         device=g.device())
    y = w4.matmul_ex(xd, p, s, fmt, path=path, workspace=ws)
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", FMTS)
def test_splitk_and_grouped_shifted(fmt):
    import torch

    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr, _ = _case(fmt, 1536, 8960, 2, seed=3, shift=0.04)
    ws = torch.empty(w4.workspace_bytes(fmt, 1536, 8960, 2, "splitk", 4), dtype=torch.uint8,
                     device=g.device())
    y = w4.matmul_ex(xd, p, s, fmt, path="splitk", split_k=4, workspace=ws)
    g.assert_y_close(fmt, y, x, pr, sr)
    # grouped: members with different shifts (zero points near 0, near 15, near 8)
    k = 1536
    members = []
    for i, (n, shift) in enumerate([(1536, 0.05), (256, -0.05), (256, 0.0)]):
        w = np.ascontiguousarray(synth_inputs.weights(n, k, seed=40 + i) + np.float32(shift),
                                 dtype=np.float32)
        pg, sg = g.gpu_quantize(fmt, g.to_dev_f32(w))
        members.append((pg, sg, *g.oracle_quantize(fmt, w)))
    for b in (1, 8):
        xb = synth_inputs.activations(b, k, g.XDT[fmt], seed=b)
        ys = w4.gemm_smallbatch_grouped(g.to_dev_x(xb, g.XDT[fmt]), [m[0] for m in members],
                                        [m[1] for m in members], fmt)
        for (pg, sg, pr_, sr_), yg in zip(members, ys):
            g.assert_y_close(fmt, yg, xb, pr_, sr_)


@pytest.mark.parametrize("fmt", FMTS)
def test_one_hot_exact(fmt):
    """x = e_j: every path returns column j of the decoded matrix, (q - z) s, exactly (the
    zero-point term is -(z - 8) s and the codes q - 8 are exact in both 16-bit types)."""
    import oracle

    import bit_weight_only_w4_amd as w4

    n, k = 200, 1024
    w = np.ascontiguousarray(synth_inputs.weights(n, k, seed=9) + np.float32(0.03), dtype=np.float32)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    w_hat = oracle.dequant("int4a", pr, sr)
    one = 0x3C00 if g.XDT[fmt] == "f16" else 0x3F80
    for path, b in (("gemv", 1), ("mfma", 16), ("tiled", 128)):
        xb = np.zeros((b, k), dtype=np.uint16)
        cols = [(7 * i + 300) % k for i in range(b)]
        for i, c in enumerate(cols):
            xb[i, c] = one
        y = w4.matmul_ex(g.to_dev_x(xb, g.XDT[fmt]), p, s, fmt, path=path).cpu().numpy()
        for i, c in enumerate(cols):
            assert np.array_equal(y[i].astype(np.float64), w_hat[:, c]), (path, i)
