"""MFMA small-batch path against the oracle's fp64 reference (per element, 2e-3 T + 1e-5)."""
import pytest

import synth_inputs
from tests import gpu_util as g

pytestmark = pytest.mark.gpu

ALL_FMTS = ["nf4_f16", "nf4_bf16", "int4_f16", "int4_bf16", "fp4_f16", "fp4_bf16", "int4a_f16",
            "int4a_bf16"]


def _case(fmt, n, k, b, seed):
    w = synth_inputs.weights(n, k, seed=seed)
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=seed + 17)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    g.assert_quant_equal(fmt, p, s, pr, sr)
    return x, g.to_dev_x(x, g.XDT[fmt]), p, s, pr, sr


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("n,k,b", [(64, 256, 16), (37, 384, 9), (100, 1536, 32), (256, 1536, 17),
                                   (130, 8960, 64), (513, 1536, 128), (65, 2048, 129),
                                   (96, 1024, 200), (200, 8192, 48)])
def test_mfma_parity(fmt, n, k, b):
    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=n * 7 + b)
    y = w4.matmul_ex(xd, p, s, fmt, path="mfma")
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ["nf4_f16", "nf4_bf16", "fp4_f16", "fp4_bf16"])
@pytest.mark.parametrize("n,k,b", [(70, 192, 16), (129, 320, 33), (40, 64, 4)])
def test_mfma_odd_block_count(fmt, n, k, b):
    """64-weight-block formats with an odd number of blocks per row (K % 128 == 64)."""
    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=n * 5 + k + b)
    y = w4.matmul_ex(xd, p, s, fmt, path="mfma")
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ["nf4_f16", "int4_bf16"])
def test_smallbatch_auto_uses_both_paths(fmt):
    """w4_gemm_smallbatch at B = 3 (GEMV) and B = 4, 32 (MFMA) on the gate shape."""
    import bit_weight_only_w4_amd as w4

    for b in (3, 4, 32):
        x, xd, p, s, pr, sr = _case(fmt, 8960, 1536, b, seed=b)
        assert w4.auto_path(fmt, 8960, 1536, b)[0] == ("gemv" if b <= 3 else "mfma")
        y = w4.gemm_smallbatch(xd, p, s, fmt)
        g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ["nf4_f16", "nf4_bf16"])
def test_mfma_deterministic(fmt):
    import torch

    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, 300, 1536, 40, seed=3)
    y1 = w4.matmul_ex(xd, p, s, fmt, path="mfma")
    y2 = w4.matmul_ex(xd, p, s, fmt, path="mfma")
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("fmt,n,k,b", [("nf4_f16", 151936, 1536, 8), ("nf4_bf16", 151936, 1536, 128),
                                       ("int4_f16", 1536, 8960, 8), ("int4_bf16", 8960, 1536, 32),
                                       ("nf4_f16", 28672, 8192, 16), ("fp4_f16", 8960, 1536, 32),
                                       ("fp4_bf16", 151936, 1536, 8), ("int4a_f16", 8960, 1536, 64),
                                       ("int4a_bf16", 1536, 8960, 8), ("int4_f16", 28672, 8192, 4),
                                       ("int4a_bf16", 28672, 8192, 16)])
def test_mfma_full_size_sampled(fmt, n, k, b):
    """Full-size matrices (persistent grids with several row tiles per workgroup, K groups, x
    windows in several phases): weights drawn on the GPU, quantized there, and 160 sampled rows
    (the first and the last among them) checked against the oracle."""
    import numpy as np
    import torch

    import bit_weight_only_w4_amd as w4

    dev = g.device()
    gen = torch.Generator(device=dev).manual_seed(n + 3 * k + b)
    w = torch.randn(n, k, generator=gen, device=dev) * 0.02
    p, s = g.gpu_quantize(fmt, w)
    rng = np.random.default_rng(n + b)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 158, replace=False)]))
    w_rows = w[torch.as_tensor(rows, device=dev)].cpu().numpy()
    del w
    pr, sr = g.oracle_quantize(fmt, w_rows)
    g.assert_quant_equal(fmt, p, s, pr, sr, rows=rows)
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=b + 5)
    y = w4.matmul_ex(g.to_dev_x(x, g.XDT[fmt]), p, s, fmt, path="mfma")
    g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("ns,k,b", [((1536, 256, 256), 1536, 8), ((300, 1000), 2048, 32),
                                    ((64, 40, 100, 17), 384, 129), ((8960, 8960), 1536, 4),
                                    ((130, 70), 8960, 16)])
def test_smallbatch_grouped_parity(fmt, ns, k, b):
    """One launch over members sharing x (the MFMA kernel over every member's row tiles from the
    MFMA threshold on): each y_g against the oracle on that member."""
    import bit_weight_only_w4_amd as w4

    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=b + k)
    xd = g.to_dev_x(x, g.XDT[fmt])
    packed, scales, refs = [], [], []
    for i, n in enumerate(ns):
        w = synth_inputs.weights(n, k, seed=n * 13 + i)
        p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
        pr, sr = g.oracle_quantize(fmt, w)
        g.assert_quant_equal(fmt, p, s, pr, sr)
        packed.append(p)
        scales.append(s)
        refs.append((pr, sr))
    ys = w4.gemm_smallbatch_grouped(xd, packed, scales, fmt)
    for y, (pr, sr) in zip(ys, refs):
        g.assert_y_close(fmt, y, x, pr, sr)


def test_smallbatch_grouped_below_threshold_is_the_grouped_gemv():
    """Below the MFMA threshold the grouped small-batch call runs the grouped fused GEMV: bitwise
    the same outputs as w4_gemv_grouped."""
    import torch

    import bit_weight_only_w4_amd as w4

    fmt, k, b = "nf4_f16", 1536, 2
    x = synth_inputs.activations(b, k, "f16", seed=5)
    xd = g.to_dev_x(x, "f16")
    packed, scales = [], []
    for i, n in enumerate((1536, 256, 256)):
        p, s = g.gpu_quantize(fmt, g.to_dev_f32(synth_inputs.weights(n, k, seed=40 + i)))
        packed.append(p)
        scales.append(s)
    a = w4.gemm_smallbatch_grouped(xd, packed, scales, fmt)
    c = w4.gemv_grouped(xd, packed, scales, fmt)
    for ya, yc in zip(a, c):
        assert torch.equal(ya, yc)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("n,k,b,splits", [(130, 8960, 8, 5), (96, 1536, 16, 2), (70, 2048, 33, 3),
                                          (40, 384, 4, 8), (200, 8192, 8, 4), (17, 1024, 129, 2)])
def test_mfma_splitk_parity(fmt, n, k, b, splits):
    """MFMA split-K (K in ranges of whole 256-weight quads, partial sums in the workspace, then the
    fixed-order reduction) against the oracle; y pre-filled with NaN and the workspace dirty, so a
    result that misses a split or accumulates into y fails.  Includes more splits than quads."""
    import torch

    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=n + k + b + splits)
    wsb = w4.workspace_bytes(fmt, n, k, b, "mfma", splits)
    assert wsb == splits * b * n * 4
    ws = torch.full((wsb,), 0x7F, dtype=torch.uint8, device=xd.device)
    y = torch.full((b, n), float("nan"), device=xd.device)
    w4.matmul_ex(xd, p, s, fmt, path="mfma", split_k=splits, workspace=ws, y=y)
    g.assert_y_close(fmt, y, x, pr, sr)
    y2 = w4.matmul_ex(xd, p, s, fmt, path="mfma", split_k=splits, workspace=ws)
    assert torch.equal(y, y2)


def test_mfma_splitk_needs_workspace():
    import torch

    import bit_weight_only_w4_amd as w4

    fmt, n, k, b = "nf4_f16", 64, 2048, 8
    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=9)
    small = torch.empty(4 * b * n * 4 - 16, dtype=torch.uint8, device=xd.device)
    with pytest.raises(RuntimeError, match="workspace"):
        w4.matmul_ex(xd, p, s, fmt, path="mfma", split_k=4, workspace=small)
    with pytest.raises(RuntimeError, match="workspace"):
        w4.matmul_ex(xd, p, s, fmt, path="mfma", split_k=4)
