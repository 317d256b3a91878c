"""Full-size parity on the hidden-8192 model's shapes (q 8192x8192, gate/up 28672x8192, down
8192x28672, lm_head 128256x8192) at B = 1 on the automatic path, which here runs the fused GEMV's
large launch shapes: teams of 128 and 512 lanes (two and eight waves summing through LDS) that
walk 8 to 126 row blocks per workgroup through the three-buffer rotation.  Weights are drawn and
quantized on the GPU; sampled rows (the first and last among them) are checked against the
oracle, packed bytes bit for bit and y within |y - y_ref| <= 2e-3 * sum |x w| + 1e-5."""
import numpy as np
import pytest

import synth_inputs
from tests import gpu_util as g

pytestmark = pytest.mark.gpu

LARGE = [(8192, 8192), (28672, 8192), (8192, 28672), (128256, 8192)]


def _plan_trips(w4, fmt, n, k):
    p = w4.gemv_plan(fmt, n, k, 1)
    rows = p["threads"] // p["team"]
    nrb = -(-n // rows)
    return p, -(-nrb // p["grid_x"])


def test_large_shapes_take_multi_wave_teams_over_many_row_blocks():
    """The cases below exercise wide teams (an LDS sum across waves inside the row-block loop)
    over more than two row blocks per workgroup, in both wave counts."""
    import bit_weight_only_w4_amd as w4

    seen = set()
    for n, k in LARGE:
        p, trips = _plan_trips(w4, "nf4_f16", n, k)
        assert w4.auto_path("nf4_f16", n, k, 1)[0] == "gemv"
        if p["team"] >= 128 and trips > 2:
            seen.add(p["team"] // 64)
    assert {2, 8} <= seen, seen


def _sampled_case(fmt, n, k, b, seed):
    import torch

    dev = g.device()
    gen = torch.Generator(device=dev).manual_seed(seed)
    w = torch.randn(n, k, generator=gen, device=dev) * synth_inputs.LARGE_SIGMA
    p, s = g.gpu_quantize(fmt, w)
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[0, 1, n - 2, n - 1], rng.choice(n, 156, replace=False)]))
    w_rows = w[torch.as_tensor(rows, device=dev)].cpu().numpy()
    del w
    pr, sr = g.oracle_quantize(fmt, w_rows)
    g.assert_quant_equal(fmt, p, s, pr, sr, rows=rows)
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=seed + 1)
    return x, g.to_dev_x(x, g.XDT[fmt]), p, s, pr, sr, rows


@pytest.mark.parametrize("fmt", ["nf4_f16", "int4_f16", "int4a_bf16", "fp4_bf16"])
@pytest.mark.parametrize("n,k", LARGE)
def test_gemv_large_auto_sampled(fmt, n, k):
    import torch

    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr, rows = _sampled_case(fmt, n, k, 1, seed=n + 7 * k)
    ws = torch.empty(1 << 22, dtype=torch.uint8, device=g.device())
    y = torch.full((1, n), float("nan"), device=g.device())
    w4.matmul_ex(xd, p, s, fmt, path="auto", workspace=ws, y=y)
    assert not torch.isnan(y).any()
    g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)
    y2 = w4.gemv(xd, p, s, fmt)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("fmt,b", [("nf4_bf16", 2), ("int4_bf16", 3)])
def test_gemv_large_small_batch_sampled(fmt, b):
    """B = 2 and 3 on 28672 x 8192 (the GEMV below the MFMA threshold on large matrices)."""
    import torch

    import bit_weight_only_w4_amd as w4

    n, k = 28672, 8192
    x, xd, p, s, pr, sr, rows = _sampled_case(fmt, n, k, b, seed=b * 11 + 3)
    y = w4.matmul_ex(xd, p, s, fmt, path="gemv")
    g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)


@pytest.mark.parametrize("fmt,b", [("int4_f16", 4), ("int4_bf16", 16), ("int4a_f16", 16),
                                   ("int4a_bf16", 4), ("nf4_bf16", 4), ("fp4_f16", 16)])
def test_mfma_long_k_sampled(fmt, b):
    """The MFMA path on the down projection 8192 x 28672 at B = 4 and 16 (the batch sizes of the
    larger model's measurements)."""
    import torch

    import bit_weight_only_w4_amd as w4

    n, k = 8192, 28672
    x, xd, p, s, pr, sr, rows = _sampled_case(fmt, n, k, b, seed=b + 101)
    y = w4.matmul_ex(xd, p, s, fmt, path="mfma")
    g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)
    auto = w4.gemm_smallbatch(xd, p, s, fmt)
    assert torch.equal(auto, y)  # the automatic choice at these batches is the MFMA kernel
