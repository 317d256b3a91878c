"""Fused GEMV / split-K / two-pass / small-batch paths against the oracle's fp64 reference,
per element, within |y - y_ref| <= 2e-3 * sum_k |x_k w_k| + 1e-5.

Every case quantizes on the GPU, checks the packed data bit for bit against the oracle, and then
checks y computed from it, so the oracle's reference is built from the oracle's own packed data.
"""
import numpy as np
import pytest

import synth_inputs
from tests import gpu_util as g

pytestmark = pytest.mark.gpu

ALL_FMTS = ["nf4_f16", "nf4_bf16", "int4_f16", "int4_bf16", "fp4_f16", "fp4_bf16", "int4a_f16",
            "int4a_bf16"]


def _case(fmt, n, k, b, seed, sigma=0.02):
    w = synth_inputs.weights(n, k, sigma=sigma, seed=seed)
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=seed + 1000)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    g.assert_quant_equal(fmt, p, s, pr, sr)
    return x, g.to_dev_x(x, g.XDT[fmt]), p, s, pr, sr


def _workspace(nbytes):
    import torch

    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=g.device())


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("n,k,b", [(256, 1536, 1), (37, 384, 1), (1, 128, 1), (300, 1536, 2),
                                   (129, 8960, 1), (129, 8960, 2), (77, 8192, 3), (64, 28672, 1),
                                   (200, 1536, 4),
                                   (45, 1024, 5), (96, 2048, 8), (33, 640, 7), (250, 256, 6)])
def test_gemv_parity(fmt, n, k, b):
    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=n + k + b)
    y = w4.gemv(xd, p, s, fmt)
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ["nf4_f16", "nf4_bf16", "fp4_f16", "fp4_bf16"])
@pytest.mark.parametrize("n,k,b", [(70, 192, 1), (129, 320, 2), (33, 64, 1), (300, 1472, 3)])
def test_gemv_odd_block_count(fmt, n, k, b):
    """64-weight-block formats with an odd number of blocks per row (K % 128 == 64)."""
    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=n + 3 * k + b)
    y = w4.gemv(xd, p, s, fmt)
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_single_gemv_workload(fmt):
    """W[256 x 1536] ~ N(0, 0.02) drawn first, then x, seed 0 (the single-GEMV workload)."""
    import bit_weight_only_w4_amd as w4

    w, x = synth_inputs.single_gemv_case(seed=0, dtype=g.XDT[fmt])
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    g.assert_quant_equal(fmt, p, s, pr, sr)
    y = w4.gemv(g.to_dev_x(x, g.XDT[fmt]), p, s, fmt)
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("splits", [2, 3, 4, 8, 16])
def test_splitk_parity_down_shape(fmt, splits):
    """Split-K on the 1536 x 8960 down projection, B = 1 and 8."""
    import bit_weight_only_w4_amd as w4

    for b in (1, 8):
        x, xd, p, s, pr, sr = _case(fmt, 1536, 8960, b, seed=40 + splits)
        ws = _workspace(w4.workspace_bytes(fmt, 1536, 8960, b, "splitk", splits))
        y = w4.matmul_ex(xd, p, s, fmt, path="splitk", split_k=splits, workspace=ws)
        g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ["nf4_f16", "int4_bf16"])
def test_splitk_deterministic_and_overwrites(fmt):
    """y pre-filled with NaN and called twice with a dirty workspace: bitwise identical results,
    nothing accumulated into y (the stale-output bug of an atomic split-K under autotuning)."""
    import torch

    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, 1536, 8960, 2, seed=77)
    ws = _workspace(w4.workspace_bytes(fmt, 1536, 8960, 2, "splitk", 8))
    ws.fill_(0x7F)
    y1 = torch.full((2, 1536), float("nan"), device=g.device())
    w4.matmul_ex(xd, p, s, fmt, path="splitk", split_k=8, workspace=ws, y=y1)
    y2 = torch.full((2, 1536), float("nan"), device=g.device())
    w4.matmul_ex(xd, p, s, fmt, path="splitk", split_k=8, workspace=ws, y=y2)
    assert torch.equal(y1, y2)
    g.assert_y_close(fmt, y1, x, pr, sr)
    y3 = w4.gemv(xd, p, s, fmt)
    y4 = w4.gemv(xd, p, s, fmt)
    assert torch.equal(y3, y4)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("n,k,b", [(256, 1536, 1), (129, 8960, 3), (40, 384, 17)])
def test_twopass_parity(fmt, n, k, b):
    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=5 * n + b)
    ws = _workspace(w4.workspace_bytes(fmt, n, k, b, "twopass"))
    y = w4.matmul_ex(xd, p, s, fmt, path="twopass", workspace=ws)
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_batch_rows_match_single_calls(fmt):
    """Each row of a B = 5 product equals (within the bound) the B = 1 product of that row."""
    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, 513, 1536, 5, seed=3)
    y = w4.gemv(xd, p, s, fmt)
    for i in range(5):
        yi = w4.gemv(xd[i:i + 1].contiguous(), p, s, fmt)
        g.assert_y_close(fmt, yi, x[i:i + 1], pr, sr)
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_one_hot_and_zero_activations(fmt):
    import torch

    import bit_weight_only_w4_amd as w4

    n, k = 96, 1536
    w = synth_inputs.weights(n, k, seed=8)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    x = np.zeros((2, k), dtype=np.uint16)
    x[0, 700] = 0x3C00 if g.XDT[fmt] == "f16" else 0x3F80  # 1.0
    y = w4.gemv(g.to_dev_x(x, g.XDT[fmt]), p, s, fmt).cpu().numpy().astype(np.float64)
    import oracle

    w_hat = oracle.dequant(g.WFMT[fmt], pr, sr)
    assert np.all(y[1] == 0)
    # decoded codes: fp16 rounding for NF4 x fp16 (<= 3.3e-4 relative), a two-term bf16 split
    # for NF4 x bf16 (<= 2^-16 relative), exact (q - 8) for INT4; FP4 codes are exact in both
    # activation types and only the fp32 product code * scale rounds (<= 2^-24 relative)
    rtol = {"nf4_f16": 3.5e-4, "nf4_bf16": 2.0 ** -16, "fp4_f16": 2.0 ** -23,
            "fp4_bf16": 2.0 ** -23}.get(fmt, 0.0)
    assert np.allclose(y[0], w_hat[:, 700], rtol=rtol, atol=0)
    assert torch.isfinite(torch.as_tensor(y)).all()


@pytest.mark.parametrize("fmt", ["nf4_f16", "int4_bf16"])
def test_decode_shapes_full_and_sampled(fmt):
    """The five Qwen2.5-1.5B decode shapes at B = 1, the path the decode step uses (auto with a
    workspace); lm_head checked on sampled rows."""
    import torch

    import bit_weight_only_w4_amd as w4

    shapes = [(1536, 1536), (256, 1536), (8960, 1536), (1536, 8960), (151936, 1536)]
    for n, k in shapes:
        w = synth_inputs.weights(n, k, seed=n ^ k)
        x = synth_inputs.activations(1, k, g.XDT[fmt], seed=11)
        p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
        rows = None if n <= 9000 else np.sort(np.random.default_rng(n).choice(n, 200, replace=False))
        pr, sr = g.oracle_quantize(fmt, w if rows is None else w[rows])
        g.assert_quant_equal(fmt, p, s, pr, sr, rows=rows)
        ws = torch.empty(1 << 22, dtype=torch.uint8, device=g.device())
        y = w4.matmul_ex(g.to_dev_x(x, g.XDT[fmt]), p, s, fmt, path="auto", workspace=ws)
        if rows is None:
            g.assert_y_close(fmt, y, x, pr, sr)
        else:
            g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)


def test_error_codes_on_device_pointers():
    import torch

    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case("nf4_f16", 64, 256, 1, seed=1)
    y = torch.empty((1, 64), device=g.device())
    L = w4.lib()
    import ctypes

    vp = ctypes.c_void_p
    st = L.w4_gemv(vp(xd.data_ptr() + 2), vp(p.data_ptr()), vp(s.data_ptr()), 1, 64, 256, 1,
                   vp(y.data_ptr()), None)
    assert st == -3  # misaligned x
    st = L.w4_gemv(vp(xd.data_ptr()), vp(p.data_ptr()), vp(s.data_ptr()), 1, 64, 192 + 32, 1,
                   vp(y.data_ptr()), None)
    assert st == -2  # K not a multiple of 64
    st = L.w4_gemv(vp(xd.data_ptr()), vp(p.data_ptr()), vp(s.data_ptr()), 3, 64, 192, 1,
                   vp(y.data_ptr()), None)
    assert st == -2  # INT4 needs K % 128
    st = L.w4_gemv(vp(xd.data_ptr()), vp(p.data_ptr()), vp(s.data_ptr()), 1, 64, 256, 1,
                   vp(xd.data_ptr()), None)
    assert st == -9  # y aliases x
    st = L.w4_matmul_ex(vp(xd.data_ptr()), vp(p.data_ptr()), vp(s.data_ptr()), 1, 64, 256, 1,
                        vp(y.data_ptr()), 2, 4, None, 0, None)
    assert st == -6  # split-K without workspace
    assert torch.cuda.synchronize() is None


def _grouped_case(fmt, ns, k, b, seed):
    members = []
    for i, n in enumerate(ns):
        w = synth_inputs.weights(n, k, sigma=0.02, seed=seed + 17 * i)
        p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
        pr, sr = g.oracle_quantize(fmt, w)
        g.assert_quant_equal(fmt, p, s, pr, sr)
        members.append((p, s, pr, sr))
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=seed + 999)
    return x, g.to_dev_x(x, g.XDT[fmt]), members


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("ns,k,b", [((1536, 256, 256), 1536, 1), ((8960, 8960), 1536, 1),
                                    ((1, 7, 300, 65), 1536, 1), ((37, 100), 384, 2),
                                    ((129, 64, 1), 8960, 1), ((70, 200, 33), 640, 4),
                                    ((96, 40), 2048, 8), ((500,), 1024, 3)])
def test_grouped_parity(fmt, ns, k, b):
    """Each member of a grouped launch against the oracle; ragged member sizes that end inside a
    row block, single-row members, and up to four members."""
    import bit_weight_only_w4_amd as w4

    x, xd, members = _grouped_case(fmt, ns, k, b, seed=sum(ns) + k + b)
    ys = w4.gemv_grouped(xd, [m[0] for m in members], [m[1] for m in members], fmt)
    for (p, s, pr, sr), y in zip(members, ys):
        g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("ns,b", [((1536, 256, 256), 1), ((8960, 8960), 1), ((1536, 256, 256), 4)])
def test_grouped_bitwise_equals_solo(fmt, ns, b):
    """When the grouped launch gets the same launch shape as each member alone, every y_g is
    bitwise equal to w4_gemv on that member (same per-row arithmetic, only the row mapping
    differs); y buffers pre-filled with NaN, so every element must be written."""
    import torch

    import bit_weight_only_w4_amd as w4

    k = 1536
    x, xd, members = _grouped_case(fmt, ns, k, b, seed=5 + b)
    plan_all = w4.gemv_plan(fmt, sum(ns), k, b)
    ys = [torch.full((b, n), float("nan"), device=g.device()) for n in ns]
    w4.gemv_grouped(xd, [m[0] for m in members], [m[1] for m in members], fmt, ys=ys)
    for n, (p, s, pr, sr), y in zip(ns, members, ys):
        plan_one = w4.gemv_plan(fmt, n, k, b)
        y_solo = w4.gemv(xd, p, s, fmt)
        assert not torch.isnan(y).any()
        if all(plan_one[f] == plan_all[f] for f in ("threads", "team", "iters")):
            assert torch.equal(y, y_solo)
        g.assert_y_close(fmt, y, x, pr, sr)


def test_grouped_long_rows_at_b8_fall_back_to_mfma():
    """B = 8 with K = 28672 has no GEMV launch shape; the grouped call then runs the members in
    one launch of the MFMA kernel and still meets the bound."""
    import bit_weight_only_w4_amd as w4

    fmt = "nf4_f16"
    x, xd, members = _grouped_case(fmt, (40, 24), 28672, 8, seed=3)
    ys = w4.gemv_grouped(xd, [m[0] for m in members], [m[1] for m in members], fmt)
    for (p, s, pr, sr), y in zip(members, ys):
        g.assert_y_close(fmt, y, x, pr, sr)
