"""2:4 sparse GEMV and its compression on the GPU against the oracle: the compressed values and
codes bit for bit, and y per element within |y - y_ref| <= 2e-3 * sum_k |x_k w_k| + 1e-5 of the
fp64 product with the decoded dense matrix."""
import numpy as np
import pytest

import synth_inputs
from oracle import sparse24 as S
from oracle.gemv import gemv_reference, violation_ratio
from tests import gpu_util as g

pytestmark = pytest.mark.gpu

XTYPES = ["f16", "bf16"]


def _compress_both(w, xdt, rows=None):
    import bit_weight_only_w4_amd as w4

    v, m = w4.sparse24_compress(g.to_dev_f32(w), xdt)
    wr = w if rows is None else w[rows]
    vr, mr = S.compress_2to4(wr, xdt)
    vg = v.cpu().numpy().view(np.uint16)
    mg = m.cpu().numpy()
    if rows is not None:
        vg, mg = vg[rows], mg[rows]
    assert np.array_equal(vg, vr), f"{np.sum(vg != vr)} values differ"
    assert np.array_equal(mg, mr), f"{np.sum(mg != mr)} code bytes differ"
    return v, m, vr, mr


def _check_y(y, x_bits, xdt, vr, mr, rows=None):
    yy = y.cpu().numpy().astype(np.float64)
    if rows is not None:
        yy = yy[:, rows]
    ref, t = gemv_reference(x_bits, xdt, S.dense_from_2to4(vr, mr, xdt))
    r = violation_ratio(yy, ref, t)
    assert r <= 1.0, f"tolerance violated: {r:.3f}"


@pytest.mark.parametrize("xdt", XTYPES)
@pytest.mark.parametrize("n,k,seed", [(64, 1536, 0), (37, 384, 1), (1, 32, 2), (129, 8960, 3),
                                      (300, 96, 4)])
def test_compress_bitexact(xdt, n, k, seed):
    w = synth_inputs.weights(n, k, seed=seed)
    _compress_both(w, xdt)


@pytest.mark.parametrize("xdt", XTYPES)
def test_compress_ties_and_zeros(xdt):
    rng = np.random.default_rng(9)
    w = (rng.integers(-2, 3, (16, 256)) * 0.25).astype(np.float32)   # many equal magnitudes
    w[3] = 0.0
    w[4, ::2] = -0.0
    w[5] = np.float32(6e4)  # large values, still inside the fp16 range
    _compress_both(w, xdt)


@pytest.mark.parametrize("xdt", XTYPES)
@pytest.mark.parametrize("n,k,b", [(256, 1536, 1), (37, 384, 1), (1, 32, 1), (300, 1536, 2),
                                   (129, 8960, 1), (77, 4096, 3), (64, 16384, 1), (200, 1536, 8),
                                   (45, 96, 5), (513, 1536, 4), (1000, 2048, 1)])
def test_gemv_parity(xdt, n, k, b):
    import bit_weight_only_w4_amd as w4

    w = synth_inputs.weights(n, k, seed=n + k)
    x = synth_inputs.activations(b, k, xdt, seed=b + 3)
    v, m, vr, mr = _compress_both(w, xdt)
    y = w4.sparse24_gemv(g.to_dev_x(x, xdt), v, m)
    _check_y(y, x, xdt, vr, mr)


@pytest.mark.parametrize("xdt", XTYPES)
def test_one_hot_exact(xdt):
    """x = e_j returns column j of the decoded matrix exactly (one product with 1.0 per row)."""
    import bit_weight_only_w4_amd as w4

    n, k = 300, 1536
    w = synth_inputs.weights(n, k, seed=12)
    v, m, vr, mr = _compress_both(w, xdt)
    dense = S.dense_from_2to4(vr, mr, xdt)
    one = 0x3C00 if xdt == "f16" else 0x3F80
    cols = [0, 1, 2, 3, 777, k - 1]
    x = np.zeros((len(cols), k), dtype=np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = one
    y = w4.sparse24_gemv(g.to_dev_x(x, xdt), v, m).cpu().numpy()
    for i, c in enumerate(cols):
        assert np.array_equal(y[i].astype(np.float64), dense[:, c])


@pytest.mark.parametrize("xdt", XTYPES)
def test_decode_shapes_full_and_sampled(xdt):
    """The five Qwen2.5-1.5B decode shapes at batch 1; lm_head on sampled rows."""
    import torch

    import bit_weight_only_w4_amd as w4

    for n, k in [(1536, 1536), (256, 1536), (8960, 1536), (1536, 8960), (151936, 1536)]:
        x = synth_inputs.activations(1, k, xdt, seed=k)
        if n > 9000:
            dev = g.device()
            gen = torch.Generator(device=dev).manual_seed(n)
            wd = torch.randn(n, k, generator=gen, device=dev) * 0.02
            rows = np.unique(np.concatenate([[0, n - 1],
                                             np.random.default_rng(n).choice(n, 158, replace=False)]))
            v, m = w4.sparse24_compress(wd, xdt)
            w_rows = wd[torch.as_tensor(rows, device=dev)].cpu().numpy()
            vr, mr = S.compress_2to4(w_rows, xdt)
            assert np.array_equal(v.cpu().numpy().view(np.uint16)[rows], vr)
            assert np.array_equal(m.cpu().numpy()[rows], mr)
        else:
            rows = None
            w = synth_inputs.weights(n, k, seed=n ^ k)
            v, m, vr, mr = _compress_both(w, xdt)
        y = w4.sparse24_gemv(g.to_dev_x(x, xdt), v, m)
        _check_y(y, x, xdt, vr, mr, rows=rows)


def test_deterministic_and_overwrites():
    import torch

    import bit_weight_only_w4_amd as w4

    w = synth_inputs.weights(700, 8960, seed=2)
    x = synth_inputs.activations(2, 8960, "f16", seed=2)
    v, m = w4.sparse24_compress(g.to_dev_f32(w), "f16")
    xd = g.to_dev_x(x, "f16")
    y1 = torch.full((2, 700), float("nan"), device=g.device())
    y2 = torch.full((2, 700), float("nan"), device=g.device())
    w4.sparse24_gemv(xd, v, m, y=y1)
    w4.sparse24_gemv(xd, v, m, y=y2)
    assert torch.equal(y1, y2) and not torch.isnan(y1).any()


@pytest.mark.parametrize("xdt", XTYPES)
@pytest.mark.parametrize("ns,k,b", [((1536, 256, 256), 1536, 1), ((8960, 8960), 1536, 1),
                                    ((1, 7, 300, 65), 384, 2), ((129, 33), 8960, 1),
                                    ((500,), 1024, 3)])
def test_grouped_bitwise_equals_solo(xdt, ns, k, b):
    """Each member of a grouped launch is bitwise the single-matrix call (same per-row arithmetic
    and launch shape) and within the bound of the oracle; y buffers pre-filled with NaN."""
    import torch

    import bit_weight_only_w4_amd as w4

    x = synth_inputs.activations(b, k, xdt, seed=k + b)
    xd = g.to_dev_x(x, xdt)
    members = []
    for i, n in enumerate(ns):
        w = synth_inputs.weights(n, k, seed=31 * i + n)
        members.append(_compress_both(w, xdt))
    ys = [torch.full((b, n), float("nan"), device=g.device()) for n in ns]
    w4.sparse24_gemv_grouped(xd, [m[0] for m in members], [m[1] for m in members], ys=ys)
    for (v, m, vr, mr), y in zip(members, ys):
        assert torch.equal(y, w4.sparse24_gemv(xd, v, m))
        _check_y(y, x, xdt, vr, mr)
