"""GPTQ's column loop on the GPU against the oracle's fp32 loop, bit for bit: codes, dequantized
weights, errors and the final weights.  Both sides take every rounding decision in fp32 with the
same order of operations (the kernels use no fused multiply-add, as the page's fused kernel does
not), so the comparison is exact.  Rows are independent in GPTQ, so full-size layers are checked
on sampled rows."""
import numpy as np
import pytest

import synth_inputs
from oracle import gptq as G
from tests import gpu_util as g

pytestmark = pytest.mark.gpu


def _grid(w, group, asym):
    """The observer's grid, fixed beforehand from the original weights: symmetric absmax / 7 with
    zero point 0 (codes -8..7), or asymmetric (max(w, 0) - min(w, 0)) / 15 with zero point
    rint(-min / s) (codes 0..15); fp32."""
    rows, cols = w.shape
    gw = w.reshape(rows, cols // group, group)
    if not asym:
        s = (np.abs(gw).max(axis=2) / np.float32(7)).astype(np.float32)
        return s, np.zeros_like(s), -8, 7
    lo = np.minimum(gw.min(axis=2), 0).astype(np.float32)
    hi = np.maximum(gw.max(axis=2), 0).astype(np.float32)
    s = ((hi - lo) / np.float32(15)).astype(np.float32)
    z = np.rint(-lo / np.where(s > 0, s, 1)).astype(np.float32)
    return s, z, 0, 15


def _dev(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to(g.device())


def _assert_same(gpu, ref, rows=None):
    q_hat, codes, err, w_final = gpu
    sel = (lambda t: t.cpu().numpy()) if rows is None else (lambda t: t.cpu().numpy()[rows])
    for name, a, b in (("codes", sel(codes).astype(np.int64), ref["codes"]),
                       ("q_hat", sel(q_hat), ref["q_hat"]), ("err", sel(err), ref["err"]),
                       ("w_final", sel(w_final), ref["w_final"])):
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), np.asarray(b, dtype=np.float32).view(np.uint32)
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{name}: {len(bad)} elements differ, first at {bad[:4].tolist()}"


def _case(rows, cols, group, block, asym, seed, check_rows=None):
    import bit_weight_only_w4_amd as w4

    w = synth_inputs.weights(rows, cols, sigma=0.02, seed=seed)
    u = synth_inputs.upper_factor(cols, seed=seed + 1)
    s, z, qmin, qmax = _grid(w, group, asym)
    wd = _dev(w)
    out = w4.gptq_quantize(wd, _dev(u), _dev(s), _dev(z), qmin, qmax, group=group, block=block)
    rsel = slice(None) if check_rows is None else check_rows
    ref = G.gptq(w[rsel], u, s[rsel], z[rsel], qmin, qmax, group=group, block=block,
                 dtype=np.float32)
    _assert_same((*out, wd), ref, rows=check_rows)
    return out, ref


@pytest.mark.parametrize("rows,cols,group,block,asym", [
    (37, 256, 256, 128, False),   # per-row grid, two full blocks, ragged rows
    (100, 320, 64, 128, True),    # groups of 64, last block of 64 columns, asymmetric
    (16, 128, 128, 128, False),   # one block
    (70, 384, 128, 32, True),     # narrower lazy blocks
    (33, 200, 40, 8, False),      # block 8, groups of 40 crossing blocks
    (5, 64, 64, 1, True),         # block 1: every update is lazy
    (1, 130, 130, 128, False),    # one row, last block of 2 columns
])
def test_gptq_bitwise(rows, cols, group, block, asym):
    w = synth_inputs.weights(rows, cols, sigma=0.02, seed=rows + cols + block)
    _, ref = _case(rows, cols, group, block, asym, seed=rows + cols + block)
    # the error feedback moves grid points away from plain rounding
    s, z, qmin, qmax = _grid(w, group, asym)
    assert np.any(ref["codes"] != G.rtn(w, s, z, qmin, qmax, group=group, dtype=np.float32)[1])


def test_block_and_lazy_entry_points_compose():
    """w4_gptq_block_update and w4_gptq_lazy_update called block by block give bitwise what
    w4_gptq_quantize gives."""
    import torch

    import bit_weight_only_w4_amd as w4

    rows, cols, group = 50, 384, 128
    w = synth_inputs.weights(rows, cols, seed=3)
    u = synth_inputs.upper_factor(cols, seed=4)
    s, z, qmin, qmax = _grid(w, group, False)
    ud, sd, zd = _dev(u), _dev(s), _dev(z)
    w1 = _dev(w)
    ref = w4.gptq_quantize(w1, ud, sd, zd, qmin, qmax, group=group, block=128)
    w2 = _dev(w)
    q_hat, codes, err = w4.gptq_outputs(w2)
    for c0 in range(0, cols, 128):
        w4.gptq_block_update(w2, ud, sd, zd, qmin, qmax, c0, 128, q_hat, codes, err, group=group)
        w4.gptq_lazy_update(w2, ud, err, c0, 128)
    for a, b in zip((q_hat, codes, err, w2), (*ref, w1)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("rows,cols,group,asym,nrows", [
    (8960, 1536, 128, False, 48),   # gate/up projection of Qwen2.5-1.5B, INT4 g128
    (1536, 8960, 128, True, 12),    # down projection, asymmetric
    (1536, 1536, 1536, False, 32),  # q/o projection, per-row grid
])
def test_gptq_full_size_sampled_rows(rows, cols, group, asym, nrows):
    rng = np.random.default_rng(rows + cols)
    check = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, nrows, replace=False)]))
    _case(rows, cols, group, 128, asym, seed=11, check_rows=check)


def test_gptq_codes_pack_into_the_int4_format():
    """Symmetric codes (qmin = -8) are the INT4 format's nibbles: packed with the group's bf16
    scale they decode through the W4 GEMV to q_hat x (scale exact in bf16 here)."""
    import torch

    import bit_weight_only_w4_amd as w4

    rows, cols = 64, 512
    w = synth_inputs.weights(rows, cols, seed=5)
    u = synth_inputs.upper_factor(cols, seed=6)
    s, z, qmin, qmax = _grid(w, 128, False)
    s = (s.view(np.uint32) & 0xFFFF0000).view(np.float32)  # bf16-exact scales
    q_hat, codes, _ = w4.gptq_quantize(_dev(w), _dev(u), _dev(s), _dev(z), qmin, qmax, group=128)
    c = codes.cpu().numpy()
    packed = ((c[:, 0::2] << 4) | c[:, 1::2]).astype(np.uint8)
    sb = (s.view(np.uint32) >> 16).astype(np.uint16)
    x = synth_inputs.activations(1, cols, "bf16", seed=7)
    y = w4.gemv(g.to_dev_x(x, "bf16"), _dev(packed), _dev(sb.view(np.int16)), "int4_bf16")
    g.assert_y_close("int4_bf16", y, x, packed, sb)
    import oracle

    assert np.array_equal(oracle.dequant("int4", packed, sb), q_hat.cpu().numpy().astype(np.float64))
    assert torch.isfinite(y).all()


def test_gptq_quantize_in_a_graph_replays_bitwise():
    """w4_gptq_quantize captured in a HIP graph (its helper stream joins the capture) and replayed
    three times, with eager work and synchronizations between replays: every replay gives the
    eager call's bits."""
    import torch

    import bit_weight_only_w4_amd as w4

    rows, cols, group = 4096, 2048, 128  # 2^23 weights: the two-stream schedule
    w = synth_inputs.weights(rows, cols, seed=21)
    u = synth_inputs.upper_factor(cols, seed=22)
    s, z, qmin, qmax = _grid(w, group, True)
    ud, sd, zd = _dev(u), _dev(s), _dev(z)
    w_eager = _dev(w)
    ref = w4.gptq_quantize(w_eager, ud, sd, zd, qmin, qmax, group=group, block=128)
    pristine = _dev(w)
    wg = pristine.clone()
    q_hat, codes, err = w4.gptq_outputs(wg)
    dev = g.device()
    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        w4.check(w4.lib().w4_gptq_quantize(
            w4._ptr(wg), w4._ptr(ud), w4._ptr(sd), w4._ptr(zd), rows, cols, group, qmin, qmax, 128,
            w4._ptr(q_hat), w4._ptr(codes), w4._ptr(err), stream.cuda_stream), "capture")
    for i in range(3):
        wg.copy_(pristine)
        q_hat.fill_(float("nan"))
        err.fill_(float("nan"))
        codes.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((q_hat, codes, err, wg), (*ref, w_eager)):
            assert torch.equal(a, b), i
        junk = torch.randn(1024, 1024, device=dev) @ torch.randn(1024, 1024, device=dev)
        torch.cuda.synchronize()
        del junk
