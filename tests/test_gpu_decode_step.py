"""The decode step as the benchmark runs it: the same Step object, launch units and HIP-graph
capture as bench.py (q|k|v and gate|up of a layer through w4_gemm_smallbatch_grouped, the others
through the automatic w4_matmul_ex with the step's workspace), on two decoder layers plus
lm_head.  Every y is filled with NaN before each eager run and each graph replay; the replays
must be bitwise equal to each other and to the eager launches, and every y must match the oracle
(q, k, v, o on all rows; gate, up, down and lm_head on sampled rows) after the packed weights have
matched it bit for bit.  The pages correctness-test every kernel version on the real shapes before
timing it (My Triton Kernel Ties bitsandbytes, "The kernels") and name graphs around the decode
step as the next step (same page, "What's next")."""
import numpy as np
import pytest

from tests import gpu_util as g

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt,b", [("nf4_f16", 1), ("int4_bf16", 1), ("fp4_f16", 1),
                                   ("nf4_f16", 8), ("int4a_bf16", 8)])
def test_decode_step_graph_matches_eager_and_oracle(fmt, b):
    import torch

    import bench

    dev = g.device()
    kept = {}

    def keep(i, name, w):
        n = w.shape[0]
        if n <= 2048:
            rows = None
            kept[i] = (rows, w.cpu().numpy())
        else:
            rng = np.random.default_rng(i + 17)
            rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 190, replace=False)]))
            kept[i] = (rows, w[torch.as_tensor(rows, device=w.device)].cpu().numpy())

    step = bench.Step(fmt, b, "auto", dev, layers=2, on_weight=keep)
    assert len(step.shapes) == 15
    units = bench.step_units(step.shapes, "grouped")
    assert len(units) == 9  # per layer q|k|v, o, gate|up, down; then lm_head
    stream = torch.cuda.current_stream()

    def fill_nan():
        for y in step.ys:
            y.fill_(float("nan"))

    fill_nan()
    for u in units:
        step.launch_unit(u, stream.cuda_stream)
    torch.cuda.synchronize()
    eager = [y.clone() for y in step.ys]
    graph = bench.capture(step, dev, units, "grouped")
    replays = []
    for _ in range(3):
        fill_nan()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replays.append([y.clone() for y in step.ys])
    for i, (name, _, _) in enumerate(step.shapes):
        assert not torch.isnan(replays[0][i]).any(), name
        for r in replays[1:]:
            assert torch.equal(replays[0][i], r[i]), f"replays differ on {name}"
        assert torch.equal(replays[0][i], eager[i]), f"replay differs from eager on {name}"
    for i, (name, n, k) in enumerate(step.shapes):
        rows, w = kept[i]
        pr, sr = g.oracle_quantize(fmt, w)
        packed, scales = step.mats[i]
        g.assert_quant_equal(fmt, packed, scales, pr, sr, rows=rows)
        x_bits = step.x[k].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        y = replays[0][i]
        if rows is not None:
            y = y[:, torch.as_tensor(rows, device=y.device)]
        g.assert_y_close(fmt, y, x_bits, pr, sr)
    del graph
