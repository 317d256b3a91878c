"""The decode-step shape list used by the tests and the benchmark, pinned against the figures the
pages print (tests/golden/qwen15_decode_step.txt carries each figure with its source)."""
import os

import synth_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "qwen15_decode_step.txt")


def _golden():
    out = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [float(v) for v in vals]
    return out


def test_shape_list_matches_printed_figures():
    g = _golden()
    shapes = synth_inputs.decode_step_shapes()
    assert len(shapes) == g["matmuls_per_step"][0]
    layer = {name: (n, k) for name, n, k in synth_inputs.QWEN15_LAYER}
    for key in ("q", "k", "v", "o"):
        k_in, n_out = g[f"{key}_width"]
        assert layer[key] == (n_out, k_in)
    assert synth_inputs.QWEN15_LAYERS == g["layers"][0]
    assert 2 * synth_inputs.QWEN15_LAYERS == g["kv_projections_replaced"][0]
    assert len({(n, k) for _, n, k in shapes}) == 5  # five distinct (N, K) shapes
    weights = sum(n * k for _, n, k in shapes)
    assert round(weights * 2 / 1e9, 3) == g["bf16_weight_gb"][0]
    assert round(weights * 0.5 / 1e9, 3) == g["int4_weight_gb"][0]
    lm = synth_inputs.QWEN15_LM_HEAD
    assert lm[1] == g["lm_head_vocab"][0]
    assert round(100 * lm[1] * lm[2] / weights) == g["lm_head_share_pct"][0]


def test_byte_accounting_figures():
    g = _golden()
    assert g["bytes_per_weight_fused_packed"][0] + 2 * g["bytes_per_weight_fp16"][0] == \
        g["bytes_per_weight_out_of_place"][0]
