"""Tiled prefill GEMM (W4_PATH_TILED, w4_gemm_prefill) against the oracle's fp64 reference, per
element within 2e-3 T + 1e-5 (T = sum over k of |x * w_hat|), as for every other path."""
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


# Tiles are 128 (or 64) weight rows x 128 activation rows over 64-weight blocks of K: the cases
# cover one block (K = 128 for INT4's group), an odd block count (K = 384, 8960 / 64 = 140 even,
# 320 / 64 = 5 odd for NF4), ragged N and B in both tile directions, B = 1, and several tiles.
@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("n,k,b", [(64, 128, 128), (37, 384, 130), (300, 1536, 512), (129, 8960, 200),
                                   (1000, 2048, 257), (96, 1024, 1), (65, 128, 33), (260, 640, 300)])
def test_tiled_parity(fmt, n, k, b):
    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=n * 5 + b)
    y = w4.matmul_ex(xd, p, s, fmt, path="tiled")
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ["nf4_f16", "nf4_bf16", "fp4_f16", "fp4_bf16"])
def test_tiled_odd_block_count(fmt):
    """K = 320: five 64-weight blocks (NF4, FP4), so the block loop ends on its remainder step."""
    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, 200, 320, 150, seed=9)
    y = w4.matmul_ex(xd, p, s, fmt, path="tiled")
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_tiled_scale_range(fmt):
    """Rows whose block scales are tiny, huge or zero next to ordinary rows: the tiled kernel
    applies every block scale in fp32 to that block's fresh partial sums, so the scale's range
    never meets a 16-bit operand; all rows within the bound."""
    import numpy as np

    import bit_weight_only_w4_amd as w4

    n, k, b = 300, 1536, 200
    w = synth_inputs.weights(n, k, seed=31)
    factors = np.array([1.0, 1e-3, 1.0, 1e6, 1e-7, 1.0, 0.0, 1.0], dtype=np.float32)
    w = (w * factors[np.arange(n) % len(factors)][:, None]).astype(np.float32)
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=32)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    g.assert_quant_equal(fmt, p, s, pr, sr)
    y = w4.matmul_ex(g.to_dev_x(x, g.XDT[fmt]), p, s, fmt, path="tiled")
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ["nf4_f16", "int4_bf16", "fp4_bf16"])
def test_prefill_entry_auto_and_determinism(fmt):
    """w4_gemm_prefill, the explicit tiled path and the automatic path at B >= W4_TILED_FROM_BATCH
    give bitwise the same y; a second call repeats it bitwise."""
    import torch

    import bit_weight_only_w4_amd as w4

    b = 512
    x, xd, p, s, pr, sr = _case(fmt, 8960, 1536, b, seed=2)
    assert w4.auto_path(fmt, 8960, 1536, b)[0] == "tiled"
    y1 = w4.gemm_prefill(xd, p, s, fmt)
    y2 = w4.matmul_ex(xd, p, s, fmt, path="tiled")
    y3 = w4.gemm_smallbatch(xd, p, s, fmt)
    assert torch.equal(y1, y2) and torch.equal(y1, y3)
    g.assert_y_close(fmt, y1, x, pr, sr)


@pytest.mark.parametrize("fmt,n,k,b", [("nf4_f16", 151936, 1536, 512), ("int4_bf16", 151936, 1536, 512),
                                       ("nf4_bf16", 1536, 8960, 512), ("int4_f16", 28672, 8192, 512),
                                       ("nf4_f16", 8960, 1536, 4096), ("fp4_bf16", 8960, 1536, 512),
                                       ("fp4_f16", 28672, 8192, 512), ("int4a_bf16", 151936, 1536, 512),
                                       ("int4a_f16", 8960, 1536, 1024), ("nf4_f16", 8960, 1536, 512),
                                       ("nf4_bf16", 8960, 1536, 512), ("int4a_bf16", 8960, 1536, 512)])
def test_tiled_full_size_sampled(fmt, n, k, b):
    """Full-size prefill matrices at 512 tokens (and 4096, the largest batch): weights drawn on the
    GPU, quantized there, and 160 sampled rows (the first and the last among them) checked
    against the oracle over every activation row."""
    import numpy as np
    import torch

    import bit_weight_only_w4_amd as w4

    dev = g.device()
    gen = torch.Generator(device=dev).manual_seed(n + 5 * k + b)
    w = torch.randn(n, k, generator=gen, device=dev) * 0.02
    p, s = g.gpu_quantize(fmt, w)
    rng = np.random.default_rng(n + b)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 158, replace=False)]))
    w_rows = w[torch.as_tensor(rows, device=dev)].cpu().numpy()
    del w
    pr, sr = g.oracle_quantize(fmt, w_rows)
    g.assert_quant_equal(fmt, p, s, pr, sr, rows=rows)
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=b + 11)
    y = w4.gemm_prefill(g.to_dev_x(x, g.XDT[fmt]), p, s, fmt)
    g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("n,k,b,splits", [(130, 8960, 200, 8), (37, 1024, 129, 2), (300, 2048, 512, 4),
                                          (64, 384, 130, 3), (96, 256, 257, 16), (65, 8192, 33, 5)])
def test_tiled_splitk_parity(fmt, n, k, b, splits):
    """Tiled GEMM over K ranges of whole 64-weight blocks (partial sums in the workspace, then the
    fixed-order reduction) against the oracle; y pre-filled with NaN and the workspace dirty, so a
    result that misses a range or accumulates into y fails.  Includes more splits than blocks
    (K = 256: four ranges of one block) and uneven ranges (140 blocks in 8, 128 in 5)."""
    import torch

    import bit_weight_only_w4_amd as w4

    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=n + k + b + splits)
    nb = k // 64
    per = -(-nb // min(splits, nb))
    ranges = -(-nb // per)
    wsb = w4.workspace_bytes(fmt, n, k, b, "tiled", splits)
    assert wsb == ranges * b * n * 4
    ws = torch.full((wsb,), 0x7F, dtype=torch.uint8, device=xd.device)
    y = torch.full((b, n), float("nan"), device=xd.device)
    w4.matmul_ex(xd, p, s, fmt, path="tiled", split_k=splits, workspace=ws, y=y)
    g.assert_y_close(fmt, y, x, pr, sr)
    y2 = w4.matmul_ex(xd, p, s, fmt, path="tiled", split_k=splits, workspace=ws)
    assert torch.equal(y, y2)


def test_tiled_splitk_needs_workspace():
    import torch

    import bit_weight_only_w4_amd as w4

    fmt, n, k, b = "nf4_f16", 64, 2048, 130
    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=9)
    small = torch.empty(4 * b * n * 4 - 16, dtype=torch.uint8, device=xd.device)
    with pytest.raises(RuntimeError, match="workspace"):
        w4.matmul_ex(xd, p, s, fmt, path="tiled", split_k=4, workspace=small)
    with pytest.raises(RuntimeError, match="workspace"):
        w4.matmul_ex(xd, p, s, fmt, path="tiled", split_k=4)
    # one range needs none: bitwise the unsplit launch
    y1 = w4.matmul_ex(xd, p, s, fmt, path="tiled", split_k=1)
    assert torch.equal(y1, w4.gemm_prefill(xd, p, s, fmt))


@pytest.mark.parametrize("fmt,n,k,b", [("nf4_f16", 1536, 8960, 512), ("int4_bf16", 1024, 8192, 128),
                                       ("int4a_f16", 1536, 8960, 256), ("fp4_bf16", 8192, 8192, 128)])
def test_tiled_splitk_auto_full_size_sampled(fmt, n, k, b):
    """The automatic path with a workspace at prefill batches: the tiled GEMM split over K for the
    matrices whose tiles do not fill the CUs (the 1536 x 8960 down projection, the 1024 x 8192 k/v
    projection, 8192 x 8192 at 128 rows), bitwise equal to the explicit call with its split count;
    160 sampled rows against the oracle over every activation row."""
    import numpy as np
    import torch

    import bit_weight_only_w4_amd as w4

    dev = g.device()
    gen = torch.Generator(device=dev).manual_seed(n + 3 * k + b)
    w = torch.randn(n, k, generator=gen, device=dev) * 0.02
    p, s = g.gpu_quantize(fmt, w)
    rng = np.random.default_rng(n + k + b)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 158, replace=False)]))
    w_rows = w[torch.as_tensor(rows, device=dev)].cpu().numpy()
    del w
    pr, sr = g.oracle_quantize(fmt, w_rows)
    g.assert_quant_equal(fmt, p, s, pr, sr, rows=rows)
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=b + 13)
    xd = g.to_dev_x(x, g.XDT[fmt])
    wsb = w4.workspace_bytes(fmt, n, k, b)
    path, sk = w4.auto_path(fmt, n, k, b, wsb)
    assert path == "tiled" and sk > 1 and wsb > 0
    ws = torch.full((wsb,), 0x7F, dtype=torch.uint8, device=dev)
    y = torch.full((b, n), float("nan"), device=dev)
    w4.matmul_ex(xd, p, s, fmt, workspace=ws, y=y)
    assert torch.equal(y, w4.matmul_ex(xd, p, s, fmt, path="tiled", split_k=sk, workspace=ws))
    g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)


@pytest.mark.parametrize("fmt", ["nf4_f16", "int4_bf16"])
def test_grouped_at_prefill_batch(fmt):
    """w4_gemm_smallbatch_grouped from W4_TILED_FROM_BATCH on: members of W4_TILED_FROM_ROWS rows
    and more through the tiled GEMM (one member: bitwise equal to w4_gemm_prefill on it), the
    others in one MFMA launch; every member against the oracle."""
    import torch

    import bit_weight_only_w4_amd as w4

    k, b = 1536, 160
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=77)
    xd = g.to_dev_x(x, g.XDT[fmt])
    packed, scales, refs, ns = [], [], [], (w4.TILED_FROM_ROWS + 100, 1536, 256)
    for i, n in enumerate(ns):
        w = synth_inputs.weights(n, k, seed=60 + i)
        p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
        packed.append(p)
        scales.append(s)
        refs.append(g.oracle_quantize(fmt, w))
    ys = w4.gemm_smallbatch_grouped(xd, packed, scales, fmt)
    assert torch.equal(ys[0], w4.gemm_prefill(xd, packed[0], scales[0], fmt))
    for y, (pr, sr) in zip(ys, refs):
        g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
def test_grouped_tiled_members(fmt):
    """Several members of W4_TILED_FROM_ROWS rows and more share one tiled launch (their tiles one
    after another, ragged row counts, an MFMA member beside them): every member against the oracle,
    bitwise equal to the same kernel on that member alone, and repeatable bitwise; y pre-filled
    with NaN.  bf16 activations: the block-scale kernel, as w4_gemm_prefill runs it on one member
    (64 x 128 tiles, two K groups both times).  fp16 activations: the launch's 210 tiles of 128
    rows at 160 activation rows take the folded kernel (from half a tile per CU), a member alone
    too few, so the reference is the folded kernel forced on the member (128-row tiles both
    times)."""
    import torch

    import bit_weight_only_w4_amd as w4

    k, b = 1024, 160
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=81)
    xd = g.to_dev_x(x, g.XDT[fmt])
    ns = (w4.TILED_FROM_ROWS + 33, 300, w4.TILED_FROM_ROWS + 1000, w4.TILED_FROM_ROWS)
    packed, scales, refs = [], [], []
    for i, n in enumerate(ns):
        w = synth_inputs.weights(n, k, seed=90 + i)
        p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
        packed.append(p)
        scales.append(s)
        refs.append(g.oracle_quantize(fmt, w))
    ys = [torch.full((b, n), float("nan"), device=xd.device) for n in ns]
    w4.gemm_smallbatch_grouped(xd, packed, scales, fmt, ys=ys)
    for i, (y, (pr, sr)) in enumerate(zip(ys, refs)):
        g.assert_y_close(fmt, y, x, pr, sr)
        if ns[i] >= w4.TILED_FROM_ROWS:
            if fmt.endswith("_f16"):
                alone = w4.matmul_ex(xd, packed[i], scales[i], fmt, path="tiled_f16")
            else:
                alone = w4.gemm_prefill(xd, packed[i], scales[i], fmt)
            assert torch.equal(y, alone)
    again = w4.gemm_smallbatch_grouped(xd, packed, scales, fmt)
    for y, y2 in zip(ys, again):
        assert torch.equal(y, y2)


@pytest.mark.parametrize("fmt", ["nf4_f16", "int4a_bf16"])
def test_grouped_tiled_gate_up_full_size(fmt):
    """The gate and up projections (8960 x 1536 each) of a 512-token prompt in one grouped call:
    one tiled launch over both, bitwise equal to w4_gemm_prefill on each (both launches run one K
    group per tile, hence the same per-block accumulation order); 160 sampled rows of each against
    the oracle."""
    import numpy as np
    import torch

    import bit_weight_only_w4_amd as w4

    dev = g.device()
    n, k, b = 8960, 1536, 512
    x = synth_inputs.activations(b, k, g.XDT[fmt], seed=515)
    xd = g.to_dev_x(x, g.XDT[fmt])
    packed, scales, checks = [], [], []
    for i in range(2):
        gen = torch.Generator(device=dev).manual_seed(4242 + i)
        w = torch.randn(n, k, generator=gen, device=dev) * 0.02
        p, s = g.gpu_quantize(fmt, w)
        rng = np.random.default_rng(77 + i)
        rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 158, replace=False)]))
        w_rows = w[torch.as_tensor(rows, device=dev)].cpu().numpy()
        del w
        pr, sr = g.oracle_quantize(fmt, w_rows)
        g.assert_quant_equal(fmt, p, s, pr, sr, rows=rows)
        packed.append(p)
        scales.append(s)
        checks.append((rows, pr, sr))
    ys = w4.gemm_smallbatch_grouped(xd, packed, scales, fmt)
    for i, (y, (rows, pr, sr)) in enumerate(zip(ys, checks)):
        assert torch.equal(y, w4.gemm_prefill(xd, packed[i], scales[i], fmt))
        g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)


@pytest.mark.parametrize("fmt", ALL_FMTS)
@pytest.mark.parametrize("path,b", [("mfma", 16), ("mfma", 40), ("tiled", 128), ("tiled", 200)])
def test_one_hot_columns_matrix_core_paths(fmt, path, b):
    """Activation row i = e_{c_i}: y[i] is column c_i of the decoded matrix, up to the rounding of
    the decoded code (fp16 NF4 codes: 3.3e-4 relative; the two-term bf16 split: 2^-16) and of the
    fp32 product with the scale (2^-24); INT4 and asymmetric INT4 come out exact."""
    import numpy as np

    import oracle

    import bit_weight_only_w4_amd as w4

    n, k = 300, 1024
    w = synth_inputs.weights(n, k, seed=77)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    w_hat = oracle.dequant(g.WFMT[fmt], pr, sr)
    one = 0x3C00 if g.XDT[fmt] == "f16" else 0x3F80
    cols = [(37 * i + 5) % k for i in range(b)]
    x = np.zeros((b, k), dtype=np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = one
    y = w4.matmul_ex(g.to_dev_x(x, g.XDT[fmt]), p, s, fmt, path=path).cpu().numpy().astype(np.float64)
    rtol = {"nf4_f16": 3.5e-4, "nf4_bf16": 2.0 ** -16 + 2.0 ** -23, "fp4_f16": 2.0 ** -23,
            "fp4_bf16": 2.0 ** -23}.get(fmt, 0.0)
    for i, c in enumerate(cols):
        assert np.allclose(y[i], w_hat[:, c], rtol=rtol, atol=0), (i, c)


@pytest.mark.parametrize("seed", range(40))
def test_random_shapes_matrix_core_paths(seed):
    """Seeded random shapes through the automatic path with its workspace (which may split K on the
    tiled GEMM or the MFMA kernel), an explicit tiled split and a grouped call of two to four
    members: format, N (1..2500), K (a multiple of the format's group up to 4096) and B (1..700)
    drawn from the seed; y pre-filled with NaN; every result against the oracle."""
    import numpy as np
    import torch

    import bit_weight_only_w4_amd as w4

    rng = np.random.default_rng(9000 + seed)
    fmt = ALL_FMTS[int(rng.integers(len(ALL_FMTS)))]
    grp = 128 if fmt.startswith("int4") else 64
    k = grp * int(rng.integers(1, 4096 // grp + 1))
    b = int(rng.choice([int(rng.integers(1, 9)), int(rng.integers(9, 128)), int(rng.integers(128, 701))]))
    n = int(rng.integers(1, 2501))
    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=seed * 7 + 3)
    wsb = w4.workspace_bytes(fmt, n, k, b)
    ws = torch.full((max(wsb, 16),), 0x7F, dtype=torch.uint8, device=xd.device)
    y = torch.full((b, n), float("nan"), device=xd.device)
    w4.matmul_ex(xd, p, s, fmt, workspace=ws, y=y)
    g.assert_y_close(fmt, y, x, pr, sr)
    splits = int(rng.integers(2, 17))
    wst = w4.workspace_bytes(fmt, n, k, b, "tiled", splits)
    wt = torch.full((max(wst, 16),), 0x7F, dtype=torch.uint8, device=xd.device)
    yt = torch.full((b, n), float("nan"), device=xd.device)
    w4.matmul_ex(xd, p, s, fmt, path="tiled", split_k=splits, workspace=wt, y=yt)
    g.assert_y_close(fmt, yt, x, pr, sr)
    # a grouped call: this matrix and one to three more of random row counts sharing x
    members = [(p, s, pr, sr)]
    for j in range(int(rng.integers(1, 4))):
        nj = int(rng.integers(1, 2501))
        w = synth_inputs.weights(nj, k, seed=seed * 31 + j)
        pj, sj = g.gpu_quantize(fmt, g.to_dev_f32(w))
        members.append((pj, sj) + tuple(g.oracle_quantize(fmt, w)))
    ys = [torch.full((b, m[0].shape[0]), float("nan"), device=xd.device) for m in members]
    w4.gemm_smallbatch_grouped(xd, [m[0] for m in members], [m[1] for m in members], fmt, ys=ys)
    for yg, m in zip(ys, members):
        g.assert_y_close(fmt, yg, x, m[2], m[3])
