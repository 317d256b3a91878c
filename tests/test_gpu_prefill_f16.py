"""Folded-scale prefill GEMM (W4_PATH_TILED_F16, fp16 activations) against the oracle's fp64
reference, per element within 2e-3 T + 1e-5 (T = sum over k of |x * w_hat|), as for every other
path; its fp32 block-scale loop for scales outside the fold range; the automatic choice inside the
tiled path."""
import numpy as np
import pytest

import synth_inputs
from tests import gpu_util as g

pytestmark = pytest.mark.gpu

F16_FMTS = ["nf4_f16", "int4_f16", "fp4_f16", "int4a_f16"]


def _case(fmt, n, k, b, seed, w=None):
    if w is None:
        w = synth_inputs.weights(n, k, seed=seed)
    x = synth_inputs.activations(b, k, "f16", seed=seed + 17)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    g.assert_quant_equal(fmt, p, s, pr, sr)
    return x, g.to_dev_x(x, "f16"), p, s, pr, sr


# Tiles are 128 weight rows x 128 activation rows over 64-weight blocks of K, eight blocks (two
# quads of scales) per unrolled trip: one block (NF4, FP4), five (no whole trip), six and ten (a
# remainder of two), 24 and 140 (three and four trips), ragged N and B in both tile directions,
# B = 1, several tiles.
@pytest.mark.parametrize("fmt", F16_FMTS)
@pytest.mark.parametrize("n,k,b", [(64, 128, 128), (37, 384, 130), (300, 1536, 512), (129, 8960, 200),
                                   (1000, 2048, 257), (96, 1024, 1), (65, 64, 33), (260, 320, 300),
                                   (33, 640, 129)])
def test_tiled_f16_parity(fmt, n, k, b):
    import torch

    import bit_weight_only_w4_amd as w4

    if fmt.startswith("int4") and k % 128:
        pytest.skip("INT4 groups are 128 weights")
    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=n * 7 + b)
    y = torch.full((b, n), float("nan"), device=xd.device)
    w4.matmul_ex(xd, p, s, fmt, path="tiled_f16", y=y)
    g.assert_y_close(fmt, y, x, pr, sr)
    assert torch.equal(y, w4.matmul_ex(xd, p, s, fmt, path="tiled_f16"))


@pytest.mark.parametrize("fmt", F16_FMTS)
def test_tiled_f16_scale_range(fmt):
    """Groups of 32 rows (one wave's rows) with ordinary scales, with one block per row scaled far
    below the fold range, with whole rows scaled far above it, and with zero rows: the waves that
    meet an unfoldable scale run all of K with the block scale applied in fp32, the others fold;
    every row within the bound, across the 128-row tiles of one launch."""
    import bit_weight_only_w4_amd as w4

    n, k, b = 512, 1536, 160
    grp = 128 if fmt.startswith("int4") else 64
    w = synth_inputs.weights(n, k, seed=41).astype(np.float64)
    rows = np.arange(n)
    kind = (rows // 32) % 4
    w[kind == 1, 3 * grp:4 * grp] *= 1e-7       # one block per row below the fold range
    w[kind == 2, :] *= 1e6                       # whole rows above it
    w[(kind == 3) & (rows % 2 == 0), :] = 0.0    # zero rows (scale 0 folds)
    w = w.astype(np.float32)
    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=42, w=w)
    y = w4.matmul_ex(xd, p, s, fmt, path="tiled_f16")
    g.assert_y_close(fmt, y, x, pr, sr)


@pytest.mark.parametrize("fmt", F16_FMTS)
@pytest.mark.parametrize("b", [128, 200])
def test_tiled_f16_one_hot_columns(fmt, b):
    """Activation row i = e_{c_i}: y[i] is column c_i of the decoded matrix up to the fp16
    rounding of the folded weight: exact for INT4 ((q - 8) s with a bf16 scale fits fp16), within
    2^-11 for asymmetric INT4 ((q - z) s rounded once), 2 * 2^-11 for FP4 (scale and product
    rounded), 3 * 2^-11 for NF4 (code, scale and product)."""
    import oracle

    import bit_weight_only_w4_amd as w4

    n, k = 300, 1024
    w = synth_inputs.weights(n, k, seed=78)
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    w_hat = oracle.dequant(g.WFMT[fmt], pr, sr)
    cols = [(41 * i + 3) % k for i in range(b)]
    x = np.zeros((b, k), dtype=np.uint16)
    for i, c in enumerate(cols):
        x[i, c] = 0x3C00
    y = w4.matmul_ex(g.to_dev_x(x, "f16"), p, s, fmt, path="tiled_f16").cpu().numpy()
    y = y.astype(np.float64)
    rtol = {"nf4_f16": 3 * 2.0 ** -11 + 2.0 ** -20, "fp4_f16": 2 * 2.0 ** -11 + 2.0 ** -20,
            "int4_f16": 0.0, "int4a_f16": 2.0 ** -11 + 2.0 ** -20}[fmt]
    for i, c in enumerate(cols):
        assert np.allclose(y[i], w_hat[:, c], rtol=rtol, atol=0), (i, c)


@pytest.mark.parametrize("fmt,n,k", [("nf4_f16", 33000, 320), ("fp4_f16", 33000, 320),
                                     ("int4_f16", 33000, 640)])
def test_tiled_f16_wide_tiles_sampled(fmt, n, k):
    """256-row tiles (chosen from two per CU) with K shorter than one unrolled trip (five blocks of
    64; INT4 ten) and a ragged last tile: 160 sampled rows against the oracle; the explicit path,
    the tiled path and the automatic path agree bitwise (the automatic choice is this kernel)."""
    import torch

    import bit_weight_only_w4_amd as w4

    dev = g.device()
    b = 512
    gen = torch.Generator(device=dev).manual_seed(n + k)
    w = torch.randn(n, k, generator=gen, device=dev) * 0.02
    p, s = g.gpu_quantize(fmt, w)
    rng = np.random.default_rng(n + 3)
    rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 158, replace=False)]))
    w_rows = w[torch.as_tensor(rows, device=dev)].cpu().numpy()
    del w
    pr, sr = g.oracle_quantize(fmt, w_rows)
    g.assert_quant_equal(fmt, p, s, pr, sr, rows=rows)
    x = synth_inputs.activations(b, k, "f16", seed=b + 5)
    xd = g.to_dev_x(x, "f16")
    y = w4.matmul_ex(xd, p, s, fmt, path="tiled_f16")
    g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)
    assert torch.equal(y, w4.matmul_ex(xd, p, s, fmt, path="tiled"))
    assert torch.equal(y, w4.gemm_prefill(xd, p, s, fmt))


@pytest.mark.parametrize("fmt", F16_FMTS)
def test_tiled_f16_grouped_members(fmt):
    """Three members of a 512-token grouped call large enough for the folded kernel (their tiles
    one after another in one launch): each bitwise equal to the folded kernel on that member
    alone and within the bound on sampled rows; y pre-filled with NaN."""
    import torch

    import bit_weight_only_w4_amd as w4

    dev = g.device()
    k, b = 1536, 512
    ns = (8960, 4100, 5000)
    x = synth_inputs.activations(b, k, "f16", seed=301)
    xd = g.to_dev_x(x, "f16")
    packed, scales, checks = [], [], []
    for i, n in enumerate(ns):
        gen = torch.Generator(device=dev).manual_seed(700 + i)
        w = torch.randn(n, k, generator=gen, device=dev) * 0.02
        p, s = g.gpu_quantize(fmt, w)
        rng = np.random.default_rng(31 + i)
        rows = np.unique(np.concatenate([[0, n - 1], rng.choice(n, 78, replace=False)]))
        w_rows = w[torch.as_tensor(rows, device=dev)].cpu().numpy()
        del w
        pr, sr = g.oracle_quantize(fmt, w_rows)
        packed.append(p)
        scales.append(s)
        checks.append((rows, pr, sr))
    ys = [torch.full((b, n), float("nan"), device=dev) for n in ns]
    w4.gemm_smallbatch_grouped(xd, packed, scales, fmt, ys=ys)
    for y, p, s, (rows, pr, sr) in zip(ys, packed, scales, checks):
        assert torch.equal(y, w4.matmul_ex(xd, p, s, fmt, path="tiled_f16"))
        g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=y.device)], x, pr, sr)


def test_tiled_f16_rejects_other_formats():
    """Formats with bf16 activations have no folded kernel: W4_ERR_PATH, y untouched."""
    import torch

    import bit_weight_only_w4_amd as w4

    for fmt in ("nf4_bf16", "int4_bf16", "fp4_bf16", "int4a_bf16"):
        x, xd, p, s, pr, sr = _case(fmt, 64, 256, 128, seed=3)
        y = torch.full((128, 64), 7.0, device=xd.device)
        with pytest.raises(ValueError):
            w4.matmul_ex(xd, p, s, fmt, path="tiled_f16", y=y)
        assert bool((y == 7.0).all())


@pytest.mark.parametrize("seed", range(24))
def test_tiled_f16_random_shapes(seed):
    """Seeded random shapes on the folded kernel, forced: format, N (1..3000), K (a multiple of the
    format's group up to 4096) and B (1..700) drawn from the seed; y pre-filled with NaN; every
    element against the oracle; 128-row tiles (the forced path's choice below the automatic
    thresholds)."""
    import torch

    import bit_weight_only_w4_amd as w4

    rng = np.random.default_rng(5000 + seed)
    fmt = F16_FMTS[int(rng.integers(len(F16_FMTS)))]
    grp = 128 if fmt.startswith("int4") else 64
    k = grp * int(rng.integers(1, 4096 // grp + 1))
    b = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 257)), int(rng.integers(257, 701))]))
    n = int(rng.integers(1, 3001))
    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=seed * 11 + 1)
    y = torch.full((b, n), float("nan"), device=xd.device)
    w4.matmul_ex(xd, p, s, fmt, path="tiled_f16", y=y)
    g.assert_y_close(fmt, y, x, pr, sr)


# K split into ranges of whole blocks (their partial sums added in range order): ragged last
# ranges, ranges shorter than one unrolled trip of eight blocks, INT4 ranges rounded to an even
# block count (k = 640: S = 4 gives ranges of 4, 4 and 2 blocks), a range of one block.
@pytest.mark.parametrize("fmt", F16_FMTS)
@pytest.mark.parametrize("n,k,b,splits", [(300, 8960, 300, 5), (129, 4096, 512, 3), (64, 1536, 256, 7),
                                          (37, 640, 130, 4), (200, 1024, 129, 16), (1536, 2048, 40, 2)])
def test_tiled_f16_split_k(fmt, n, k, b, splits):
    import torch

    import bit_weight_only_w4_amd as w4

    if fmt.startswith("int4") and k % 128:
        pytest.skip("INT4 groups are 128 weights")
    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=n * 5 + splits)
    wsb = w4.workspace_bytes(fmt, n, k, b, "tiled_f16", splits)
    assert wsb > 0
    ws = torch.full((wsb // 4,), float("nan"), device=xd.device).view(torch.uint8)
    y = torch.full((b, n), float("nan"), device=xd.device)
    w4.matmul_ex(xd, p, s, fmt, path="tiled_f16", split_k=splits, workspace=ws, y=y)
    g.assert_y_close(fmt, y, x, pr, sr)
    y2 = w4.matmul_ex(xd, p, s, fmt, path="tiled_f16", split_k=splits, workspace=ws)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("fmt", F16_FMTS)
def test_tiled_f16_split_k_scale_range(fmt):
    """The scale-range rows of the unsplit test, K split in three: a wave whose range holds an
    unfoldable scale takes the fp32 route for that range only; every row within the bound."""
    import torch

    import bit_weight_only_w4_amd as w4

    n, k, b = 512, 1536, 160
    grp = 128 if fmt.startswith("int4") else 64
    w = synth_inputs.weights(n, k, seed=41).astype(np.float64)
    rows = np.arange(n)
    kind = (rows // 32) % 4
    w[kind == 1, 3 * grp:4 * grp] *= 1e-7
    w[kind == 2, :] *= 1e6
    w[(kind == 3) & (rows % 2 == 0), :] = 0.0
    w = w.astype(np.float32)
    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=42, w=w)
    ws = torch.empty(w4.workspace_bytes(fmt, n, k, b, "tiled_f16", 3), dtype=torch.uint8,
                     device=xd.device)
    y = w4.matmul_ex(xd, p, s, fmt, path="tiled_f16", split_k=3, workspace=ws)
    g.assert_y_close(fmt, y, x, pr, sr)


def _tail_case(fmt, ns, k, b, seed):
    """Members drawn on the GPU, quantized there, with rows sampled for the oracle: the last 128-row
    tiles of the last member (the launch's last round) always among them."""
    import torch

    dev = g.device()
    packed, scales, checks = [], [], []
    for i, n in enumerate(ns):
        gen = torch.Generator(device=dev).manual_seed(seed + i)
        w = torch.randn(n, k, generator=gen, device=dev) * 0.02
        p, s = g.gpu_quantize(fmt, w)
        rng = np.random.default_rng(seed + 100 + i)
        last = np.arange(max(0, n - 300), n)
        rows = np.unique(np.concatenate([[0], rng.choice(n, 60, replace=False), last[::3]]))
        w_rows = w[torch.as_tensor(rows, device=dev)].cpu().numpy()
        del w
        pr, sr = g.oracle_quantize(fmt, w_rows)
        packed.append(p)
        scales.append(s)
        checks.append((rows, pr, sr))
    return packed, scales, checks


# The tiled path runs a one-pass launch whose last round of 128-row tiles holds at most CUs / 4
# tiles as a second launch of 32-row slices (on 256 CUs: 513..576 tiles, 1025..1088, ...):
# gate|up as one grouped call at 512 and at 400 activation rows (the last 128-row tile 16 rows:
# its slices past row 400 do nothing), and one 17000-row matrix (133 x 4 = 532 tiles).  Every
# output written (y pre-filled with NaN), sampled rows within the bound, the grouped call bitwise
# equal to its members alone (their launches have no such round), two calls bitwise equal.
@pytest.mark.parametrize("fmt", F16_FMTS)
@pytest.mark.parametrize("ns,b", [((8960, 8960), 512), ((8960, 8960), 400), ((17000,), 512)])
def test_tiled_f16_last_round_slices(fmt, ns, b):
    import torch

    import bit_weight_only_w4_amd as w4

    k = 1536
    dev = g.device()
    x = synth_inputs.activations(b, k, "f16", seed=b + len(ns))
    xd = g.to_dev_x(x, "f16")
    packed, scales, checks = _tail_case(fmt, ns, k, b, seed=900 + b)
    ys = [torch.full((b, n), float("nan"), device=dev) for n in ns]
    if len(ns) > 1:
        w4.gemm_smallbatch_grouped(xd, packed, scales, fmt, ys=ys)
    else:
        w4.matmul_ex(xd, packed[0], scales[0], fmt, path="tiled", y=ys[0])
    for y, p, s, (rows, pr, sr) in zip(ys, packed, scales, checks):
        assert bool(torch.isfinite(y).all())
        g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=dev)], x, pr, sr)
        alone = w4.matmul_ex(xd, p, s, fmt, path="tiled_f16")
        if len(ns) > 1:
            assert torch.equal(y, alone)
        else:
            assert torch.equal(y, w4.matmul_ex(xd, p, s, fmt, path="tiled"))


@pytest.mark.parametrize("splits", [1, 3])
def test_tiled_f16_int4a_zero_points(splits):
    """Asymmetric INT4 with zero points at the ends of the grid: rows of one sign only (zero
    point 0 or 15, so the zero-point term carries most of each weight) next to ordinary rows,
    folded as ((q - 8) + (8 - z)) s; every element within the bound, in one pass and over K
    ranges."""
    import torch

    import bit_weight_only_w4_amd as w4

    fmt = "int4a_f16"
    n, k, b = 384, 2048, 300
    w = synth_inputs.weights(n, k, seed=77).astype(np.float64)
    rows = np.arange(n)
    w[rows % 3 == 1] = np.abs(w[rows % 3 == 1]) + 0.01
    w[rows % 3 == 2] = -np.abs(w[rows % 3 == 2]) - 0.01
    w = w.astype(np.float32)
    x, xd, p, s, pr, sr = _case(fmt, n, k, b, seed=78, w=w)
    z = (sr >> 16) & 15
    assert (z[rows % 3 == 1] <= 1).all() and (z[rows % 3 == 2] >= 14).all()
    ws = None
    if splits > 1:
        ws = torch.empty(w4.workspace_bytes(fmt, n, k, b, "tiled_f16", splits), dtype=torch.uint8,
                         device=xd.device)
    y = w4.matmul_ex(xd, p, s, fmt, path="tiled_f16", split_k=splits, workspace=ws)
    g.assert_y_close(fmt, y, x, pr, sr)


# 129 to 192 activation rows over at least one 128-weight-row tile per CU run as one 192-row tile
# per weight tile (33000 rows: 258 tiles): ragged B inside the tile, every output written (y
# pre-filled with NaN), sampled rows within the bound, and the rows bitwise equal to the same rows
# computed as 128 + (b - 128) rows in two calls (128-row tiles; the sums over K take the same
# order in either tile), and to the automatic path.
@pytest.mark.parametrize("fmt", F16_FMTS)
@pytest.mark.parametrize("b", [129, 160, 192])
def test_tiled_f16_192_row_tiles(fmt, b):
    import torch

    import bit_weight_only_w4_amd as w4

    n, k = 33000, 640
    dev = g.device()
    packed, scales, checks = _tail_case(fmt, (n,), k, b, seed=700 + b)
    p, s, (rows, pr, sr) = packed[0], scales[0], checks[0]
    x = synth_inputs.activations(b, k, "f16", seed=b + 11)
    xd = g.to_dev_x(x, "f16")
    y = torch.full((b, n), float("nan"), device=dev)
    w4.matmul_ex(xd, p, s, fmt, path="tiled_f16", y=y)
    assert bool(torch.isfinite(y).all())
    g.assert_y_close(fmt, y[:, torch.as_tensor(rows, device=dev)], x, pr, sr)
    top = w4.matmul_ex(xd[:128].contiguous(), p, s, fmt, path="tiled_f16")
    rest = w4.matmul_ex(xd[128:].contiguous(), p, s, fmt, path="tiled_f16")
    assert torch.equal(y[:128], top)
    assert torch.equal(y[128:], rest)
    assert torch.equal(y, w4.gemm_prefill(xd, p, s, fmt))
