"""w4_matmul_splitk_noalloc (split-K with the library's static scratch instead of a workspace)
through the C ABI against w4_matmul_ex with W4_PATH_SPLITK and a caller's workspace: bitwise
equal (same kernels, same split count) and within the oracle's bound, on two calls in a row whose
second is smaller (the scratch keeps the first call's partials; nothing may leak into the second),
plus the size limit."""
import ctypes

import numpy as np
import pytest

import synth_inputs
from tests import gpu_util as g

pytestmark = pytest.mark.gpu


def _noalloc(L, xd, p, s, fmt_id, n, k, b, y, split_k):
    vp = ctypes.c_void_p
    return L.w4_matmul_splitk_noalloc(vp(xd.data_ptr()), vp(p.data_ptr()), vp(s.data_ptr()),
                                      fmt_id, n, k, b, vp(y.data_ptr()), split_k, None)


@pytest.mark.parametrize("fmt", ["nf4_f16", "int4_bf16", "int4a_f16"])
def test_noalloc_splitk_equals_workspace_splitk_twice(fmt):
    import torch

    import bit_weight_only_w4_amd as w4

    L = w4.lib()
    dev = g.device()
    cases = [(1536, 8960, 8, 16), (300, 1536, 3, 4)]  # the second call is smaller
    for n, k, b, split_k in cases:
        w = synth_inputs.weights(n, k, seed=n + b)
        x = synth_inputs.activations(b, k, g.XDT[fmt], seed=k + b)
        xd = g.to_dev_x(x, g.XDT[fmt])
        p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
        pr, sr = g.oracle_quantize(fmt, w)
        g.assert_quant_equal(fmt, p, s, pr, sr)
        y = torch.full((b, n), float("nan"), device=dev)
        assert _noalloc(L, xd, p, s, w4.FORMATS[fmt], n, k, b, y, split_k) == 0
        ws = torch.empty(w4.workspace_bytes(fmt, n, k, b, "splitk", split_k), dtype=torch.uint8,
                         device=dev)
        ref = w4.matmul_ex(xd, p, s, fmt, path="splitk", split_k=split_k, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
        g.assert_y_close(fmt, y, x, pr, sr)


def test_noalloc_limits():
    import torch

    import bit_weight_only_w4_amd as w4

    L = w4.lib()
    dev = g.device()
    n, k, b = 151936, 1536, 8
    fmt = "nf4_f16"
    x = torch.zeros(b, k, dtype=torch.float16, device=dev)
    p = torch.zeros(n, k // 2, dtype=torch.uint8, device=dev)
    s = torch.zeros(n, k // 64, dtype=torch.float32, device=dev)
    y = torch.empty(b, n, device=dev)
    assert 4 * 16 * b * n > w4.NOALLOC_SCRATCH_BYTES
    assert _noalloc(L, x, p, s, w4.FORMATS[fmt], n, k, b, y, 16) == -6  # beyond the scratch
    assert _noalloc(L, x, p, s, w4.FORMATS[fmt], n, k, b, y, 1) == -7  # not a split
    assert _noalloc(L, x, p, s, w4.FORMATS[fmt], n, k, 9, y, 4) == -7  # B beyond the GEMV
    # the largest call that fits: 4 * S * B * N == the scratch size exactly
    n2 = w4.NOALLOC_SCRATCH_BYTES // (4 * 2 * 8)
    y2 = torch.full((8, n2), float("nan"), device=dev)
    assert _noalloc(L, x, p[:n2], s[:n2], w4.FORMATS[fmt], n2, k, 8, y2, 2) == 0
    torch.cuda.synchronize()
    assert torch.equal(y2, torch.zeros_like(y2))
