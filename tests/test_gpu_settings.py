"""w4_set_path / w4_set_workspace steering w4_gemv and w4_gemm_smallbatch on the GPU, and the
quantizers' non-finite reports under concurrent calls from two threads on two streams."""
import threading

import numpy as np
import pytest

import synth_inputs
from tests import gpu_util as g

pytestmark = pytest.mark.gpu


def test_forced_paths_equal_explicit_calls():
    import torch

    import bit_weight_only_w4_amd as w4

    fmt, n, k, b = "int4_bf16", 1536, 8960, 2
    w = synth_inputs.weights(n, k, seed=5)
    x = synth_inputs.activations(b, k, "bf16", seed=6)
    xd = g.to_dev_x(x, "bf16")
    p, s = g.gpu_quantize(fmt, g.to_dev_f32(w))
    pr, sr = g.oracle_quantize(fmt, w)
    ws = torch.empty(n * k * 2, dtype=torch.uint8, device=g.device())
    try:
        w4.set_workspace(ws)
        for path, extra in (("splitk", {"split_k": 4}), ("mfma", {}), ("twopass", {}),
                            ("gemv", {}), ("tiled", {})):
            w4.set_path(path)
            assert w4.get_path() == path
            y_gemv = w4.gemv(xd, p, s, fmt)
            y_small = w4.gemm_smallbatch(xd, p, s, fmt)
            ref = w4.matmul_ex(xd, p, s, fmt, path=path, workspace=ws, **extra)
            assert torch.equal(y_gemv, ref), path
            assert torch.equal(y_small, ref), path
            g.assert_y_close(fmt, y_gemv, x, pr, sr)
        w4.set_path("auto")
        assert torch.equal(w4.gemv(xd, p, s, fmt), w4.matmul_ex(xd, p, s, fmt, path="gemv"))
        w4.set_workspace(None)
        w4.set_path("splitk")
        with pytest.raises(ValueError):
            w4.gemv(xd, p, s, fmt)  # nothing registered any more
    finally:
        w4.set_path("auto")
        w4.set_workspace(None)
    torch.cuda.synchronize()


def test_concurrent_quantize_calls_keep_their_own_nonfinite_report():
    """Two threads quantize at the same time on two streams, one matrix with a NaN and one clean:
    each call reports its own result every time (the flag word is reset, set and read under a
    host lock)."""
    import ctypes

    import torch

    import bit_weight_only_w4_amd as w4

    dev = g.device()
    n, k = 2048, 1536
    clean = torch.randn(n, k, device=dev) * 0.02
    dirty = clean.clone()
    dirty[n // 2, 77] = float("nan")
    L = w4.lib()
    vp = ctypes.c_void_p
    results = {"clean": [], "dirty": []}

    def worker(name, w):
        st = torch.cuda.Stream(device=dev)
        packed = torch.empty(n, k // 2, dtype=torch.uint8, device=dev)
        absmax = torch.empty(n, k // 64, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for _ in range(40):
            r = L.w4_quantize_nf4(vp(w.data_ptr()), n, k, vp(packed.data_ptr()),
                                  vp(absmax.data_ptr()), vp(st.cuda_stream))
            results[name].append(r)

    ts = [threading.Thread(target=worker, args=("clean", clean)),
          threading.Thread(target=worker, args=("dirty", dirty))]
    for t in ts:
        t.start()
    for t in ts:
        t.join(timeout=120)
    assert results["clean"] == [0] * 40
    assert results["dirty"] == [-5] * 40
