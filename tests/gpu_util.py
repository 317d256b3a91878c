"""Helpers shared by the GPU tests: move seeded inputs to the device, run the oracle beside the
library, and compare."""
from __future__ import annotations

import numpy as np

import oracle

WFMT = {"nf4_f16": "nf4", "nf4_bf16": "nf4", "int4_f16": "int4", "int4_bf16": "int4",
        "fp4_f16": "fp4", "fp4_bf16": "fp4", "int4a_f16": "int4a", "int4a_bf16": "int4a"}
XDT = {f: f.split("_")[1] for f in WFMT}


def device():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda:0")


def to_dev_f32(w: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(device())


def to_dev_x(x_bits: np.ndarray, xdt: str):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16))
    t = t.view(torch.float16 if xdt == "f16" else torch.bfloat16)
    return t.to(device()).contiguous()


def gpu_quantize(fmt: str, w_dev):
    import bit_weight_only_w4_amd as w4

    return w4.quantize(fmt, w_dev)


def scales_to_np(fmt: str, s_dev) -> np.ndarray:
    s = s_dev.cpu().numpy()
    if WFMT[fmt] == "int4a":
        return s.view(np.uint32)
    return s if WFMT[fmt] in ("nf4", "fp4") else s.view(np.uint16)


def oracle_quantize(fmt: str, w: np.ndarray):
    return {"nf4": oracle.quantize_nf4, "int4": oracle.quantize_int4, "fp4": oracle.quantize_fp4,
            "int4a": oracle.quantize_int4_asym}[WFMT[fmt]](w)


def assert_quant_equal(fmt, packed_dev, scales_dev, packed_ref, scales_ref, rows=None):
    p = packed_dev.cpu().numpy()
    s = scales_to_np(fmt, scales_dev)
    if rows is not None:
        p, s = p[rows], s[rows]
    assert p.shape == packed_ref.shape
    bad = np.argwhere(p != packed_ref)
    assert bad.size == 0, f"{len(bad)} packed bytes differ, first at {bad[:5].tolist()}"
    sv = s.view(np.uint32) if s.dtype in (np.float32, np.int32) else s
    rv = scales_ref.view(np.uint32) if scales_ref.dtype in (np.float32, np.int32) else scales_ref
    bad = np.argwhere(sv != rv)
    assert bad.size == 0, f"{len(bad)} scales differ, first at {bad[:5].tolist()}"


def assert_y_close(fmt, y_dev, x_bits, packed_ref, scales_ref, rows=None):
    """Check GPU y (rows `rows` of W, or all) against the oracle's fp64 reference and bound."""
    y = y_dev.cpu().numpy().astype(np.float64)
    if rows is not None:
        packed_ref = packed_ref[rows]
        scales_ref = scales_ref[rows]
        y = y[:, rows]
    w_hat = oracle.dequant(WFMT[fmt], packed_ref, scales_ref)
    y_ref, t = oracle.gemv_reference(x_bits, XDT[fmt], w_hat)
    ratio = oracle.violation_ratio(y, y_ref, t)
    assert ratio <= 1.0, f"tolerance violated: max |dy| / bound = {ratio:.3f}"
    return ratio
