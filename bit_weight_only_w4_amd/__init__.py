"""Python binding of the W4 C ABI (include/w4.h).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libw4.so``.  PyTorch supplies device memory and the current stream.  There is no fallback:
if the library is not built, every call raises ``RuntimeError``.

Formats are named ``"nf4_f16"``, ``"nf4_bf16"``, ``"int4_f16"`` and ``"int4_bf16"`` (weight format
x activation dtype).  Scales are fp32 ``[N, K/64]`` for NF4 and bf16 bit patterns stored in an
int16 tensor ``[N, K/128]`` for INT4.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libw4.so")

FORMATS = {"nf4_f16": 1, "nf4_bf16": 2, "int4_f16": 3, "int4_bf16": 4, "fp4_f16": 5, "fp4_bf16": 6,
           "int4a_f16": 7, "int4a_bf16": 8}
PATHS = {"auto": 0, "gemv": 1, "splitk": 2, "mfma": 3, "twopass": 4, "tiled": 5, "tiled_f16": 6}
PATH_NAMES = {v: k for k, v in PATHS.items()}
STATUS = {0: "OK", -1: "NULL", -2: "SHAPE", -3: "ALIGN", -4: "FORMAT", -5: "NONFINITE",
          -6: "WORKSPACE", -7: "PATH", -8: "HIP", -9: "ALIAS"}
MAX_BATCH = 4096
TILED_FROM_BATCH = 128
TILED_FROM_ROWS = 4096
MAX_SPLIT_K = 64
NOALLOC_SCRATCH_BYTES = 8 << 20

_lib = None


class W4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class W4ValueError(W4Error, ValueError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded ``libw4.so``; raises RuntimeError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"W4 HIP library not built ({LIB_PATH} missing); run "
                "`python -m bit_weight_only_w4_amd.build` on a machine with ROCm")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, sz, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.w4_quantize_nf4.argtypes = [vp, i64, i64, vp, vp, vp]
        L.w4_quantize_int4.argtypes = [vp, i64, i64, vp, vp, vp]
        L.w4_quantize_fp4.argtypes = [vp, i64, i64, vp, vp, vp]
        L.w4_quantize_int4_asym.argtypes = [vp, i64, i64, vp, vp, vp]
        L.w4_gptq_block_update.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, i64, i64, vp, vp,
                                           vp, vp]
        L.w4_gptq_lazy_update.argtypes = [vp, vp, vp, i64, i64, i64, i64, vp]
        L.w4_gptq_quantize.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, i64, vp, vp, vp, vp]
        L.w4_sparse24_compress.argtypes = [vp, i64, i64, ci, vp, vp, vp]
        L.w4_sparse24_gemv.argtypes = [vp, vp, vp, ci, i64, i64, i64, vp, vp]
        L.w4_sparse24_gemv_grouped.argtypes = [vp, ci, vp, vp, vp, ci, i64, i64, vp, vp]
        L.w4_gemv.argtypes = [vp, vp, vp, ci, i64, i64, i64, vp, vp]
        L.w4_gemm_smallbatch.argtypes = [vp, vp, vp, ci, i64, i64, i64, vp, vp]
        L.w4_gemm_prefill.argtypes = [vp, vp, vp, ci, i64, i64, i64, vp, vp]
        L.w4_matmul_ex.argtypes = [vp, vp, vp, ci, i64, i64, i64, vp, ci, ci, vp, sz, vp]
        L.w4_workspace_bytes.argtypes = [ci, i64, i64, i64, ci, ci]
        L.w4_workspace_bytes.restype = sz
        L.w4_auto_path.argtypes = [ci, i64, i64, i64, sz, ctypes.POINTER(ci)]
        ip = ctypes.POINTER(ci)
        L.w4_gemv_plan.argtypes = [ci, i64, i64, i64, ci, ip, ip, ip, ip, ip]
        L.w4_nf4_codebook.restype = ctypes.POINTER(ctypes.c_float)
        L.w4_status_string.argtypes = [ci]
        L.w4_status_string.restype = ctypes.c_char_p
        vpp = ctypes.POINTER(vp)
        L.w4_gemv_grouped.argtypes = [vp, ci, vpp, vpp, ctypes.POINTER(i64), vpp, ci, i64, i64, vp]
        L.w4_gemm_smallbatch_grouped.argtypes = [vp, ci, vpp, vpp, ctypes.POINTER(i64), vpp, ci, i64,
                                                 i64, vp]
        L.w4_gemv_grouped_plan.argtypes = [ci, ci, ctypes.POINTER(i64), i64, i64, ip, ip, ip, ip, ip]
        L.w4_probe_read.argtypes = [vp, sz, vp, vp]
        L.w4_probe_copy.argtypes = [vp, vp, sz, vp]
        L.w4_matmul_splitk_noalloc.argtypes = [vp, vp, vp, ci, i64, i64, i64, vp, ci, vp]
        L.w4_set_path.argtypes = [ci]
        L.w4_get_path.argtypes = []
        L.w4_set_workspace.argtypes = [vp, sz]
        for name in ("w4_quantize_nf4", "w4_quantize_int4", "w4_quantize_fp4", "w4_quantize_int4_asym",
                     "w4_gemv", "w4_gemm_smallbatch", "w4_matmul_ex", "w4_auto_path",
                     "w4_gemv_plan", "w4_version", "w4_probe_read", "w4_probe_copy",
                     "w4_gemv_grouped", "w4_gemv_grouped_plan", "w4_gemm_smallbatch_grouped",
                     "w4_gemm_prefill", "w4_gptq_block_update", "w4_gptq_lazy_update",
                     "w4_gptq_quantize", "w4_sparse24_compress", "w4_sparse24_gemv",
                     "w4_sparse24_gemv_grouped", "w4_set_path", "w4_get_path",
                     "w4_matmul_splitk_noalloc",
                     "w4_set_workspace"):
            getattr(L, name).restype = ci
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().w4_status_string(int(status)).decode()


def check(status: int, what: str = "w4") -> None:
    if status == 0:
        return
    msg = f"{what}: {STATUS.get(status, status)} ({status_string(status)})"
    if status == -8:
        raise W4Error(status, msg)
    raise W4ValueError(status, msg)


def nf4_codebook():
    """The 16 fp32 NF4 code points the kernels decode with (host copy from the library)."""
    p = lib().w4_nf4_codebook()
    return [p[i] for i in range(16)]


def _fmt(fmt) -> int:
    if isinstance(fmt, int):
        return fmt
    try:
        return FORMATS[fmt]
    except KeyError:
        raise ValueError(f"unknown format {fmt!r}; expected one of {sorted(FORMATS)}") from None


def _stream(stream=None) -> int:
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous and on the GPU")


def quantize_nf4(w, stream=None):
    """fp32 [N, K] device weights -> (packed uint8 [N, K/2], absmax fp32 [N, K/64])."""
    import torch

    _need_cuda(w)
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor")
    n, k = w.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    absmax = torch.empty((n, max(k // 64, 1)), dtype=torch.float32, device=w.device)
    check(lib().w4_quantize_nf4(_ptr(w), n, k, _ptr(packed), _ptr(absmax), _stream(stream)),
          "w4_quantize_nf4")
    return packed, absmax


def quantize_fp4(w, stream=None):
    """fp32 [N, K] device weights -> (packed uint8 [N, K/2], scale fp32 [N, K/64]) in FP4 (E2M1)."""
    import torch

    _need_cuda(w)
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor")
    n, k = w.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scale = torch.empty((n, max(k // 64, 1)), dtype=torch.float32, device=w.device)
    check(lib().w4_quantize_fp4(_ptr(w), n, k, _ptr(packed), _ptr(scale), _stream(stream)),
          "w4_quantize_fp4")
    return packed, scale


def quantize_int4(w, stream=None):
    """fp32 [N, K] device weights -> (packed uint8 [N, K/2], bf16 scale bits int16 [N, K/128])."""
    import torch

    _need_cuda(w)
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor")
    n, k = w.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    scale = torch.empty((n, max(k // 128, 1)), dtype=torch.int16, device=w.device)
    check(lib().w4_quantize_int4(_ptr(w), n, k, _ptr(packed), _ptr(scale), _stream(stream)),
          "w4_quantize_int4")
    return packed, scale


def quantize_int4_asym(w, stream=None):
    """fp32 [N, K] device weights -> (packed uint8 [N, K/2], words int32 [N, K/128]) in asymmetric
    INT4: each word holds the group's bf16 scale bits (bits 0-15) and zero point (bits 16-19)."""
    import torch

    _need_cuda(w)
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor")
    n, k = w.shape
    packed = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    words = torch.empty((n, max(k // 128, 1)), dtype=torch.int32, device=w.device)
    check(lib().w4_quantize_int4_asym(_ptr(w), n, k, _ptr(packed), _ptr(words), _stream(stream)),
          "w4_quantize_int4_asym")
    return packed, words


def weight_format(fmt: str) -> str:
    """"nf4", "int4", "int4a" or "fp4": the weight encoding of a format name such as "fp4_bf16"."""
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    return fmt.split("_")[0]


def quantize(fmt: str, w, stream=None):
    """Quantize fp32 [N, K] device weights in the weight encoding of `fmt` (activation type aside):
    the packed nibbles and the scales that the matmul entry points take for that format."""
    q = {"nf4": quantize_nf4, "int4": quantize_int4, "int4a": quantize_int4_asym,
         "fp4": quantize_fp4}[weight_format(fmt)]
    return q(w, stream)


def _mm_shapes(x, packed):
    if x.dim() == 1:
        x = x.unsqueeze(0)
    b, k = x.shape
    n = packed.shape[0]
    return x, n, k, b


def gemv(x, packed, scales, fmt, y=None, stream=None):
    """y[B, N] = x[B, K] . W_hat^T via the fused single-pass GEMV (B <= 8)."""
    import torch

    x, n, k, b = _mm_shapes(x, packed)
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _need_cuda(x, packed, scales, y)
    check(lib().w4_gemv(_ptr(x), _ptr(packed), _ptr(scales), _fmt(fmt), n, k, b, _ptr(y),
                        _stream(stream)), "w4_gemv")
    return y


def grouped_args(x, packed, scales, ys):
    """ctypes arrays for w4_gemv_grouped: (packed**, scales**, N*, y**) over the members."""
    g = len(packed)
    vp = ctypes.c_void_p
    return ((vp * g)(*[p.data_ptr() for p in packed]), (vp * g)(*[s.data_ptr() for s in scales]),
            (ctypes.c_int64 * g)(*[p.shape[0] for p in packed]),
            (vp * g)(*[y.data_ptr() for y in ys]))


def _grouped_call(entry, x, packed, scales, fmt, ys, stream):
    import torch

    if len(packed) != len(scales) or (ys is not None and len(ys) != len(packed)):
        raise ValueError("packed, scales and ys must have one entry per member")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    b, k = x.shape
    if ys is None:
        ys = [torch.empty((b, p.shape[0]), dtype=torch.float32, device=x.device) for p in packed]
    _need_cuda(x, *packed, *scales, *ys)
    pp, sp, n, yp = grouped_args(x, packed, scales, ys)
    check(getattr(lib(), entry)(_ptr(x), len(packed), pp, sp, n, yp, _fmt(fmt), k, b,
                                _stream(stream)), entry)
    return ys


def gemv_grouped(x, packed, scales, fmt, ys=None, stream=None):
    """[y_g] = [x . W_hat_g^T] for weight matrices that share x, in one fused-GEMV launch.
    packed / scales are equal-length lists (at most 4 members); returns the list of y_g [B, N_g]."""
    return _grouped_call("w4_gemv_grouped", x, packed, scales, fmt, ys, stream)


def gemm_smallbatch_grouped(x, packed, scales, fmt, ys=None, stream=None):
    """gemv_grouped for batches up to W4_MAX_BATCH: one launch of the kernel the automatic path
    picks for the members' summed rows (the fused GEMV, or the MFMA kernel for larger batches);
    from W4_TILED_FROM_BATCH rows one tiled launch over the members of TILED_FROM_ROWS rows and
    more, one MFMA launch over the others."""
    return _grouped_call("w4_gemm_smallbatch_grouped", x, packed, scales, fmt, ys, stream)


def gemm_smallbatch(x, packed, scales, fmt, y=None, stream=None):
    """y[B, N] = x[B, K] . W_hat^T for B <= MAX_BATCH, GEMV, MFMA or tiled path chosen by the
    library."""
    import torch

    x, n, k, b = _mm_shapes(x, packed)
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _need_cuda(x, packed, scales, y)
    check(lib().w4_gemm_smallbatch(_ptr(x), _ptr(packed), _ptr(scales), _fmt(fmt), n, k, b,
                                   _ptr(y), _stream(stream)), "w4_gemm_smallbatch")
    return y


def gemm_prefill(x, packed, scales, fmt, y=None, stream=None):
    """y[B, N] = x[B, K] . W_hat^T through the tiled GEMM (prefill: B = prompt tokens)."""
    import torch

    x, n, k, b = _mm_shapes(x, packed)
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _need_cuda(x, packed, scales, y)
    check(lib().w4_gemm_prefill(_ptr(x), _ptr(packed), _ptr(scales), _fmt(fmt), n, k, b,
                                _ptr(y), _stream(stream)), "w4_gemm_prefill")
    return y


def workspace_bytes(fmt, n, k, b, path="auto", split_k=0) -> int:
    return int(lib().w4_workspace_bytes(_fmt(fmt), n, k, b, PATHS[path], split_k))


def auto_path(fmt, n, k, b, workspace_bytes=0):
    """(path name, split count) that the automatic choice would run."""
    sk = ctypes.c_int(0)
    r = lib().w4_auto_path(_fmt(fmt), n, k, b, workspace_bytes, ctypes.byref(sk))
    if r < 0:
        check(r, "w4_auto_path")
    return PATH_NAMES[r], sk.value


def gemv_plan(fmt, n, k, b, split_k=1):
    """dict(threads, team, iters, chunks_per_split, grid_x) of the fused GEMV launch."""
    vals = [ctypes.c_int(0) for _ in range(5)]
    r = lib().w4_gemv_plan(_fmt(fmt), n, k, b, split_k, *[ctypes.byref(v) for v in vals])
    check(r, "w4_gemv_plan")
    return dict(zip(("threads", "team", "iters", "chunks_per_split", "grid_x"),
                    (v.value for v in vals)))


def gemv_grouped_plan(fmt, ns, k, b):
    """dict(threads, team, iters, grid_x, grid_z) of the grouped fused-GEMV launch over members
    of ns rows."""
    vals = [ctypes.c_int(0) for _ in range(5)]
    arr = (ctypes.c_int64 * len(ns))(*ns)
    r = lib().w4_gemv_grouped_plan(_fmt(fmt), len(ns), arr, k, b, *[ctypes.byref(v) for v in vals])
    check(r, "w4_gemv_grouped_plan")
    return dict(zip(("threads", "team", "iters", "grid_x", "grid_z"), (v.value for v in vals)))


def matmul_ex(x, packed, scales, fmt, path="auto", split_k=0, workspace=None, y=None,
              stream=None):
    """The same product with an explicit path, split count and workspace (a uint8 tensor)."""
    import torch

    x, n, k, b = _mm_shapes(x, packed)
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    _need_cuda(x, packed, scales, y, workspace)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib().w4_matmul_ex(_ptr(x), _ptr(packed), _ptr(scales), _fmt(fmt), n, k, b, _ptr(y),
                             PATHS[path], int(split_k), _ptr(workspace), wbytes, _stream(stream)),
          f"w4_matmul_ex[{path}]")
    return y


def set_path(path) -> None:
    """Override the automatic path of w4_gemv / w4_gemm_smallbatch ("auto" removes it)."""
    check(lib().w4_set_path(PATHS[path] if isinstance(path, str) else int(path)), "w4_set_path")


def get_path() -> str:
    """The current override's name; raises if W4_FORCE_PATH held an unknown value."""
    r = lib().w4_get_path()
    if r < 0:
        check(r, "w4_get_path")
    return PATH_NAMES[r]


def set_workspace(ws=None) -> None:
    """Register a device tensor (or None to unregister) as the current device's workspace for
    w4_gemv / w4_gemm_smallbatch.  The caller keeps the tensor alive while it is registered."""
    if ws is None:
        check(lib().w4_set_workspace(None, 0), "w4_set_workspace")
    else:
        _need_cuda(ws)
        check(lib().w4_set_workspace(_ptr(ws), ws.numel() * ws.element_size()), "w4_set_workspace")


def probe_read(src, sink, stream=None):
    _need_cuda(src, sink)
    check(lib().w4_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                              _stream(stream)), "w4_probe_read")


def probe_copy(src, dst, stream=None):
    _need_cuda(src, dst)
    check(lib().w4_probe_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(),
                              _stream(stream)), "w4_probe_copy")


def _gptq_args(w, u, scale, zero, group):
    import torch

    _need_cuda(w, u, scale, zero)
    for t in (w, u, scale, zero):
        if t.dtype != torch.float32 or t.dim() != 2:
            raise ValueError("w, u, scale and zero must be 2-D float32 tensors")
    rows, cols = w.shape
    if tuple(u.shape) != (cols, cols):
        raise ValueError("u must be [cols, cols]")
    group = cols if group is None else int(group)
    if group < 1 or cols % group or tuple(scale.shape) != (rows, cols // group) or \
            tuple(zero.shape) != (rows, cols // group):
        raise ValueError("scale and zero must be [rows, cols // group]")
    return rows, cols, group


def gptq_outputs(w):
    """Empty (q_hat fp32, codes uint8, err fp32) buffers shaped like w."""
    import torch

    return (torch.empty_like(w), torch.empty(w.shape, dtype=torch.uint8, device=w.device),
            torch.empty_like(w))


def gptq_quantize(w, u, scale, zero, qmin, qmax, group=None, block=128, stream=None):
    """GPTQ's column loop on w [rows, cols] (fp32, updated in place) with U the upper Cholesky
    factor of the dampened inverse Hessian [cols, cols], grid scale/zero [rows, cols // group],
    codes in [qmin, qmax], lazy blocks of `block` columns.  Returns (q_hat, codes, err)."""
    rows, cols, group = _gptq_args(w, u, scale, zero, group)
    q_hat, codes, err = gptq_outputs(w)
    check(lib().w4_gptq_quantize(_ptr(w), _ptr(u), _ptr(scale), _ptr(zero), rows, cols, group,
                                 int(qmin), int(qmax), int(block), _ptr(q_hat), _ptr(codes),
                                 _ptr(err), _stream(stream)), "w4_gptq_quantize")
    return q_hat, codes, err


def gptq_block_update(w, u, scale, zero, qmin, qmax, col0, bcols, q_hat, codes, err, group=None,
                      stream=None):
    """One lazy block [col0, col0 + bcols) of the column loop (outputs written in place)."""
    rows, cols, group = _gptq_args(w, u, scale, zero, group)
    _need_cuda(q_hat, codes, err)
    check(lib().w4_gptq_block_update(_ptr(w), _ptr(u), _ptr(scale), _ptr(zero), rows, cols, group,
                                     int(qmin), int(qmax), int(col0), int(bcols), _ptr(q_hat),
                                     _ptr(codes), _ptr(err), _stream(stream)),
          "w4_gptq_block_update")


def gptq_lazy_update(w, u, err, col0, bcols, stream=None):
    """W[:, col0 + bcols:] -= E[:, col0:col0 + bcols] U[col0:col0 + bcols, col0 + bcols:]."""
    _need_cuda(w, u, err)
    rows, cols = w.shape
    check(lib().w4_gptq_lazy_update(_ptr(w), _ptr(u), _ptr(err), rows, cols, int(col0), int(bcols),
                                    _stream(stream)), "w4_gptq_lazy_update")


S24_TYPES = {"f16": 0, "bf16": 1}


def sparse24_compress(w, xtype="f16", stream=None):
    """fp32 [N, K] device weights -> (values int16 [N, K/2] (16-bit bits of `xtype`), codes uint8
    [N, K/8]) in the 2:4 format: the two largest magnitudes of every group of four kept."""
    import torch

    _need_cuda(w)
    if w.dtype != torch.float32 or w.dim() != 2:
        raise ValueError("w must be a 2-D float32 tensor")
    n, k = w.shape
    values = torch.empty((n, k // 2), dtype=torch.int16, device=w.device)
    meta = torch.empty((n, max(k // 8, 1)), dtype=torch.uint8, device=w.device)
    check(lib().w4_sparse24_compress(_ptr(w), n, k, S24_TYPES[xtype], _ptr(values), _ptr(meta),
                                     _stream(stream)), "w4_sparse24_compress")
    return values, meta


def sparse24_gemv(x, values, meta, y=None, stream=None):
    """y [B, N] fp32 = x [B, K] (fp16 or bf16) times the 2:4 matrix (values of x's type)."""
    import torch

    _need_cuda(x, values, meta)
    x2 = x if x.dim() == 2 else x.view(1, -1)
    xtype = {torch.float16: "f16", torch.bfloat16: "bf16"}[x2.dtype]
    b, k = x2.shape
    n = values.shape[0]
    if y is None:
        y = torch.empty((b, n), dtype=torch.float32, device=x.device)
    check(lib().w4_sparse24_gemv(_ptr(x2), _ptr(values), _ptr(meta), S24_TYPES[xtype], n, k, b,
                                 _ptr(y), _stream(stream)), "w4_sparse24_gemv")
    return y


def sparse24_gemv_grouped(x, values, meta, ys=None, stream=None):
    """Several 2:4 matrices sharing x in one launch: returns [y_g] (fp32 [B, N_g])."""
    import torch

    x2 = x if x.dim() == 2 else x.view(1, -1)
    _need_cuda(x2, *values, *meta)
    xtype = {torch.float16: "f16", torch.bfloat16: "bf16"}[x2.dtype]
    b, k = x2.shape
    ns = [v.shape[0] for v in values]
    if ys is None:
        ys = [torch.empty((b, n), dtype=torch.float32, device=x.device) for n in ns]
    g = len(values)
    arr = ctypes.c_void_p * g
    check(lib().w4_sparse24_gemv_grouped(
        _ptr(x2), g, arr(*[v.data_ptr() for v in values]), arr(*[m.data_ptr() for m in meta]),
        (ctypes.c_int64 * g)(*ns), S24_TYPES[xtype], k, b, arr(*[y.data_ptr() for y in ys]),
        _stream(stream)), "w4_sparse24_gemv_grouped")
    return ys
