"""The C ABI library loads on the host, exports every function include/w4.h declares, and rejects
invalid arguments on the host before any launch.  No compute call is made (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4.h")


def _lib():
    import bit_weight_only_w4_amd as w4

    if not os.path.exists(w4.LIB_PATH):
        pytest.fail("libw4.so is not built; run `python -m bit_weight_only_w4_amd.build`")
    return w4, w4.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for required in ("w4_quantize_nf4", "w4_quantize_int4", "w4_quantize_fp4",
                     "w4_quantize_int4_asym", "w4_gemv",
                     "w4_gemm_smallbatch",
                     "w4_matmul_ex", "w4_workspace_bytes"):
        assert required in names


def test_every_declared_symbol_is_exported():
    _, L = _lib()
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing


def test_codebook_matches_oracle_bitwise():
    w4, _ = _lib()
    lib_code = np.array(w4.nf4_codebook(), dtype=np.float32)
    assert np.array_equal(lib_code.view(np.uint32), oracle.nf4_codebook().view(np.uint32))


def test_version_and_status_strings():
    w4, L = _lib()
    assert L.w4_version() == 1
    for st in range(0, -10, -1):
        assert w4.status_string(st) not in ("", "unknown status")
    assert w4.status_string(-42) == "unknown status"


FAKE = 0x10000  # a non-null, well-aligned address that is never dereferenced


def _gemv(L, x=FAKE, p=FAKE * 2, s=FAKE * 3, fmt=1, n=64, k=256, b=1, y=FAKE * 4):
    vp = ctypes.c_void_p
    return L.w4_gemv(vp(x), vp(p), vp(s), fmt, n, k, b, vp(y), None)


def test_host_validation_codes():
    _, L = _lib()
    assert _gemv(L, x=0) == -1
    assert _gemv(L, y=0) == -1
    assert _gemv(L, fmt=0) == -4
    assert _gemv(L, fmt=9) == -4  # 5, 6 are FP4, 7, 8 asymmetric INT4
    assert _gemv(L, n=0) == -2
    assert _gemv(L, k=96) == -2  # NF4 needs K % 64
    assert _gemv(L, fmt=3, k=192) == -2  # INT4 needs K % 128
    assert _gemv(L, b=0) == -2
    assert _gemv(L, b=9) == -2  # w4_gemv is the B <= 8 entry point
    assert _gemv(L, x=FAKE + 8) == -3  # x must be 16-byte aligned
    assert _gemv(L, p=FAKE + 4) == -3
    assert _gemv(L, y=FAKE + 2) == -3
    assert _gemv(L, y=FAKE * 2) == -9  # y overlaps the packed weights
    vp = ctypes.c_void_p
    # split-K without a workspace; two-pass without a workspace; unknown path
    assert L.w4_matmul_ex(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), 1, 64, 256, 1, vp(FAKE * 4), 2, 4,
                          None, 0, None) == -6
    assert L.w4_matmul_ex(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), 1, 64, 256, 1, vp(FAKE * 4), 4, 0,
                          None, 0, None) == -6
    assert L.w4_matmul_ex(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), 1, 64, 256, 1, vp(FAKE * 4), 9, 0,
                          None, 0, None) == -7
    assert L.w4_quantize_nf4(None, 4, 64, vp(FAKE), vp(FAKE * 2), None) == -1
    assert L.w4_quantize_nf4(vp(FAKE), 4, 96, vp(FAKE * 8), vp(FAKE * 9), None) == -2
    assert L.w4_quantize_int4(vp(FAKE), 4, 64, vp(FAKE * 8), vp(FAKE * 9), None) == -2
    assert L.w4_quantize_fp4(None, 4, 64, vp(FAKE), vp(FAKE * 2), None) == -1
    assert L.w4_quantize_fp4(vp(FAKE), 4, 96, vp(FAKE * 8), vp(FAKE * 9), None) == -2  # K % 64
    assert L.w4_quantize_fp4(vp(FAKE), 4, 64, vp(FAKE * 8 + 4), vp(FAKE * 9), None) == -3
    assert _gemv(L, fmt=5, k=96) == -2  # FP4 needs K % 64
    assert _gemv(L, fmt=7, k=192) == -2  # asymmetric INT4 needs K % 128
    assert _gemv(L, fmt=8, s=FAKE * 3 + 2) == -3  # its scale words are 4-byte
    assert L.w4_quantize_int4_asym(None, 4, 128, vp(FAKE), vp(FAKE * 2), None) == -1
    assert L.w4_quantize_int4_asym(vp(FAKE), 4, 64, vp(FAKE * 8), vp(FAKE * 9), None) == -2
    assert L.w4_quantize_int4_asym(vp(FAKE), 4, 128, vp(FAKE * 8), vp(FAKE * 9 + 2), None) == -3
    assert _gemv(L, fmt=6, s=FAKE * 3 + 2) == -3  # FP4 scales are fp32
    assert L.w4_probe_read(vp(FAKE), 24, vp(FAKE * 2), None) == -2


def _prefill(L, x=FAKE, p=FAKE * 2, s=FAKE * 3, fmt=1, n=64, k=256, b=512, y=FAKE * 64):
    vp = ctypes.c_void_p
    return L.w4_gemm_prefill(vp(x), vp(p), vp(s), fmt, n, k, b, vp(y), None)


def test_prefill_validation_codes():
    """w4_gemm_prefill takes 1 <= B <= W4_MAX_BATCH = 4096 and checks like w4_gemv (every case
    here fails validation, before any launch)."""
    import bit_weight_only_w4_amd as w4

    _, L = _lib()
    assert w4.MAX_BATCH == 4096
    assert _prefill(L, x=0) == -1
    assert _prefill(L, s=0) == -1
    assert _prefill(L, fmt=0) == -4
    assert _prefill(L, b=0) == -2
    assert _prefill(L, b=4097) == -2
    assert _prefill(L, k=96) == -2
    assert _prefill(L, fmt=4, k=192) == -2
    assert _prefill(L, p=FAKE + 8) == -3
    assert _prefill(L, y=FAKE + 4) == -9  # y [512, 64] floats overlaps x
    vp = ctypes.c_void_p
    # the explicit tiled path validates the same way
    assert L.w4_matmul_ex(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), 1, 64, 256, 4097, vp(FAKE * 64), 5,
                          0, None, 0, None) == -2


def test_workspace_and_plan_logic():
    w4, _ = _lib()
    assert w4.workspace_bytes("nf4_f16", 1536, 8960, 1, "splitk", 4) == 4 * 1536 * 4
    assert w4.workspace_bytes("nf4_f16", 8960, 1536, 2, "twopass") == 8960 * 1536 * 2
    assert w4.workspace_bytes("nf4_f16", 8960, 1536, 1, "gemv") == 0
    assert w4.workspace_bytes("nf4_f16", 8960, 100, 1, "gemv") == 0  # invalid K
    plan = w4.gemv_plan("nf4_f16", 8960, 1536, 1)
    assert plan["team"] * plan["iters"] >= 1536 // 32
    assert plan["chunks_per_split"] == 1536 // 32
    plan = w4.gemv_plan("int4_bf16", 1536, 8960, 1, split_k=4)
    assert plan["chunks_per_split"] * 4 >= 8960 // 32
    with pytest.raises(ValueError):
        w4.gemv_plan("nf4_f16", 64, 256, 9)
    assert w4.auto_path("nf4_f16", 8960, 1536, 1) == ("gemv", 1)
    assert w4.auto_path("nf4_f16", 8960, 1536, 3)[0] == "gemv"
    assert w4.auto_path("nf4_f16", 8960, 1536, 4)[0] == "mfma"
    assert w4.auto_path("nf4_f16", 1536, 1536, 4)[0] == "gemv"  # under 4 MiB: MFMA from B = 5
    assert w4.auto_path("nf4_f16", 1536, 1536, 5)[0] == "mfma"
    assert w4.auto_path("nf4_f16", 8960, 1536, 64)[0] == "mfma"
    assert w4.auto_path("nf4_f16", 151936, 1536, 2)[0] == "gemv"  # 116 MB: MFMA from B = 3
    assert w4.auto_path("nf4_f16", 151936, 1536, 3)[0] == "mfma"
    assert w4.auto_path("nf4_f16", 8960, 1536, w4.TILED_FROM_BATCH - 1)[0] == "mfma"
    assert w4.auto_path("nf4_f16", 8960, 1536, w4.TILED_FROM_BATCH)[0] == "tiled"
    assert w4.auto_path("int4_bf16", 151936, 1536, 4096)[0] == "tiled"
    assert w4.auto_path("nf4_f16", 1536, 8960, 512)[0] == "mfma"  # too few rows for the tiles
    assert w4.auto_path("nf4_f16", w4.TILED_FROM_ROWS, 1536, 512)[0] == "tiled"
    assert w4.workspace_bytes("nf4_f16", 8960, 1536, 512, "tiled") == 0


def test_mfma_split_rule():
    """The automatic MFMA split-K count (host logic; the CU count falls back to MI355X's 256 where
    no GPU is visible): rows of at most 3072 weights never split; longer rows take the smallest
    power of two that keeps held rows x K / S x 2 bytes within 128 KiB and gives two 16-row tiles
    per CU, at most 16, each range at least two quads; only with a large enough workspace."""
    w4, _ = _lib()
    big = 1 << 30
    assert w4.auto_path("nf4_f16", 1536, 8960, 8) == ("mfma", 1)  # no workspace: one pass
    assert w4.auto_path("nf4_f16", 1536, 8960, 8, big) == ("mfma", 8)  # 2 by x, 8 by the tiles
    assert w4.auto_path("nf4_f16", 1536, 8960, 8, 8 * 8 * 1536 * 4 - 1) == ("mfma", 1)
    assert w4.workspace_bytes("nf4_f16", 1536, 8960, 8) == 8 * 8 * 1536 * 4
    assert w4.auto_path("nf4_f16", 8192, 28672, 32, big) == ("mfma", 16)  # x: 32*28672*2/128Ki = 14
    assert w4.auto_path("nf4_f16", 8192, 8192, 8, big) == ("mfma", 1)  # exactly 128 KiB
    assert w4.auto_path("nf4_f16", 8192, 8192, 16, big) == ("mfma", 2)
    assert w4.auto_path("int4_bf16", 1024, 8192, 4, big) == ("mfma", 8)
    assert w4.auto_path("nf4_f16", 8960, 1536, 32, big) == ("mfma", 1)  # 6 quads: never
    assert w4.auto_path("nf4_f16", 1536, 3072, 8, big) == ("mfma", 1)  # 12 quads: never
    assert w4.auto_path("nf4_f16", 64, 3328, 8, big) == ("mfma", 4)  # 13 quads: >= 2 per range
    assert w4.workspace_bytes("nf4_f16", 8960, 1536, 8) == 0
    assert w4.auto_path("nf4_f16", 128256, 8192, 32, big) == ("mfma", 1)  # 1002 tiles of 128 rows
    assert w4.auto_path("nf4_f16", 28672, 8192, 32, big) == ("mfma", 4)
    assert w4.workspace_bytes("nf4_f16", 1536, 8960, 8, "mfma", 4) == 4 * 8 * 1536 * 4
    assert w4.workspace_bytes("nf4_f16", 1536, 8960, 8, "mfma", 1) == 0


def test_tiled_split_rule():
    """The automatic tiled GEMM's split-K count (host logic, 256 CUs where no GPU is visible).
    Block-scale kernel (bf16 activations, and fp16 below 256 rows): from B = 128 the smallest power
    of two S with ceil(N / 64) * ceil(B / 128) * S >= 192, at least 16 blocks of 64 weights per
    range, at most 16 ranges.  Matrices under 4096 rows take the tiled GEMM only when K splits and
    the workspace holds the partials, else the MFMA path."""
    w4, _ = _lib()
    big = 1 << 30
    assert w4.auto_path("nf4_bf16", 1536, 8960, 512) == ("mfma", 1)  # no workspace
    assert w4.auto_path("nf4_bf16", 1536, 8960, 512, big) == ("tiled", 2)  # 96 tiles
    assert w4.auto_path("nf4_bf16", 1536, 8960, 256, big) == ("tiled", 4)  # 48 tiles
    assert w4.auto_path("nf4_f16", 1536, 8960, 128, big) == ("tiled", 8)  # 140 / 16 >= 8
    assert w4.auto_path("int4_bf16", 1024, 8192, 512, big) == ("tiled", 4)
    assert w4.auto_path("int4_bf16", 1024, 8192, 128, big) == ("tiled", 8)  # 128 / 16 < 16
    assert w4.auto_path("nf4_bf16", 8192, 8192, 128, big) == ("tiled", 2)
    assert w4.auto_path("nf4_bf16", 8192, 8192, 512, big) == ("tiled", 1)  # 512 tiles
    assert w4.auto_path("nf4_f16", 8960, 1536, 128, big) == ("tiled", 1)  # 24 blocks: no split
    assert w4.auto_path("nf4_bf16", 1536, 1536, 512, big) == ("mfma", 1)
    assert w4.auto_path("nf4_f16", 1536, 8960, 64, big) == ("mfma", 16)  # below the tiled batch
    assert w4.workspace_bytes("nf4_bf16", 1536, 8960, 512) == 2 * 512 * 1536 * 4
    assert w4.workspace_bytes("nf4_f16", 1536, 8960, 128) == 8 * 128 * 1536 * 4
    assert w4.auto_path("nf4_bf16", 1536, 8960, 512, 2 * 512 * 1536 * 4 - 1) == ("mfma", 1)
    assert w4.workspace_bytes("nf4_f16", 8192, 8192, 512) == 0
    # explicit splits: ceil(K / 64 / ceil(K / 64 / S)) ranges, 4 * ranges * B * N bytes
    assert w4.workspace_bytes("nf4_f16", 1536, 8960, 512, "tiled", 8) == 8 * 512 * 1536 * 4
    assert w4.workspace_bytes("nf4_f16", 64, 192, 130, "tiled", 2) == 2 * 130 * 64 * 4  # 3 blocks
    assert w4.workspace_bytes("nf4_f16", 64, 192, 130, "tiled", 16) == 3 * 130 * 64 * 4
    assert w4.workspace_bytes("nf4_f16", 64, 192, 130, "tiled", 1) == 0


def test_tiled_split_rule_folded():
    """NF4, INT4, FP4 and asymmetric INT4 with fp16 activations (the folded-scale kernel, 128-row
    tiles, T tiles): below one tile per CU with rows of 4096+ weights, S = min(16, 512 / T) when
    that leaves 32+ blocks per range, else S = min(16, 256 / T, K / 64 / 12), at least 2 from half
    a tile per CU, when that is 2 or more; from one to two
    tiles per CU with rows of 16384+ weights, S = 2; otherwise one pass (and shorter rows keep the
    MFMA path under 4096 matrix rows).  From 256 activation rows, and from 128 with at least 32
    tiles (fewer: the block-scale kernel's rule)."""
    w4, _ = _lib()
    big = 1 << 30
    for fmt in ("nf4_f16", "int4_f16", "fp4_f16", "int4a_f16"):
        assert w4.auto_path(fmt, 1536, 8960, 512, big) == ("tiled", 5)  # 48 tiles
        assert w4.auto_path(fmt, 1536, 8960, 256, big) == ("tiled", 10)  # 24 tiles
        assert w4.auto_path(fmt, 1024, 8192, 512, big) == ("tiled", 8)  # 32 tiles
        assert w4.auto_path(fmt, 200, 8192, 512, big) == ("tiled", 10)  # 8 tiles; 128 / 12 blocks
        assert w4.auto_path(fmt, 8192, 28672, 512, big) == ("tiled", 2)  # 256 tiles, long rows
        assert w4.auto_path(fmt, 8192, 28672, 512) == ("tiled", 1)  # no workspace: one pass
        assert w4.auto_path(fmt, 8192, 8192, 512, big) == ("tiled", 1)  # 256 tiles
        assert w4.auto_path(fmt, 16384, 28672, 512, big) == ("tiled", 1)  # 512 tiles
        assert w4.auto_path(fmt, 1536, 1536, 512, big) == ("mfma", 1)  # 24 blocks: no split
        assert w4.auto_path(fmt, 1536, 2048, 512, big) == ("mfma", 1)  # 32 blocks: no split
        # from 128 rows; below 256 only with at least 32 tiles (else the block-scale rule)
        assert w4.auto_path(fmt, 8192, 8192, 128, big) == ("tiled", 4)  # 64 tiles
        assert w4.auto_path(fmt, 28672, 8192, 128, big) == ("tiled", 2)  # 224 tiles: half per CU
        assert w4.auto_path(fmt, 8192, 28672, 192, big) == ("tiled", 4)  # 128 tiles: 2 per CU
        assert w4.auto_path(fmt, 8192, 28672, 128, big) == ("tiled", 8)  # 64 tiles, 56 blocks each
        assert w4.auto_path(fmt, 8192, 8192, 192, big) == ("tiled", 4)  # 32 blocks per range
        assert w4.auto_path(fmt, 1536, 8960, 128, big) == ("tiled", 8)  # 12 tiles: block-scale rule
        assert w4.auto_path(fmt, 151936, 1536, 128, big) == ("tiled", 1)
    assert w4.workspace_bytes("nf4_f16", 1536, 8960, 512) == 5 * 512 * 1536 * 4
    assert w4.workspace_bytes("int4_f16", 1536, 8960, 256) == 10 * 256 * 1536 * 4
    assert w4.workspace_bytes("fp4_f16", 8192, 28672, 512) == 2 * 512 * 8192 * 4


def _grouped(L, n=(64, 32, 32), x=FAKE, p=None, s=None, y=None, fmt=1, k=256, b=1, groups=None,
             entry="w4_gemv_grouped"):
    vp = ctypes.c_void_p
    g = len(n)
    p = p if p is not None else [FAKE * (10 + i) for i in range(g)]
    s = s if s is not None else [FAKE * (20 + i) for i in range(g)]
    y = y if y is not None else [FAKE * (30 + i) for i in range(g)]
    return getattr(L, entry)(vp(x), g if groups is None else groups, (vp * g)(*p), (vp * g)(*s),
                             (ctypes.c_int64 * g)(*n), (vp * g)(*y), fmt, k, b, None)


def test_grouped_validation_codes():
    _, L = _lib()
    vp = ctypes.c_void_p
    assert _grouped(L, groups=0) == -2
    assert _grouped(L, n=(8,) * 5) == -2  # more members than W4_MAX_GROUP
    assert L.w4_gemv_grouped(vp(FAKE), 1, None, None, None, None, 1, 256, 1, None) == -1
    assert _grouped(L, x=0) == -1
    assert _grouped(L, y=[FAKE * 30, 0, FAKE * 32]) == -1
    assert _grouped(L, n=(64, 0, 32)) == -2
    assert _grouped(L, k=96) == -2
    assert _grouped(L, b=9) == -2
    assert _grouped(L, fmt=9) == -4
    assert _grouped(L, p=[FAKE * 10, FAKE * 11 + 4, FAKE * 12]) == -3
    # y of member 1 overlaps y of member 0 (64 rows x 4 bytes from FAKE * 30)
    assert _grouped(L, y=[FAKE * 30, FAKE * 30 + 128, FAKE * 32]) == -9
    # y of member 2 overlaps the packed weights of member 0
    assert _grouped(L, y=[FAKE * 30, FAKE * 31, FAKE * 10]) == -9
    # the sum of N must stay below 2^31 (addresses 1 TiB apart so that nothing overlaps)
    far = [1 << 40, 1 << 41, 1 << 42, 1 << 43, 1 << 44, 1 << 45]
    assert _grouped(L, n=(1 << 30, 1 << 30), k=64, p=far[0:2], s=far[2:4], y=far[4:6]) == -2


def test_grouped_smallbatch_validation_codes():
    """w4_gemm_smallbatch_grouped rejects what w4_gemv_grouped rejects, but takes B up to
    W4_MAX_BATCH = 4096 (every case here fails validation, before any launch)."""
    _, L = _lib()
    e = "w4_gemm_smallbatch_grouped"
    assert _grouped(L, groups=0, entry=e) == -2
    assert _grouped(L, n=(8,) * 5, entry=e) == -2
    assert _grouped(L, x=0, b=32, entry=e) == -1
    assert _grouped(L, n=(64, 0, 32), b=32, entry=e) == -2
    assert _grouped(L, k=96, b=32, entry=e) == -2
    assert _grouped(L, b=4097, entry=e) == -2
    assert _grouped(L, fmt=9, b=32, entry=e) == -4
    assert _grouped(L, y=[FAKE * 30, FAKE * 30 + 128, FAKE * 32], b=1, entry=e) == -9
    # with B = 32 each y_g is 32 rows: y_1 placed inside y_0
    assert _grouped(L, y=[FAKE * 30, FAKE * 30 + 64 * 4 * 8, FAKE * 32], b=32, entry=e) == -9


def test_grouped_plan_logic():
    """Host-side plan of a grouped launch: the shared per-row shape of the summed rows, and one
    range of workgroups per member along x, never more than the member's row blocks (no idle
    workgroups) and together within the single-launch cap."""
    w4, L = _lib()
    p = w4.gemv_grouped_plan("nf4_f16", [1536, 256, 256], 1536, 1)
    solo = w4.gemv_plan("nf4_f16", 2048, 1536, 1)
    assert p["grid_z"] == 1
    assert (p["threads"], p["team"], p["iters"]) == (solo["threads"], solo["team"], solo["iters"])
    rows = p["threads"] // p["team"]
    blocks = sum((n + rows - 1) // rows for n in (1536, 256, 256))
    assert p["grid_x"] == blocks  # 192 + 32 + 32 row blocks, within the cap: one workgroup each
    p2 = w4.gemv_grouped_plan("int4_bf16", [8960, 8960], 1536, 2)
    assert p2["grid_z"] == 1 and p2["grid_x"] <= 2 * 256  # within 2 workgroups per CU
    with pytest.raises(ValueError):
        w4.gemv_grouped_plan("nf4_f16", [64] * 5, 256, 1)
    with pytest.raises(ValueError):
        w4.gemv_grouped_plan("nf4_f16", [64, 0], 256, 1)
    assert L.w4_gemv_grouped_plan(1, 2, None, 256, 1, None, None, None, None, None) == -1


G_SP = 1 << 24  # spacing of the fake GPTQ buffers: large enough that none overlaps another


def _gptq(L, w=G_SP, u=G_SP * 2, s=G_SP * 3, z=G_SP * 4, rows=64, cols=256, group=128, qmin=-8,
          qmax=7, block=128, q=G_SP * 5, c=G_SP * 6, e=G_SP * 7):
    vp = ctypes.c_void_p
    return L.w4_gptq_quantize(vp(w), vp(u), vp(s), vp(z), rows, cols, group, qmin, qmax, block,
                              vp(q), vp(c), vp(e), None)


def test_gptq_validation_codes():
    """The GPTQ calls check shapes, the code range, alignment and overlaps on the host (every
    case here fails validation, before any launch)."""
    _, L = _lib()
    vp = ctypes.c_void_p
    assert _gptq(L, w=0) == -1
    assert _gptq(L, e=0) == -1
    assert _gptq(L, rows=0) == -2
    assert _gptq(L, cols=1 << 22) == -2
    assert _gptq(L, group=100) == -2          # does not divide cols
    assert _gptq(L, block=0) == -2
    assert _gptq(L, block=129) == -2
    assert _gptq(L, qmin=7, qmax=7) == -2
    assert _gptq(L, qmin=0, qmax=256) == -2   # codes are bytes
    assert _gptq(L, s=G_SP * 3 + 2) == -3
    assert _gptq(L, q=G_SP + 64) == -9        # q_hat overlaps w
    assert _gptq(L, c=G_SP * 5 + 8) == -9     # codes overlap q_hat
    assert _gptq(L, u=G_SP + 4096) == -9      # u overlaps w
    # one block: col0 + bcols within cols, 1 <= bcols <= 128
    blk = L.w4_gptq_block_update
    args = [vp(G_SP), vp(G_SP * 2), vp(G_SP * 3), vp(G_SP * 4), 64, 256, 128, -8, 7]
    outs = [vp(G_SP * 5), vp(G_SP * 6), vp(G_SP * 7), None]
    assert blk(*args, 200, 64, *outs) == -2
    assert blk(*args, 0, 0, *outs) == -2
    assert blk(*args, 0, 129, *outs) == -2
    lazy = L.w4_gptq_lazy_update
    assert lazy(vp(G_SP), vp(G_SP * 2), None, 64, 256, 0, 128, None) == -1
    assert lazy(vp(G_SP), vp(G_SP * 2), vp(G_SP * 7), 64, 256, 192, 128, None) == -2
    assert lazy(vp(G_SP), vp(G_SP + 8), vp(G_SP * 7), 64, 256, 0, 128, None) == -9


def test_sparse24_validation_codes():
    _, L = _lib()
    vp = ctypes.c_void_p
    S = 1 << 24

    def gemv(x=S, v=2 * S, m=3 * S, xt=0, n=64, k=256, b=1, y=4 * S):
        return L.w4_sparse24_gemv(vp(x), vp(v), vp(m), xt, n, k, b, vp(y), None)

    assert gemv(x=0) == -1
    assert gemv(xt=2) == -4
    assert gemv(k=48) == -2            # K % 32
    assert gemv(k=16384 + 32) == -2    # longest row 16384
    assert gemv(b=9) == -2
    assert gemv(b=0) == -2
    assert gemv(x=S + 8) == -3
    assert gemv(m=3 * S + 2) == -3
    assert gemv(y=2 * S + 64) == -9    # y overlaps the values
    comp = L.w4_sparse24_compress
    assert comp(None, 4, 64, 0, vp(2 * S), vp(3 * S), None) == -1
    assert comp(vp(S), 4, 64, 5, vp(2 * S), vp(3 * S), None) == -4
    assert comp(vp(S), 4, 40, 0, vp(2 * S), vp(3 * S), None) == -2
    assert comp(vp(S + 4), 4, 64, 0, vp(2 * S), vp(3 * S), None) == -3
    assert comp(vp(S), 4, 64, 0, vp(S + 16), vp(3 * S), None) == -9


def test_sparse24_grouped_validation_codes():
    _, L = _lib()
    S = 1 << 24
    arr = ctypes.c_void_p * 2
    vals, meta, ys = arr(2 * S, 3 * S), arr(4 * S, 5 * S), arr(6 * S, 7 * S)
    ns = (ctypes.c_int64 * 2)(64, 32)
    f = L.w4_sparse24_gemv_grouped
    vp = ctypes.c_void_p
    assert f(vp(S), 0, vals, meta, ns, 0, 256, 1, ys, None) == -2
    assert f(vp(S), 5, vals, meta, ns, 0, 256, 1, ys, None) == -2
    assert f(vp(S), 2, vals, meta, ns, 3, 256, 1, ys, None) == -4
    assert f(vp(S), 2, vals, meta, ns, 0, 250, 1, ys, None) == -2
    assert f(vp(S), 2, arr(2 * S, 0), meta, ns, 0, 256, 1, ys, None) == -1
    assert f(vp(S), 2, vals, meta, (ctypes.c_int64 * 2)(64, 0), 0, 256, 1, ys, None) == -2
    assert f(vp(S), 2, vals, meta, ns, 0, 256, 1, arr(6 * S, 6 * S + 64), None) == -9  # y overlap


def test_tiled_f16_host_checks():
    """W4_PATH_TILED_F16 runs fp16 activations with NF4, INT4, FP4 or asymmetric INT4 weights:
    bf16 activations fail with W4_ERR_PATH before any launch; unsplit it asks for no workspace;
    split over K it needs one fp32 plane per K range (W4_ERR_WORKSPACE without one, W4_ERR_PATH past
    W4_MAX_SPLIT_K), with ceil(K/64 / S) blocks per range, an even count for the formats with
    128-weight groups (fewer ranges where that rounds up)."""
    w4, L = _lib()
    vp = ctypes.c_void_p
    for fmt in (2, 4, 6, 8):
        assert L.w4_matmul_ex(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), fmt, 64, 256, 200, vp(FAKE * 64),
                              6, 0, None, 0, None) == -7
    assert L.w4_matmul_ex(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), 1, 64, 256, 200, vp(FAKE * 64), 6, 2,
                          None, 0, None) == -6
    assert L.w4_matmul_ex(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), 1, 64, 256, 200, vp(FAKE * 64), 6, 65,
                          None, 0, None) == -7
    for fmt in ("nf4_f16", "int4_f16", "fp4_f16"):
        assert w4.workspace_bytes(fmt, 8960, 1536, 512, "tiled_f16") == 0
        assert w4.workspace_bytes(fmt, 1536, 8960, 512, "tiled_f16", 5) == 5 * 512 * 1536 * 4
    # 140 blocks, S = 11: 13 blocks per range (11 ranges); INT4 rounds to 14 (10 ranges)
    assert w4.workspace_bytes("nf4_f16", 1536, 8960, 512, "tiled_f16", 11) == 11 * 512 * 1536 * 4
    assert w4.workspace_bytes("int4_f16", 1536, 8960, 512, "tiled_f16", 11) == 10 * 512 * 1536 * 4
    assert w4.workspace_bytes("int4a_f16", 1536, 8960, 512, "tiled_f16", 11) == 10 * 512 * 1536 * 4
    assert w4.workspace_bytes("nf4_bf16", 1536, 8960, 512, "tiled_f16", 4) == 0


def test_path_override_and_workspace_registration():
    """w4_set_path / w4_get_path / w4_set_workspace on the host: unknown paths are rejected, the
    override steers w4_gemv and w4_gemm_smallbatch into w4_matmul_ex's checks (a forced split-K
    or two-pass without a registered workspace fails before any launch), and registration checks
    its pointer."""
    w4, L = _lib()
    vp = ctypes.c_void_p
    try:
        assert L.w4_set_path(9) == -7
        assert L.w4_set_path(7) == -7
        assert L.w4_set_path(-1) == -7
        for path in range(7):
            assert L.w4_set_path(path) == 0
            assert L.w4_get_path() == path
        assert L.w4_set_path(2) == 0  # split-K, nothing registered on this host
        assert _gemv(L) == -6
        assert _gemv(L, x=0) == -1  # validation still comes first
        assert L.w4_gemm_smallbatch(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), 1, 64, 256, 1,
                                    vp(FAKE * 4), None) == -6
        assert L.w4_set_path(4) == 0  # two-pass, no workspace
        assert _gemv(L) == -6
        assert L.w4_set_path(6) == 0  # the folded GEMM runs fp16 activations only
        assert L.w4_gemm_smallbatch(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), 2, 64, 256, 200,
                                    vp(FAKE * 64), None) == -7
        assert L.w4_set_path(1) == 0  # the GEMV path has no launch shape for B = 9
        assert L.w4_gemm_smallbatch(vp(FAKE), vp(FAKE * 2), vp(FAKE * 3), 1, 64, 256, 9,
                                    vp(FAKE * 64), None) == -7
        w4.set_path("auto")
        assert w4.get_path() == "auto"
        assert L.w4_set_workspace(None, 16) == -1
        assert L.w4_set_workspace(vp(FAKE + 8), 64) == -3
        # a registration needs a current device: W4_ERR_HIP on a host without one
        st = L.w4_set_workspace(vp(FAKE), 64)
        assert st in (0, -8)
        assert L.w4_set_workspace(None, 0) in (0, -8)
    finally:
        L.w4_set_path(0)


@pytest.mark.parametrize("value,expect", [("mfma", "3"), ("splitk", "2"), ("5", "5"),
                                          ("bogus", "-7")])
def test_force_path_environment_read_at_load(value, expect):
    """W4_FORCE_PATH is read once when the library loads; an unknown name leaves every steered
    call failing with W4_ERR_PATH (no silent default) until w4_set_path is called."""
    import subprocess
    import sys

    code = ("import ctypes, bit_weight_only_w4_amd as w4; L = w4.lib(); vp = ctypes.c_void_p; "
            "print(L.w4_get_path()); "
            "print(L.w4_gemv(vp(0x10000), vp(0x20000), vp(0x30000), 1, 64, 256, 1, vp(0x40000), None)); "
            "L.w4_set_path(0); print(L.w4_get_path())")
    env = dict(os.environ, W4_FORCE_PATH=value)
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    got, gemv_status, after = out.stdout.split()
    assert got == expect
    if value == "bogus":
        assert gemv_status == "-7"
    assert after == "0"


def test_workspace_must_not_overlap_inputs():
    """A workspace that a path writes into may not overlap x, the packed weights or the scales."""
    _, L = _lib()
    vp = ctypes.c_void_p
    x, p, s, y = FAKE, FAKE * 2, FAKE * 3, FAKE * 4  # n = 64, k = 256, b = 1: scales 1 KiB
    splitk = 4 * 64 * 4
    for ws in (x, p + 4096, s + 512):
        assert L.w4_matmul_ex(vp(x), vp(p), vp(s), 1, 64, 256, 1, vp(y), 2, 4, vp(ws), splitk,
                              None) == -9
    twopass = 64 * 256 * 2
    for ws in (s - twopass + 16, x - twopass + 16):
        assert L.w4_matmul_ex(vp(x), vp(p), vp(s), 1, 64, 256, 1, vp(y), 4, 0, vp(ws), twopass,
                              None) == -9
