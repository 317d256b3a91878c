"""Plain, slow CPU oracle for the fused W4 dequantize-and-multiply GEMV.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or call anything in this package.  The product library never
imports it, and this package never imports the product library: the two share no code.

What it computes (all in numpy fp64 unless a storage format fixes the precision):

* ``nf4_codebook``   -- the 16 NormalFloat code points.  The pages fix only that there are 16
  unevenly spaced codes for normally distributed weights, stored fp32 (LLM Quantization on RTX 4060,
  sections "Standard Expectation from Quantization" and "Kernel Implementation"); the values come
  from the standard NormalFloat construction, written out in ``nf4.py``.
* ``quantize_nf4``   -- blockwise absmax NF4, block 64 along K, one fp32 absmax per block, two
  nibbles per byte with element 2i in the high nibble (same page, same sections).
* ``quantize_int4``  -- symmetric INT4 with a +8 zero point (My Triton Kernel Ties bitsandbytes,
  section "The kernels", first bug), one bf16 scale per 128-column group, round half to even
  (LLM Compressor 0.14, section "Details worth knowing").
* ``quantize_int4_asym`` -- asymmetric INT4: unsigned codes 0..15 with a zero point per group,
  one bf16 scale per 128-column group, code = rint(clamp(w / s + z, 0, 15)) (LLM Compressor
  0.14, sections "The fused kernel" and "What those numbers leave out").
* ``quantize_fp4``   -- FP4 (E2M1) codes through a 16-entry table, block 64, fp32 scale
  absmax / 6, the pages' threshold rounding with exact ties on even codes (LLM Compressor 0.14,
  section "Details worth knowing"; the FP4-named fused kernel of My Triton Kernel Ties
  bitsandbytes, section "The kernels").
* ``gptq``           -- GPTQ's column loop with lazy blocks (module ``oracle.gptq``): dampening, the
  upper Cholesky factor of H^-1, per-column quantize with error feedback, the lazy update (LLM
  Compressor 0.14, sections "The problem GPTQ solves" to "The fused kernel"), in fp64 for the
  algorithm's checks or fp32 with a fixed order of operations for parity with the GPU kernels.
* ``sparse24``       -- 2:4 structured sparsity (module ``oracle.sparse24``): two kept 16-bit
  values per group of four, position codes two per byte, and the dense matrix they stand for (Do
  Quantization and Sparsity make LLM Inference Faster?, "Library 2:4 sparsity" and "Custom CUDA
  2:4 GEMV").
* ``dequant_*``      -- the decoded weights, exact in fp64.
* ``gemv_reference`` -- y = x . W_hat^T and T = |x| . |W_hat|^T in fp64: the fused kernel only moves
  where dequantization happens (LLM Quantization on RTX 4060, section "Kernel Implementation"), so
  its result is this plain definition.
* ``accept``         -- the per-element bound |y - y_ref| <= 2e-3 T + 1e-5.

Pins: every function is checked against facts fixed by the pages or by mathematics in the
``-m "not gpu"`` tests (``tests/test_oracle_*.py``).  No function here is "parity unpinned".
"""
from .bits import bf16_bits_to_f64, f16_bits_to_f64, f32_to_bf16_rne_bits, x_bits_to_f64
from .nf4 import NF4_BLOCK, dequant_nf4, nf4_codebook, nf4_midpoints, quantize_nf4
from .int4 import INT4_GROUP, dequant_int4, quantize_int4
from .int4_asym import INT4A_GROUP, dequant_int4_asym, int4_asym_scale_zero, quantize_int4_asym
from .fp4 import FP4_BLOCK, FP4_GRID, dequant_fp4, fp4_codebook, fp4_magnitude_index, quantize_fp4
from .gemv import accept, dequant, gemv_reference, unpack_nibbles, violation_ratio

__all__ = [
    "NF4_BLOCK", "INT4_GROUP",
    "nf4_codebook", "nf4_midpoints", "quantize_nf4", "dequant_nf4",
    "quantize_int4", "dequant_int4",
    "INT4A_GROUP", "int4_asym_scale_zero", "quantize_int4_asym", "dequant_int4_asym",
    "FP4_BLOCK", "FP4_GRID", "fp4_codebook", "fp4_magnitude_index", "quantize_fp4", "dequant_fp4",
    "unpack_nibbles", "dequant", "gemv_reference", "accept", "violation_ratio",
    "f16_bits_to_f64", "bf16_bits_to_f64", "x_bits_to_f64", "f32_to_bf16_rne_bits",
]
