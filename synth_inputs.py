"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds none of the W4 method's arithmetic: it only draws random numbers and rounds
activations once to their 16-bit storage type.  Both the CPU oracle and the GPU library receive
exactly the arrays made here, so neither side generates inputs for the other.

Shapes follow the pages' workloads:

* Qwen2.5-1.5B decode projections, q 1536->1536, k/v 1536->256, o 1536->1536 (LLM Quantization on
  RTX 4060, section "Why k/v Projections"), gate/up 1536->8960 and down 8960->1536, 28 layers, and
  the tied 151,936-token lm_head (My Triton Kernel Ties bitsandbytes, section "The roofline first");
  one decode step is 197 matrix multiplications (Do Quantization and Sparsity make LLM Inference
  Faster?, section "What we did").
* A larger single-GPU model with hidden 8192 and intermediate 28672 (q 8192x8192, kv 1024x8192,
  gate/up 28672x8192, down 8192x28672, lm_head 128256x8192).

Weights are fp32 ~ N(0, sigma) (sigma 0.02, or 0.015 for the larger model); activations are
N(0, 1) drawn in fp32 and rounded round-to-nearest-even to fp16 or bf16.  Every draw takes an
explicit seed; the generator is numpy's PCG64 (``numpy.random.default_rng``).
"""
from __future__ import annotations

import numpy as np

# (name, N = out_features, K = in_features) of one Qwen2.5-1.5B decoder layer.
QWEN15_LAYER = (
    ("q", 1536, 1536),
    ("k", 256, 1536),
    ("v", 256, 1536),
    ("o", 1536, 1536),
    ("gate", 8960, 1536),
    ("up", 8960, 1536),
    ("down", 1536, 8960),
)
QWEN15_LAYERS = 28
QWEN15_LM_HEAD = ("lm_head", 151936, 1536)
QWEN15_SIGMA = 0.02

# Larger single-GPU model (hidden 8192, intermediate 28672).
LARGE_SHAPES = (
    ("q", 8192, 8192),
    ("kv", 1024, 8192),
    ("gate", 28672, 8192),
    ("up", 28672, 8192),
    ("down", 8192, 28672),
    ("lm_head", 128256, 8192),
)
LARGE_SIGMA = 0.015


def decode_step_shapes(layers: int = QWEN15_LAYERS):
    """The ordered list of (name, N, K) for one decode step: 28 x 7 projections + lm_head."""
    out = []
    for layer in range(layers):
        for name, n, k in QWEN15_LAYER:
            out.append((f"L{layer}.{name}", n, k))
    out.append(QWEN15_LM_HEAD)
    return out


def weights(n: int, k: int, sigma: float = QWEN15_SIGMA, seed: int = 0) -> np.ndarray:
    """fp32 [n, k] ~ N(0, sigma), PCG64 seeded with ``seed``."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((n, k), dtype=np.float32) * np.float32(sigma)


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def to_storage_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values once, to nearest even, to fp16 or bf16; return the uint16 bit patterns."""
    if dtype == "f16":
        return np.ascontiguousarray(a, dtype=np.float32).astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return _f32_to_bf16_bits(a)
    raise ValueError(f"unknown activation dtype {dtype!r}")


def activations(b: int, k: int, dtype: str = "f16", seed: int = 7) -> np.ndarray:
    """uint16 bit patterns [b, k] of N(0, 1) fp32 draws rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    return to_storage_bits(rng.standard_normal((b, k), dtype=np.float32), dtype)


def single_gemv_case(seed: int = 0, n: int = 256, k: int = 1536, dtype: str = "f16"):
    """The single-GEMV workload: W [n, k] ~ N(0, 0.02) drawn first, then x [1, k] ~ N(0, 1),
    both from one PCG64 stream seeded with ``seed``."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(QWEN15_SIGMA)
    x = to_storage_bits(rng.standard_normal((1, k), dtype=np.float32), dtype)
    return w, x


def random_packed(fmt: str, n: int, k: int, seed: int):
    """Storage arrays of an [n, k] 4-bit matrix filled with random bits, for timing code whose cost
    does not depend on the values: packed bytes uniform over 0..255 ([n, k/2] uint8) and per-block
    scales in the format's storage type -- fp32 [n, k/64] for "nf4" and "fp4", bf16 bit patterns
    [n, k/128] for "int4", and for "int4a" uint32 words [n, k/128] holding bf16 scale bits in bits
    0-15 and a random zero point 0..15 in bits 16-19.  Scales are drawn from U(0.004, 0.006)."""
    rng = np.random.default_rng(seed)
    packed = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    if fmt in ("nf4", "fp4"):
        scales = rng.uniform(0.004, 0.006, size=(n, k // 64)).astype(np.float32)
    elif fmt == "int4":
        scales = _f32_to_bf16_bits(rng.uniform(0.004, 0.006, size=(n, k // 128)))
    elif fmt == "int4a":
        bits = _f32_to_bf16_bits(rng.uniform(0.004, 0.006, size=(n, k // 128))).astype(np.uint32)
        scales = bits | (rng.integers(0, 16, size=bits.shape, dtype=np.uint32) << np.uint32(16))
    else:
        raise ValueError(f"unknown weight format {fmt!r}")
    return packed, scales


def upper_factor(cols: int, seed: int, off_sigma: float = 0.3) -> np.ndarray:
    """A seeded random upper-triangular fp32 matrix [cols, cols]: diagonal ~ U(0.5, 1.5),
    entries above it ~ N(0, off_sigma^2 / cols), zeros below.  Any such matrix U is the upper
    Cholesky factor of the inverse of the symmetric positive definite matrix (U^T U)^-1, so it
    stands for the factor that GPTQ's column loop takes as input."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((cols, cols), dtype=np.float32) * np.float32(off_sigma / np.sqrt(cols))
    u = np.triu(u, 1)
    u[np.diag_indices(cols)] = rng.uniform(0.5, 1.5, cols).astype(np.float32)
    return u
