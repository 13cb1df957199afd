"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no quantizing, packing, dequantizing or dot products), so
the CPU oracle and the HIP library can both be fed from it without sharing any
code with each other.

Distributions follow the workloads the library is measured on: weights are
fp32 ~ N(0, 0.02) (standard deviation 0.02), activations are fp16 ~ N(0, 1)
(drawn in fp64 and rounded to binary16 by numpy), MoE experts are picked by a
seeded uniform draw without replacement.  Every stream is keyed by
(seed, purpose, shape) so a shape's inputs do not depend on what else ran.

Shapes follow the real model tables the pages benchmark: the Llama-3-8B
projection matrices [sm8x-bench, Q4_0 table], the Qwen expert / attention / MLP
tables [volta-kernel-bakeoff, "What's in the race" and "Results"].
"""
from __future__ import annotations

import numpy as np

# purpose tags: one independent stream per kind of input
_W, _X, _IDX, _POOL, _STRESS, _X32 = 0, 1, 2, 3, 4, 5


def _rng(seed: int, tag: int, *dims: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(tag), *[int(d) for d in dims]])


def weights(N: int, K: int, seed: int = 0) -> np.ndarray:
    """fp32 [N][K] row-major weights ~ N(0, 0.02)."""
    g = _rng(seed, _W, N, K)
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(0.02)
    return w


def activations(M: int, K: int, seed: int = 0) -> np.ndarray:
    """fp16 [M][K] activations ~ N(0, 1), rounded from fp64 to binary16 (RNE)."""
    g = _rng(seed, _X, M, K)
    return g.standard_normal((M, K)).astype(np.float16)


def activations32(M: int, K: int, seed: int = 0) -> np.ndarray:
    """fp32 [M][K] activations ~ N(0, 1), not rounded to binary16 (the input of
    the fp32-activation entry points, which round them themselves)."""
    g = _rng(seed, _X32, M, K)
    return g.standard_normal((M, K)).astype(np.float32)


def expert_pool(P: int, N: int, K: int, seed: int = 0) -> np.ndarray:
    """fp32 [P][N][K]: P distinct experts, each ~ N(0, 0.02)."""
    g = _rng(seed, _POOL, P, N, K)
    w = g.standard_normal((P, N, K), dtype=np.float32)
    w *= np.float32(0.02)
    return w


def expert_indices(P: int, E: int, seed: int = 0, call: int = 0) -> np.ndarray:
    """int32 [E]: E distinct experts drawn uniformly from a pool of P."""
    g = _rng(seed, _IDX, P, E, call)
    return g.choice(P, size=E, replace=False).astype(np.int32)


def stress_activations(M: int, K: int, seed: int = 0, kind: str = "large") -> np.ndarray:
    """fp16 activations with planted extremes.

    "large": about 1 in 16 entries replaced by +-U(20000, 60000) (values such as
    real down-projection inputs reach) [volta-kernel-bakeoff, "Results", the
    few-tokens bullet on precision].  "tiny": every entry scaled into the
    binary16 subnormal / small-normal range.
    """
    g = _rng(seed, _STRESS, M, K, 0 if kind == "large" else 1)
    x = g.standard_normal((M, K))
    if kind == "large":
        mask = g.random((M, K)) < (1.0 / 16.0)
        big = g.uniform(20000.0, 60000.0, size=(M, K)) * np.where(g.random((M, K)) < 0.5, -1.0, 1.0)
        x = np.where(mask, big, x)
    elif kind == "tiny":
        x = x * 2.0**-16
    else:
        raise ValueError(kind)
    return x.astype(np.float16)


# Model table shapes (N out x K in).
LLAMA3_8B_SHAPES = [
    (4096, 4096),     # o_proj
    (6144, 4096),     # fused qkv
    (14336, 4096),    # up_proj
    (4096, 14336),    # down_proj
    (28672, 4096),    # fused gate_up
    (128256, 4096),   # lm_head
]
SMALL_BATCH_SHAPES = [(6144, 2048), (2048, 6144), (8192, 2048)]
MOE_CONFIGS = [  # (pool P, experts per call E, N, K)
    (128, 10, 640, 2560),
    (256, 8, 512, 2048),
]
PREFILL_SHAPES = [(12288, 2560), (2560, 6144), (6144, 2048)]
PREFILL_TOKENS = [64, 512]
# fp32 activations in: one token on Llama-3-8B tables, up to 4 tokens on
# expert-sized ones [volta-kernel-bakeoff, "Results", the like-for-like bullets]
F32IN_CASES = [(4096, 4096, 1), (14336, 4096, 1), (640, 2560, 1), (640, 2560, 4), (6144, 2048, 4)]
# gate + up (N rows each, stacked) + SwiGLU: Qwen3-1.7B's MLP (6144 x 2048)
# [volta-kernel-bakeoff, "Results"], Llama-3-8B's (14336 x 4096) and an
# expert's gate / up (640 x 2560)
SWIGLU_SHAPES = [(6144, 2048), (14336, 4096), (640, 2560)]
SWIGLU_TOKENS = [1, 2, 4, 8]
