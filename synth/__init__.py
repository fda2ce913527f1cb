"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and casts them to bf16 bit patterns; it holds
none of the quantization or GEMM arithmetic. Every tensor is drawn in float32
with ``numpy.random.default_rng`` (PCG64) and rounded to bf16 with
round-to-nearest-even, so the CPU oracle and the GPU path consume the same
bytes. Shapes and value distributions follow the workloads the pages measure
(single GEMMs, decode-shaped and prefill-shaped linear layers, square sweeps,
a 24-layer forward); no dataset or trained weight is involved.
"""
from __future__ import annotations

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def rng(seed: int, index: int = 0) -> np.random.Generator:
    """Generator for tensor number ``index`` of a workload seeded with ``seed``."""
    return np.random.default_rng(np.random.SeedSequence([seed, index]))


def normal(shape, std: float, seed: int, index: int = 0) -> np.ndarray:
    g = rng(seed, index)
    return bf16_bits(g.standard_normal(shape, dtype=np.float32) * np.float32(std))


def student_t(shape, nu: float, mult: float, seed: int, index: int = 0,
              plant: float | None = None, n_plant: int = 0) -> np.ndarray:
    """t(nu) * mult, with ``n_plant`` entries set to +-plant at seeded positions."""
    g = rng(seed, index)
    x = (g.standard_t(nu, size=shape) * mult).astype(np.float32)
    if plant is not None and n_plant > 0:
        flat = x.reshape(-1)
        pos = g.choice(flat.size, size=n_plant, replace=False)
        sign = np.where(g.random(n_plant) < 0.5, -1.0, 1.0).astype(np.float32)
        flat[pos] = sign * np.float32(plant)
    return bf16_bits(x)


def single_gemm_inputs(seed: int = 0):
    """A[16,256] ~ N(0,1) with 1% of entries x100, W[256,256] ~ N(0, 0.02).

    One generator seeded with ``seed`` draws A, the outlier mask, then W."""
    g = np.random.default_rng(seed)
    a = g.standard_normal((16, 256), dtype=np.float32)
    mask = g.random((16, 256)) < 0.01
    a[mask] *= np.float32(100.0)
    w = g.standard_normal((256, 256), dtype=np.float32) * np.float32(0.02)
    return bf16_bits(a), bf16_bits(w)


DECODE_SHAPES = [(5120, 5120), (5120, 17408), (17408, 5120)]   # (K, N)
DECODE_M = [1, 8, 32]


def decode_inputs(m: int, k: int, n: int, seed: int = 0):
    """Decode-shaped linear: A[m,k] ~ N(0,1), W[n,k] ~ N(0,0.02)."""
    return normal((m, k), 1.0, seed, 2 * k + 1), normal((n, k), 0.02, seed, 2 * n + 2)


PREFILL_LAYERS = {   # name: (K, N) of a Llama-style 3B block, M = 4096 tokens
    "q": (3072, 3072), "k": (3072, 1024), "v": (3072, 1024), "o": (3072, 3072),
    "gate": (3072, 8192), "up": (3072, 8192), "down": (8192, 3072),
}
PREFILL_M = 4096
PREFILL_PLANT = 3616.0   # the block maximum the pages' activation probe reports


def prefill_inputs(name: str, seed: int = 0, m: int = PREFILL_M):
    """Activations t(3) * 4 with eight planted +-3616 entries; W ~ N(0, 0.02)."""
    k, n = PREFILL_LAYERS[name]
    idx = list(PREFILL_LAYERS).index(name)
    a = student_t((m, k), 3.0, 4.0, seed, 100 + idx, plant=PREFILL_PLANT, n_plant=8)
    w = normal((n, k), 0.02, seed, 200 + idx)
    return a, w


SQUARE_SIZES = [4096, 8192, 16384]


def square_inputs(size: int, seed: int = 0):
    return normal((size, size), 1.0, seed, 300 + size), normal((size, size), 1.0, seed, 301 + size)


# 24-layer forward: per layer Q, K, V, O, then four (up, down) pairs.
FORWARD_LAYER = [("q", 2880, 4096), ("k", 2880, 512), ("v", 2880, 512), ("o", 4096, 2880)] + \
    [(f"{p}{i}", k, n) for i in range(4) for (p, k, n) in (("up", 2880, 5760), ("down", 5760, 2880))]
FORWARD_LAYERS = 24
FORWARD_M = [1, 8, 32, 128]


def forward_weight(layer: int, j: int, seed: int = 0):
    _, k, n = FORWARD_LAYER[j]
    return normal((n, k), 0.02, seed, 10_000 + 100 * layer + j)


def forward_act(layer: int, j: int, m: int, seed: int = 0):
    _, k, _ = FORWARD_LAYER[j]
    return normal((m, k), 1.0, seed, 20_000 + 100 * layer + j)
