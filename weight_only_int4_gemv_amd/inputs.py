"""Seeded synthetic inputs for the W4A16 layer (no quantizer or matmul
arithmetic lives here; both the HIP path's tests and the oracle's draw from it).

The workloads are LLaMA-3-8B, Qwen-2.5-7B and 70B-class linear layers, whose
trained weights are not available: values are drawn from the distributions the
layers are described with, and GEMV/GEMM timing does not depend on them.

Recipe (numpy PCG64, float32 draws, then round-to-nearest-even to fp16):
  weights W [N, K], in blocks of 256 rows; block b uses the generator seeded
  with (seed..., b) and draws, in this order,
    1. 0.02 * standard_normal(block)
    2. outlier mask = random(block) < 1e-3
    3. the masked entries are replaced by 0.5 * standard_normal(count)
  activations X [M, K]: standard_normal((M, K)) from the generator seeded
  with the activation seed.
Blocks are independent, so they are drawn on a thread pool; the values do
not depend on the number of threads.
Seeds: the 4096 x 4096 single layer uses weight seed 0 and activation seed
(1000, 0); layer matrices use (case, layer, matrix) sequences.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SIGMA_W = 0.02
OUTLIER_P = 1e-3
SIGMA_OUTLIER = 0.5
ROW_BLOCK = 256

# Decoder layer shapes as (name, K = in_features, N = out_features).
LLAMA3_8B = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
             ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
QWEN25_7B = [("q", 3584, 3584), ("k", 3584, 512), ("v", 3584, 512), ("o", 3584, 3584),
             ("gate", 3584, 18944), ("up", 3584, 18944), ("down", 18944, 3584)]
LLAMA3_8B_LAYERS = 32
QWEN25_7B_LAYERS = 28
FFN_70B = [("gate_up_70b", 8192, 28672)]


def _seed_list(seed):
    if isinstance(seed, (int, np.integer)):
        return [int(seed)]
    return [int(s) for s in seed]


def _workers() -> int:
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n or 1))


def weight(n: int, k: int, seed) -> np.ndarray:
    """W fp16 [n, k]: N(0, 0.02) with 0.1 % of entries replaced by N(0, 0.5)."""
    out = np.empty((n, k), dtype=np.float16)
    base = _seed_list(seed)

    def block(b):
        r0, r1 = b * ROW_BLOCK, min(n, (b + 1) * ROW_BLOCK)
        rng = np.random.default_rng(base + [b])
        w = rng.standard_normal((r1 - r0, k), dtype=np.float32)
        w *= np.float32(SIGMA_W)
        mask = rng.random((r1 - r0, k), dtype=np.float32) < np.float32(OUTLIER_P)
        w[mask] = rng.standard_normal(int(mask.sum()), dtype=np.float32) * np.float32(SIGMA_OUTLIER)
        out[r0:r1] = w.astype(np.float16)

    nblocks = (n + ROW_BLOCK - 1) // ROW_BLOCK
    if nblocks <= 1:
        for b in range(nblocks):
            block(b)
    else:
        with ThreadPoolExecutor(max_workers=_workers()) as pool:
            list(pool.map(block, range(nblocks)))
    return out


def weight_skewed(n: int, k: int, seed) -> np.ndarray:
    """W fp16 [n, k] with a mean far from zero, for asymmetric INT4: the
    fp16 values of ``weight(n, k, seed)`` plus a per-row offset, uniform on
    [-0.05, 0.05] (generator seeded with (seed..., 2**20)), summed in
    float32 and rounded to fp16.  With sigma 0.02 most 128-element groups
    stay two-signed and some rows are nearly one-signed."""
    rng = np.random.default_rng(_seed_list(seed) + [2 ** 20])
    off = rng.uniform(-0.05, 0.05, size=(n, 1)).astype(np.float32)
    return (weight(n, k, seed).astype(np.float32) + off).astype(np.float16)


def activation(m: int, k: int, seed) -> np.ndarray:
    """X fp16 [m, k] ~ N(0, 1)."""
    rng = np.random.default_rng(_seed_list(seed))
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16)


def weight_and_activation(n: int, k: int, m: int, seed):
    """(W [n, k], X [m, k]) with the activation seed (1000, seed...)."""
    return weight(n, k, seed), activation(m, k, [1000] + _seed_list(seed))


def matrix_seed(case_id: int, layer: int, matrix_id: int):
    return [case_id, layer, matrix_id]
