"""Seeded synthetic inputs for the W4A16 layer (no quantizer or matmul
arithmetic lives here; both the HIP path's tests and the oracle's draw from it).

The workloads are LLaMA-3-8B, Qwen-2.5-7B and 70B-class linear layers, whose
trained weights are not available: values are drawn from the distributions the
layers are described with, and GEMV/GEMM timing does not depend on them.

Recipe (numpy PCG64, float32 draws, in this order, then RNE to fp16):
  1. W  = 0.02 * standard_normal((N, K))
  2. outlier mask = random((N, K)) < 1e-3
  3. W[mask] = 0.5 * standard_normal(mask.sum())   (replaces, not adds)
  4. X  = standard_normal((M, K))                   (activations)
Seeds: the 4096x4096 single-layer case uses seed 0; every other matrix uses
the sequence seed [case_id, layer, matrix_id].
"""
from __future__ import annotations

import numpy as np

SIGMA_W = 0.02
OUTLIER_P = 1e-3
SIGMA_OUTLIER = 0.5

# Decoder layer shapes as (name, K = in_features, N = out_features).
LLAMA3_8B = [("q", 4096, 4096), ("k", 4096, 1024), ("v", 4096, 1024), ("o", 4096, 4096),
             ("gate", 4096, 14336), ("up", 4096, 14336), ("down", 14336, 4096)]
QWEN25_7B = [("q", 3584, 3584), ("k", 3584, 512), ("v", 3584, 512), ("o", 3584, 3584),
             ("gate", 3584, 18944), ("up", 3584, 18944), ("down", 18944, 3584)]
LLAMA3_8B_LAYERS = 32
QWEN25_7B_LAYERS = 28
FFN_70B = [("gate_up_70b", 8192, 28672)]


def weight_and_activation(n: int, k: int, m: int, seed):
    """(W fp16 [n, k], X fp16 [m, k]) drawn with the recipe above."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32)
    w *= np.float32(SIGMA_W)
    mask = rng.random((n, k), dtype=np.float32) < np.float32(OUTLIER_P)
    count = int(mask.sum())
    w[mask] = rng.standard_normal(count, dtype=np.float32) * np.float32(SIGMA_OUTLIER)
    x = rng.standard_normal((m, k), dtype=np.float32)
    return w.astype(np.float16), x.astype(np.float16)


def weight(n: int, k: int, seed):
    """W fp16 [n, k] only (same stream as weight_and_activation)."""
    return weight_and_activation(n, k, 0, seed)[0]


def activation(m: int, k: int, seed):
    """X fp16 [m, k] ~ N(0, 1) from its own stream."""
    rng = np.random.default_rng(seed)
    return rng.standard_normal((m, k), dtype=np.float32).astype(np.float16)


def matrix_seed(case_id: int, layer: int, matrix_id: int):
    return [case_id, layer, matrix_id]
