"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers: it holds none of CommVQ's arithmetic.
Workload shapes follow LLaMA-3.1-8B's attention layer (32 query heads, 8 KV
heads, head_dim 128) at the context lengths of the decode workloads; the
distributions are stated per function. Every array is produced on the host
from NumPy's PCG64 so the same bytes reach the oracle and the GPU.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def codebook(seed: int, n_kv_heads: int, head_dim: int, group_size: int, n_entries: int,
             n_rounds: int) -> np.ndarray:
    """Codebook [Hkv, D/g, R, Nc, g] fp16: every (x, y) pair drawn N(0, 1) once in
    float64 and rounded to fp16 once."""
    G = head_dim // group_size
    a = rng(seed).standard_normal((n_kv_heads, G, n_rounds, n_entries, group_size))
    return a.astype(np.float16)


def kv(seed: int, n_tokens: int, n_kv_heads: int, head_dim: int, heavy_tail: bool = False,
       batch: int | None = None) -> np.ndarray:
    """Keys or values, fp16 [N, Hkv, D] (or [B, N, Hkv, D] when batch is given):
    N(0, 1) times a per-(head, channel) scale s with ln s ~ N(0, 0.5^2), fixed over
    tokens. heavy_tail multiplies round(1% of Hkv*D) channels, picked by a seeded
    permutation, by 8."""
    g = rng(seed)
    scale = np.exp(0.5 * g.standard_normal((n_kv_heads, head_dim)))
    if heavy_tail:
        n_heavy = int(round(0.01 * n_kv_heads * head_dim))
        pick = g.permutation(n_kv_heads * head_dim)[:n_heavy]
        flat = scale.reshape(-1)
        flat[pick] *= 8.0
        scale = flat.reshape(n_kv_heads, head_dim)
    shape = (n_tokens, n_kv_heads, head_dim) if batch is None else (batch, n_tokens, n_kv_heads, head_dim)
    x = g.standard_normal(shape, dtype=np.float32) * scale.astype(np.float32)
    return x.astype(np.float16)


def queries(seed: int, batch: int, n_q_heads: int, head_dim: int) -> np.ndarray:
    """Queries fp32 [B, Hq, D] drawn N(0, 1)."""
    return rng(seed).standard_normal((batch, n_q_heads, head_dim), dtype=np.float32)


def ragged_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths drawn uniformly from the integers [lo, hi]."""
    return rng(seed).integers(lo, hi + 1, size=batch).astype(np.int32)


def random_codes(seed: int, shape, n_entries: int) -> np.ndarray:
    """Uniform code indices in [0, Nc) (used to build caches without encoding)."""
    return rng(seed).integers(0, n_entries, size=shape).astype(np.int64)


@dataclass(frozen=True)
class Workload:
    """One decode workload: shapes, quantiser and seeds."""
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    context: int  # cache capacity Lmax
    group_size: int
    n_entries: int
    n_rounds: int
    theta_base: float = 500000.0
    steps: int = 1
    ragged: tuple | None = None  # (lo, hi) for per-sequence lengths
    heavy_tail: bool = False
    seed: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "tiny_gqa4_ctx2k_2bit": Workload(
        "tiny_gqa4_ctx2k_2bit", batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128, context=2048,
        group_size=8, n_entries=256, n_rounds=2, seed=1000,
        notes="B1, 4q/1kv, D128, L2048, 2-bit (g8, Nc256, R2): encode all, one decode step"),
    "llama8b_ctx32k_2bit": Workload(
        "llama8b_ctx32k_2bit", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, context=32768,
        group_size=8, n_entries=256, n_rounds=2, seed=2000,
        notes="LLaMA-3.1-8B layer shape, B1, L32768, 2-bit"),
    "llama8b_ctx128k_1bit_64steps": Workload(
        "llama8b_ctx128k_1bit_64steps", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128,
        context=131072, group_size=8, n_entries=256, n_rounds=1, steps=64, seed=3000,
        notes="LLaMA-3.1-8B layer shape, B1, 1-bit, prefill 131008 then 64 append+decode steps"),
    "llama8b_b16_ctx32k_ragged_2bit": Workload(
        "llama8b_b16_ctx32k_ragged_2bit", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128,
        context=32768, group_size=8, n_entries=256, n_rounds=2, ragged=(16384, 32768), seed=4000,
        notes="B16 ragged lengths U{16384..32768}, masked"),
    "llama8b_encode128k_b4_2bit": Workload(
        "llama8b_encode128k_b4_2bit", batch=4, n_q_heads=32, n_kv_heads=8, head_dim=128,
        context=131072, group_size=8, n_entries=256, n_rounds=2, heavy_tail=True, seed=5000,
        notes="encode 131072 x 8 heads (1% channels x8), then batch-4 decode at full context"),
    "llama8b_ctx32k_paper_1bit": Workload(
        "llama8b_ctx32k_paper_1bit", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, context=32768,
        group_size=64, n_entries=64, n_rounds=11, seed=6000,
        notes="the paper's 1-bit quantizer (g 64, Nc' 64, R 11: 1.03 bits per scalar), B1, L32768"),
    "llama8b_ctx32k_paper_2bit": Workload(
        "llama8b_ctx32k_paper_2bit", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, context=32768,
        group_size=64, n_entries=64, n_rounds=21, seed=6100,
        notes="the paper's 2-bit quantizer (g 64, Nc' 64, R 21: 1.97 bits per scalar), B1, L32768"),
}
