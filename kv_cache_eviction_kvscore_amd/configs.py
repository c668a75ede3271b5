"""The five synthetic workloads the library is tested and measured on.

Each workload fixes the model shape (layers, query/KV heads, head dim), the ragged
prompt lengths, the observation window, the heavy-key and sink structure of the
synthetic keys, the seed, and how the per-layer budget total is set. Shapes follow
the model families the pages evaluate (Llama-3.1-8B: 32 layers, 32 query / 8 KV
heads, d = 128; Qwen2.5-7B: 28 layers, 28 query / 4 KV heads, d = 128); the data are
seeded Gaussians, not model activations (no weights or datasets are used).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seqlens: Tuple[int, ...]
    window: int
    heavy_count: Optional[Tuple[int, ...]]  # heavy keys per (seq, layer, KV head); one entry per sequence
    budget_kind: str  # "fixed" | "uniform" | "profile"
    budget_value: float  # fixed per-layer budget, or the fraction of tokens kept
    ratio: float = 1.0  # exponential multiplier ratio r for "profile"
    gamma: float = math.inf
    sink: bool = True
    heavy_scale: float = 3.0
    sink_scale: float = 4.0

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    def cu_seqlens(self) -> List[int]:
        cu = [0]
        for n in self.seqlens:
            cu.append(cu[-1] + int(n))
        return cu

    def sensitivity_profile(self) -> np.ndarray:
        """s_l = 1 + 0.5 sin(l/5) + N(0, 0.1), l = 0..L-1 (radians; std 0.1)."""
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(self.seed).spawn(1)[0]))
        ell = np.arange(self.num_layers, dtype=np.float64)
        return 1.0 + 0.5 * np.sin(ell / 5.0) + rng.normal(0.0, 0.1, self.num_layers)

    def budget_request(self, s: int):
        """(profile, ratio, gamma, total) for sequence s, as passed to the budget map."""
        n = self.seqlens[s]
        L = self.num_layers
        if self.budget_kind == "fixed":
            return np.zeros(L), 1.0, math.inf, int(self.budget_value) * L
        if self.budget_kind == "uniform":
            return np.zeros(L), 1.0, math.inf, int(math.floor(self.budget_value * n)) * L
        if self.budget_kind == "profile":
            return self.sensitivity_profile(), self.ratio, self.gamma, int(math.floor(self.budget_value * L * n))
        raise ValueError(self.budget_kind)

    def kv_bytes(self) -> int:
        """bf16 K+V bytes: 2 tensors * 2 bytes * L * Hkv * d * N (PyramidKV page's sizing formula)."""
        return 2 * 2 * self.num_layers * self.num_kv_heads * self.head_dim * self.total_tokens


def _heavy(frac: float, seqlens) -> Tuple[int, ...]:
    return tuple(int(round(frac * n)) for n in seqlens)


WORKLOADS = {
    # 1 layer, GQA 4:1, d=64, n=2048, W=32, 16 heavy keys, sink; keep recent 32 + top-128.
    1: Workload("gqa4_d64_n2k_w32", 0, 1, 4, 1, 64, (2048,), 32, (16,), "fixed", 160),
    # Llama-3.1-8B-shaped single layer, n=32768, W=64, 0.5% heavy, 5% per KV head (1638).
    2: Workload("llama8b_1layer_n32k", 1, 1, 32, 8, 128, (32768,), 64, _heavy(0.005, (32768,)), "uniform", 0.05),
    # 32 layers, n=32768, 16 heavy keys, exponential layer budgets (r=2) totalling 10%.
    3: Workload("llama8b_32layer_n32k_exp", 2, 32, 32, 8, 128, (32768,), 64, (16,), "profile", 0.10, ratio=2.0),
    # 32 layers, n=131072, 0.2% heavy, uniform 5% (6553 per layer and KV head).
    4: Workload("llama8b_32layer_n128k", 3, 32, 32, 8, 128, (131072,), 64, _heavy(0.002, (131072,)), "uniform", 0.05),
    # Qwen2.5-7B-shaped ragged batch of 4 sequences, 0.3% heavy, exponential budgets (r=3), 5% per sequence.
    5: Workload("qwen7b_28layer_ragged4", 4, 28, 28, 4, 128, (131072, 65536, 40000, 12345), 64,
                _heavy(0.003, (131072, 65536, 40000, 12345)), "profile", 0.05, ratio=3.0),
}


def small_variant(base: Workload, **kw) -> Workload:
    """A reduced copy of a workload for fast tests (same structure, smaller sizes)."""
    fields = dict(base.__dict__)
    fields.update(kw)
    return Workload(**fields)
