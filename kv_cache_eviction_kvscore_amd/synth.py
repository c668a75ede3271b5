"""Seeded synthetic inputs (the only module shared by the library's tests and the oracle).

This module holds none of the method's arithmetic. It draws post-RoPE-like window
queries and full-cache keys/values with the structure the pages describe for real
prefill: Gaussian entries, a few "heavy-hitter" keys scaled up, and an attention
sink at token 0 (PyramidKV page: attention concentrates on the first tokens), and
rounds them once to bf16 (round-to-nearest-even).

Layouts produced:
  q : [L][S][Hq][W][d] bf16   (the last W positions of each sequence)
  k : [L][Hkv][N][d]   bf16   (N = sum of sequence lengths, sequences concatenated)
  v : [L][Hkv][N][d]   bf16

Randomness: every (sequence, layer, tensor, head) block draws from its own torch
generator seeded from ``numpy.random.SeedSequence(seed, spawn_key=...)``, so a block
does not depend on generation order. The same seed gives the same bits on the same
device type; CPU and GPU streams differ, so a parity test generates once and hands
the same tensors to both the library and the oracle.
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np
import torch

from .configs import Workload

_Q, _K, _V, _HEAVY = 1, 2, 3, 4


def _gen(device, seed: int, *key: int) -> torch.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=tuple(int(x) for x in key))
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & 0x7FFFFFFFFFFFFFFF))
    return g


def generate(w: Workload, device="cpu") -> Dict[str, torch.Tensor]:
    """Build q, k, v (bf16) for workload ``w`` on ``device``."""
    L, S, Hq, Hkv, d, W = w.num_layers, w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.window
    G = Hq // Hkv
    cu = w.cu_seqlens()
    N = cu[-1]
    dev = torch.device(device)
    q = torch.empty((L, S, Hq, W, d), dtype=torch.bfloat16, device=dev)
    k = torch.empty((L, Hkv, N, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty((L, Hkv, N, d), dtype=torch.bfloat16, device=dev)
    for s in range(S):
        n = w.seqlens[s]
        lo, hi = cu[s], cu[s + 1]
        for l in range(L):
            qf = torch.randn((Hq, W, d), generator=_gen(dev, w.seed, s, l, _Q), device=dev, dtype=torch.float32)
            q[l, s] = qf.to(torch.bfloat16)
            qb = q[l, s].float()
            for g in range(Hkv):
                kf = torch.randn((n, d), generator=_gen(dev, w.seed, s, l, _K, g), device=dev, dtype=torch.float32)
                vf = torch.randn((n, d), generator=_gen(dev, w.seed, s, l, _V, g), device=dev, dtype=torch.float32)
                if w.heavy_count is not None and w.heavy_count[s] > 0 and n - W > 1:
                    cnt = min(w.heavy_count[s], n - W - 1)
                    perm = torch.randperm(n - W - 1, generator=_gen(dev, w.seed, s, l, _HEAVY, g), device=dev)
                    pos = perm[:cnt] + 1  # heavy keys never at the sink position 0 or in the window
                    kf[pos] *= w.heavy_scale
                if w.sink:
                    mean_q = qb[g * G:(g + 1) * G].reshape(-1, d).mean(dim=0)
                    kf[0] = w.sink_scale * math.sqrt(d) * mean_q / mean_q.norm()
                k[l, g, lo:hi] = kf.to(torch.bfloat16)
                v[l, g, lo:hi] = vf.to(torch.bfloat16)
    return {"q": q, "k": k, "v": v}


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a bf16 tensor's bits."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
