"""The whole hot path on one stream: attention forward -> score -> merge -> top-k -> compact.

torch provides device memory and the stream; every step is a libkvscore call. Buffers
are allocated once per (problem, budgets) so repeated runs allocate nothing.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import api


def layer_budgets(w, s: int, n_sink: int = 0) -> np.ndarray:
    """Per-layer budgets of sequence s of a workload (host map of the library); every
    layer keeps at least the window and the sinks."""
    prof, ratio, gamma, total = w.budget_request(s)
    lo = w.window + min(n_sink, w.seqlens[s] - w.window)
    return api.budget(prof, ratio, gamma, total, lo, w.seqlens[s])


def workload_budgets(w, n_sink: int = 0) -> np.ndarray:
    return np.stack([layer_budgets(w, s, n_sink) for s in range(w.num_seqs)]).astype(np.int32)


class Pipeline:
    """Owns the outputs and workspaces of one problem and runs the hot path."""

    def __init__(self, prob: api.Problem, budgets: np.ndarray, device="cuda", *, pool: int = 1, n_sink: int = 0,
                 heads: bool = False):
        self.p = prob
        self.pool, self.n_sink, self.heads = pool, n_sink, heads
        self.budgets = np.ascontiguousarray(np.asarray(budgets, dtype=np.int32))
        dev = torch.device(device)
        d, rows = prob.head_dim, prob.rows
        L, Hkv, N = prob.num_layers, prob.num_kv_heads, prob.total_tokens
        self.tq = prob.num_query_tiles()
        self.a = torch.empty((rows, d), dtype=torch.float32, device=dev)
        self.lse = torch.empty(rows, dtype=torch.float32, device=dev)
        self.jstar = torch.empty(rows, dtype=torch.int32, device=dev)
        self.dom = torch.empty(rows, dtype=torch.float32, device=dev)
        self.partial = torch.empty((L, Hkv, self.tq, N), dtype=torch.float32, device=dev)
        # one query tile: the partial row is the score row, and the merge adds the isolated
        # terms in place
        self.score = (self.partial.view(L, Hkv, N) if self.tq == 1
                      else torch.empty((L, Hkv, N), dtype=torch.float32, device=dev))
        self.ws_fwd = torch.empty(max(1, prob.workspace_size(api.WS_ATTN_FWD)), dtype=torch.uint8, device=dev)
        self.ws_score = torch.empty(max(1, prob.workspace_size(api.WS_SCORE)), dtype=torch.uint8, device=dev)
        self.ws_topk = (torch.empty(prob.workspace_size(api.WS_TOPK), dtype=torch.uint8, device=dev)
                        if pool > 1 else None)
        self.seg_off_host = api.segment_offsets(prob, self.budgets)
        self.seg_off = torch.from_numpy(self.seg_off_host).to(dev)
        R = int(self.seg_off_host[-1])
        self.kept = torch.empty(max(R, 1), dtype=torch.int32, device=dev)
        self.k_out = torch.empty((max(R, 1), d), dtype=torch.bfloat16, device=dev)
        self.v_out = torch.empty((max(R, 1), d), dtype=torch.bfloat16, device=dev)
        self.kept_rows = R
        # head budgets chosen jointly per layer: the heads' offsets come from the selection
        self.head_off = torch.empty(prob.units + 1, dtype=torch.int64, device=dev) if heads else None
        if heads:  # the joint select's scratch, then (pool > 1) the pooled keys
            nb = prob.workspace_size(api.WS_TOPK_HEADS) - (0 if pool > 1 else prob.workspace_size(api.WS_TOPK))
            self.ws_topk = torch.empty(nb, dtype=torch.uint8, device=dev)

    def attn(self, q, k, v, stream=None):
        api.attn_fwd(self.p, q, k, v, self.a, self.lse, self.jstar, self.dom, self.ws_fwd, stream)

    def scores(self, q, k, v, stream=None):
        api.score(self.p, q, k, v, self.a, self.lse, self.jstar, self.partial, self.ws_score, stream)
        api.merge(self.p, self.partial, self.jstar, self.dom, self.score, stream)

    def select(self, k, v, stream=None):
        if self.heads:
            api.topk_heads(self.p, self.score, self.budgets, self.seg_off, self.head_off, self.kept, stream,
                           pool=self.pool, n_sink=self.n_sink, ws=self.ws_topk)
            api.compact_heads(self.p, k, v, self.budgets, self.head_off, self.kept, self.k_out, self.v_out, stream)
            return
        api.topk(self.p, self.score, self.budgets, self.seg_off, self.kept, stream, pool=self.pool,
                 n_sink=self.n_sink, ws=self.ws_topk)
        api.compact(self.p, k, v, self.budgets, self.seg_off, self.kept, self.k_out, self.v_out, stream)

    def run(self, q, k, v, stream=None):
        self.attn(q, k, v, stream)
        self.scores(q, k, v, stream)
        self.select(k, v, stream)

    def outputs(self) -> Dict[str, torch.Tensor]:
        R = self.kept_rows
        return {"a": self.a, "lse": self.lse, "jstar": self.jstar, "dom": self.dom, "partial": self.partial,
                "score": self.score, "kept": self.kept[:R], "k_out": self.k_out[:R], "v_out": self.v_out[:R],
                "seg_off": self.head_off.cpu().numpy() if self.heads else self.seg_off_host}


def problem_for(w, k: torch.Tensor, v: torch.Tensor, mode: int = api.MODE_L2) -> api.Problem:
    return api.Problem.for_tensors(k, v, num_q_heads=w.num_q_heads, window=w.window, cu_seqlens=w.cu_seqlens(),
                                   mode=mode)
