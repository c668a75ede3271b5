"""Brute-force single-token removal (fp64, NumPy) -- an independent check of the oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

DropKV page, "Methodology in Plain English": removing one token does not merely
subtract its value vector; the softmax renormalises over the surviving tokens.
This module does exactly that, by recomputation: for every visible key j of a
query row it deletes j, recomputes the softmax over the survivors and the new
output a^(-j), and measures ||a - a^(-j)||_2. It never uses the closed form
p_j/(1-p_j)*||a - v_j||, so agreement with ``oracle.scores`` pins that formula.
O(t^2 d) per row: tiny inputs only.
"""
from __future__ import annotations

import numpy as np


def _softmax_out(logits, vals):
    m = logits.max()
    e = np.exp(logits - m)
    p = e / e.sum()
    return p @ vals


def removal_shifts(q_row, keys, vals, scale):
    """||a - a^(-j)||_2 for every visible key j of one query row (keys = visible keys)."""
    logits = (keys @ q_row) * scale
    a = _softmax_out(logits, vals)
    t = keys.shape[0]
    out = np.zeros(t)
    for j in range(t):
        keep = np.ones(t, dtype=bool)
        keep[j] = False
        a_minus = _softmax_out(logits[keep], vals[keep])
        out[j] = np.linalg.norm(a - a_minus)
    return out


def unit_scores(q_rows, keys, vals, window, scale, mode=0):
    """Score of every token of one (sequence, layer, KV head) unit by brute force.

    q_rows: [G*W][d] fp64 (head-major, then window row); keys, vals: [n][d] fp64.
    Row r = (head, i) sits at position n - W + i and sees keys 0..n-W+i.
    mode 0 sums the shifts, mode 1 sums their squares.
    """
    n = keys.shape[0]
    score = np.zeros(n)
    for r in range(q_rows.shape[0]):
        i = r % window
        t = n - window + i
        sh = removal_shifts(q_rows[r], keys[: t + 1], vals[: t + 1], scale)
        score[: t + 1] += sh * sh if mode == 1 else sh
    return score
