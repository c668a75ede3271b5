"""Brute-force study on the GPU path's own selection: F(J_hat_gpu) / F(J*).

DropKV page, limitations paragraph: on small candidate subsets the decoupled selection's
objective F(J_hat) is compared with the exact optimum F(J*) found by enumeration. Here J_hat
is what the HIP pipeline (forward, score, merge, top-k) evicts on tiny synthetic units:
n = W + m tokens, budget W + m - k, so exactly k of the m candidates go. The oracle
enumerates every k-subset for J*. Asserted: the GPU's evicted set is the oracle's decoupled
choice (tokens may differ only inside the parity band around the k-th score) and never
beats the optimum; the ratio distribution is printed.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_eviction_kvscore_amd.configs import Workload
from parity import BAND_RTOL, run_gpu, say

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f64(bits):
    return (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("W,m,kev,d", [(8, 12, 4, 64), (4, 10, 3, 128)])
def test_gpu_selection_against_brute_force_optimum(W, m, kev, d):
    L, S, Hkv = 4, 3, 2
    n = W + m
    w = Workload(f"study_w{W}_m{m}", 40 + W, L, Hkv, Hkv, d, (n,) * S, W, None, "fixed", W + m - kev, sink=False)
    say(f"study {w.name}: {L * S * Hkv} units, C({m},{kev}) subsets each")
    run = run_gpu(w)
    q, k, v = _bits(run["q"]), _bits(run["k"]), _bits(run["v"])
    kept, off = run["out"]["kept"].cpu().numpy(), run["out"]["seg_off"]
    ratios = []
    for l in range(L):
        for s in range(S):
            for g in range(Hkv):
                u = (l * S + s) * Hkv + g
                qf = _f64(q[l, s, g]).reshape(W, d)
                kf = _f64(k[l, g, s * n:(s + 1) * n]).reshape(n, d)
                vf = _f64(v[l, g, s * n:(s + 1) * n]).reshape(n, d)
                kept_u = set(int(x) for x in kept[off[u]:off[u + 1]])
                j_gpu = tuple(j for j in range(m) if j not in kept_u)
                assert len(j_gpu) == kev
                sc = oracle.scores(q[l:l + 1, s:s + 1, g:g + 1], k[l:l + 1, g:g + 1, s * n:(s + 1) * n],
                                   v[l:l + 1, g:g + 1, s * n:(s + 1) * n], num_seqs=1, num_layers=1, num_q_heads=1,
                                   num_kv_heads=1, head_dim=d, window=W, cu_seqlens=[0, n])["score"][0, 0]
                j_or = oracle.decoupled_eviction(sc, range(m), kev)
                if j_gpu != j_or:  # only near-ties may differ
                    thr = np.sort(sc[:m])[kev - 1:kev + 1]
                    for j in set(j_gpu) ^ set(j_or):
                        assert min(abs(sc[j] - t) for t in thr) <= BAND_RTOL * max(abs(thr).max(), 1e-30), (u, j)
                js, fs = oracle.best_eviction(qf, kf, vf, range(m), kev)
                fh = oracle.eviction_shift(qf, kf, vf, j_gpu)
                assert fh >= fs * (1 - 1e-12), u
                ratios.append(fh / fs)
    r = np.array(ratios)
    say(f"F(J_hat_gpu)/F(J*) over {len(r)} units (m={m}, k={kev}, W={W}, d={d}): median {np.median(r):.3f}, "
        f"p95 {np.percentile(r, 95):.3f}, max {r.max():.3f}, exact {np.mean(r < 1 + 1e-12):.0%}")
