"""Randomized whole-pipeline parity: seeded random shapes, modes, pools, sinks and budgets.

Each case draws a small problem (1-3 layers and sequences, 1-3 KV heads, 1-8 query heads
per KV head, d = 64 or 128, windows from 1 to 128 rows, ragged lengths up to ~6000 keys,
heavy keys, an optional sink aligned with the window queries), runs the pipeline once and
checks sampled units against the fp64 oracle to the same bars as the other parity tests:
scores within 1e-3 relative, the GPU's selection the full sort of its own scores and equal
to the oracle's outside the 1e-3 band, the packed cache bit-exact. The head-budget cases
check each (sequence, layer) group's joint selection. Cases like these found a row whose
argmax outweighs the rest by ~45 nats, and a mode-SQ case that needed the fp16 A_hat.

KVSCORE_SWEEP_CASES (default 16) and KVSCORE_SWEEP_SEED (default 9000) set how many cases are
drawn and from which seed on, for longer runs over other seeds; the head-budget cases take a
third as many from the seed plus 500.
"""
import os

import numpy as np
import pytest

from kv_cache_eviction_kvscore_amd import api
from kv_cache_eviction_kvscore_amd.configs import Workload
from parity import check_unit, run_gpu, sample_units, say

pytestmark = pytest.mark.gpu


def _draw(seed, heads=False):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 4))
    Hkv = int(rng.choice([2, 4])) if heads else int(rng.integers(1, 4))
    G = int(rng.choice([1, 2, 4, 7, 8]))
    d = int(rng.choice([64, 128]))
    W = int(rng.choice([1, 2, 7, 16, 33, 64, 128]))
    W = min(W, 512 // G)
    S = int(rng.integers(1, 4))
    lens = tuple(int(x) for x in rng.integers(W + 2, 6000, S))
    heavy = tuple(int(rng.integers(0, 30)) for _ in range(S))
    mode = api.MODE_L2 if heads else int(rng.choice([api.MODE_L2, api.MODE_L2, 1, 2]))
    pool = int(rng.choice([1, 1, 3, 11]))
    n_sink = int(rng.choice([0, 0, 4]))
    kind = str(rng.choice(["fixed", "uniform"]))
    # every budget must hold the window and the sinks: a fraction at least (W + sinks + 1) / n
    lo = min(1.0, (W + n_sink + 1) / min(lens))
    val = (float(rng.integers(W + n_sink, min(lens) + 1)) if kind == "fixed"
           else float(rng.uniform(max(0.02, lo), max(0.6, lo))))
    w = Workload(f"rand{'_heads' if heads else ''}{seed}", int(rng.integers(0, 1 << 20)), L, G * Hkv, Hkv, d, lens,
                 W, heavy, kind, val, sink=bool(rng.integers(0, 2)))
    return w, mode, pool, n_sink


NCASES = int(os.environ.get("KVSCORE_SWEEP_CASES", "16"))
SEED0 = int(os.environ.get("KVSCORE_SWEEP_SEED", "9000"))


@pytest.mark.parametrize("seed", range(NCASES))
def test_random_pipeline(seed):
    w, mode, pool, n_sink = _draw(SEED0 + seed)
    say(f"[sweep] {w} mode={mode} pool={pool} sinks={n_sink}")
    run = run_gpu(w, mode=mode, pool=pool, n_sink=n_sink)
    worst = max(check_unit(w, run, u, mode) for u in sample_units(w, 4))
    say(f"[sweep] {w.name}: max rel score err {worst:.2e}")


@pytest.mark.parametrize("seed", range(max(1, (NCASES + 2) // 3)))
def test_random_head_budgets(seed):
    from test_gpu_heads import _check_group

    w, mode, pool, n_sink = _draw(SEED0 + 500 + seed, heads=True)
    say(f"[sweep] {w} heads pool={pool} sinks={n_sink}")
    run = run_gpu(w, mode=mode, pool=pool, n_sink=n_sink, heads=True)
    for l in range(w.num_layers):
        for s in range(w.num_seqs):
            _check_group(w, run, l, s)
