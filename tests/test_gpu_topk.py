"""Per-unit selection on hand-made scores: GPU vs the oracle's full sort.

DropKV page, "Methodology in Plain English": keep the largest scores, the recent window
always. The selection is integer work decided on the same fp32 values on both sides, so
every segment must equal the oracle's (a full sort on (-score, position)) exactly.

Most units are selected in one read of the scores: a strided sample (one 4-key run per
thread of the workgroup, 4096 keys) gives a band of keys around the threshold's expected
rank; one read marks the keys above the band and lists the band's keys in LDS, and the
threshold is found in that list. A unit with at most 11264 competitors lists them all. When
the band missed the threshold or overflowed the list (all keys equal; a periodic pattern
whose high half the sample never sees; the band's keys all in one wave's share of the read,
overflowing that wave's list region), the unit is selected from scratch by the radix select
below, so the sample never changes the result.

The score distributions steer the radix select down its routes: when at most 11264 keys
share the threshold's top 14 bits, the second pass lists them (key and position) in LDS and
marks every competitor above those bits in an LDS bitmask; the last pass and the ordered
emission then read no score. Otherwise the last pass and the emission read the scores
again, and so does the emission of a unit with more competitors than the bitmasks hold
(253952). Covered: a log-uniform spread, one top byte for every key (uniform in [2, 8)),
sixteen distinct values (ties decided by position), ties inside a listed bin (all of these
take the list), a narrow range whose keys all share their top 14 bits but differ below (no
list, distinct keys), all keys equal (no list, all ties), budgets keeping every competitor
or none, sinks (which shift the bitmasks' positions off word boundaries), and a unit too
long for the bitmasks.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_eviction_kvscore_amd import api
from parity import say

pytestmark = pytest.mark.gpu


def _scores(kind, n, rng):
    if kind == "log_uniform":
        return np.exp2(rng.uniform(-60.0, 0.0, n)).astype(np.float32)
    if kind == "one_top_byte":
        return rng.uniform(2.0, 8.0, n).astype(np.float32)
    if kind == "sixteen_values":
        return (2.0 + 0.25 * rng.integers(0, 16, n)).astype(np.float32)
    if kind == "narrow":  # one 14-bit bin: sign, exponent and the top five mantissa bits shared
        return rng.uniform(2.0, 2.0625, n).astype(np.float32)
    if kind == "all_equal":
        return np.full(n, 3.0, dtype=np.float32)
    if kind == "ties_in_list":  # a threshold bin of 8000 keys with sixteen values, over a wide spread
        x = np.exp2(rng.uniform(-60.0, 0.0, n)).astype(np.float32)
        x[rng.choice(n, 8000, replace=False)] = (2.0 + 0.25 * rng.integers(0, 16, 8000)).astype(np.float32)
        return x
    if kind == "periodic":  # high scores in the second half of every 128 positions, low in the first
        j = np.arange(n)
        return np.where(j % 128 >= 64, rng.uniform(4.0, 8.0, n), rng.uniform(0.0, 1.0, n)).astype(np.float32)
    if kind == "one_wave_band":
        # the scores near the threshold all sit where one wave of the read takes its float4s
        # (float4 index mod 1024 below 64); 4000 high scores elsewhere, the rest low
        j = np.arange(n)
        mine = ((j // 4) % 1024) < 64
        x = rng.uniform(0.0, 1.0, n)
        x[rng.choice(np.flatnonzero(~mine), 4000, replace=False)] = rng.uniform(8.0, 9.0, 4000)
        x[mine] = rng.uniform(2.0, 2.001, int(mine.sum()))
        return x.astype(np.float32)
    raise ValueError(kind)


KINDS = ["log_uniform", "one_top_byte", "sixteen_values", "all_equal", "ties_in_list", "narrow", "periodic",
         "one_wave_band"]


@pytest.mark.parametrize("budget_extra,n_sink,n", [(5000, 0, 60011), (0, 0, 60011), (70000, 0, 60011),
                                                    (5000, 5, 60011), (5000, 37, 60011), (20000, 3, 300007),
                                                    (5000, 0, 131088), (70000, 0, 131088), (500, 0, 9000),
                                                    (6000, 2, 9000), (3000, 0, 11280), (3000, 0, 11281),
                                                    (5000, 0, 253968)])
def test_topk_threshold_bins_both_routes(budget_extra, n_sink, n):
    # n = 60011 is ragged against the 4-key loads; 300007 - W competitors exceed the bitmasks;
    # 131088 - W = 2^17 competitors put every sampled run in the low half of the periodic
    # scores; 11280 - W competitors fit the LDS list whole, 11281 - W do not; 253968 - W fill
    # the bitmasks exactly (eight words per thread in the emission)
    L, S, Hkv, Hq, d, W = 1, 1, len(KINDS), len(KINDS), 128, 16
    rng = np.random.default_rng(budget_extra + 5 + n_sink)
    p = api.Problem(num_seqs=S, num_layers=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, window=W,
                    cu_seqlens=[0, n], k_strides=(Hkv * n * d, n * d, d), v_strides=(Hkv * n * d, n * d, d))
    sc = np.stack([_scores(kind, n, rng) for kind in KINDS])  # [Hkv][n]
    b = min(W + n_sink + budget_extra, n)
    budgets = np.full((S, L), b, dtype=np.int32)
    off = api.segment_offsets(p, budgets)
    kept = torch.full((int(off[-1]),), -7, dtype=torch.int32, device="cuda")
    say(f"top-k on hand-made scores: n={n}, budget {b}, sinks {n_sink}, kinds {KINDS}")
    api.topk(p, torch.from_numpy(sc.reshape(-1)).cuda(), budgets, torch.from_numpy(off).cuda(), kept,
             n_sink=n_sink)
    torch.cuda.synchronize()
    got = kept.cpu().numpy()
    for g, kind in enumerate(KINDS):
        ref = oracle.kept_positions(sc[g].astype(np.float64), n, W, b, n_sink=n_sink)
        np.testing.assert_array_equal(got[off[g]:off[g + 1]], ref, err_msg=kind)
