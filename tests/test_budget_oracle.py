"""Pins of the oracle's layer-budget map (RippleKV page, Eq. 5, 9-12) and of its selection rule."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "budgets.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["why"][:40])
def test_hand_derived_examples(case):
    gamma = math.inf if case["gamma"] is None else case["gamma"]
    got = oracle.layer_budgets(case["sens"], case["ratio"], gamma, case["total"], case["lo"], case["hi"])
    assert got == case["expect"]


def test_multiplier_ratio_is_exactly_r():
    """Eq. 10: for a non-constant profile max/min multiplier before clipping equals r."""
    rng = np.random.default_rng(0)
    for r in (1.5, 2.0, 3.0, 10.0):
        s = rng.normal(size=12)
        w = oracle._multipliers(s, r, math.inf)
        assert abs(max(w) / min(w) - r) < 1e-12 * r
        assert min(w) == 1.0  # the least sensitive layer has s_hat = 0 -> r^0


@pytest.mark.parametrize("seed", range(20))
def test_randomised_properties(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 40))
    s = rng.normal(size=L) * rng.uniform(0.01, 10)
    r = float(rng.uniform(1.0, 5.0))
    gamma = math.inf if seed % 3 else float(rng.uniform(1.0, 3.0))
    lo = int(rng.integers(0, 50))
    hi = lo + int(rng.integers(1, 5000))
    total = int(rng.integers(L * lo, L * hi + 1))
    b = oracle.layer_budgets(s, r, gamma, total, lo, hi)
    assert sum(b) == total  # Eq. 5
    assert all(lo <= x <= hi for x in b)
    # monotone in sensitivity (Eq. 10 is monotone; clipping and rounding keep the order up to one slot)
    order = np.argsort(s, kind="stable")
    bs = np.asarray(b)[order]
    assert (np.diff(bs) >= -1).all()
    # invariance to positive affine maps of the profile (Eq. 9)
    b2 = oracle.layer_budgets(3.5 * s + 2.0, r, gamma, total, lo, hi)
    assert b2 == b or max(abs(x - y) for x, y in zip(b, b2)) <= 1


def test_workload_totals():
    """Budget totals of the five workloads (floor of the kept fraction)."""
    from kv_cache_eviction_kvscore_amd.configs import WORKLOADS
    w = WORKLOADS
    assert w[1].budget_request(0)[3] == 160
    assert w[2].budget_request(0)[3] == 1638
    assert w[3].budget_request(0)[3] == 104857
    assert w[4].budget_request(0)[3] == 6553 * 32
    assert [w[5].budget_request(s)[3] for s in range(4)] == [183500, 91750, 56000, 17283]
    assert w[5].heavy_count == (393, 197, 120, 37)
    assert w[2].heavy_count == (164,) and w[4].heavy_count == (262,)
    # uniform requests give uniform budgets
    prof, r, g, tot = w[4].budget_request(0)
    assert oracle.layer_budgets(prof, r, g, tot, 64, 131072) == [6553] * 32


def test_infeasible_totals_raise():
    with pytest.raises(ValueError):
        oracle.layer_budgets([0, 1], 2.0, math.inf, 5, 3, 10)
    with pytest.raises(ValueError):
        oracle.layer_budgets([0, 1], 2.0, math.inf, 21, 3, 10)


# ------------------------------------------------------------------ selection (DropKV page)
def _sorted_reference(score, n, W, b):
    cand = n - W
    k = min(max(b - W, 0), cand)
    chosen = sorted(range(cand), key=lambda j: (-score[j], j))[:k]
    return sorted(chosen + list(range(cand, n)))


@pytest.mark.parametrize("seed", range(10))
def test_kept_positions_match_python_sort_and_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(5, 300))
    W = int(rng.integers(1, n))
    b = int(rng.integers(W, n + 1))
    score = rng.integers(0, 20, size=n).astype(np.float64)  # many ties on purpose
    kept = oracle.kept_positions(score, n, W, b)
    assert list(kept) == _sorted_reference(list(score), n, W, b)
    assert len(kept) == b
    assert set(range(n - W, n)) <= set(kept.tolist())
    assert (np.diff(kept) > 0).all()
    cand = n - W
    kin = [j for j in kept if j < cand]
    kout = [j for j in range(cand) if j not in set(kin)]
    if kin and kout:
        assert min(score[kin]) >= max(score[kout])


def test_gather_is_a_row_copy():
    rng = np.random.default_rng(1)
    k = rng.integers(0, 2 ** 16, size=(50, 8), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(50, 8), dtype=np.uint16)
    pos = np.array([0, 3, 4, 49], dtype=np.int32)
    ko, vo = oracle.gather(k, v, pos)
    assert (ko == k[[0, 3, 4, 49]]).all() and (vo == v[[0, 3, 4, 49]]).all()


# ---- PyramidKV schedule (PyramidKV page, "Layer-Adaptive Dynamic Budget Allocation":
# C_l = C_min + (C_max - C_min)(1 - (l-1)/(L-1))^gamma; the layers share the uniform total)
# Hand-derived cases (0-based l, f_l = (1 - l/(L-1))^gamma, x_l = lo + lam f_l, sum = total):
#   L=5, gamma=1, lo=10, T=100: f = 1, .75, .5, .25, 0 (sum 2.5), lam = 50/2.5 = 20
#                              -> 30, 25, 20, 15, 10
#   L=3, gamma=2, lo=8, T=44:   f = 1, .25, 0 (sum 1.25), lam = 20/1.25 = 16 -> 24, 12, 8
#   L=3, gamma=1, lo=10, hi=40, T=90: unclipped 50, 30, 10 exceeds hi; x_0 = 40 and
#                              10 + lam/2 = 40 (lam = 60) -> 40, 40, 10
#   L=3, gamma=1, lo=10, T=40:  lam = 20/3 -> 16.67, 13.33, 10; floors sum 39, the extra
#                              slot goes to the largest remainder (layer 0) -> 17, 13, 10
#   L=1: the one layer takes the total
PYRAMID_CASES = [
    (5, 100, 10, 1000, 1.0, [30, 25, 20, 15, 10]),
    (3, 44, 8, 1000, 2.0, [24, 12, 8]),
    (3, 90, 10, 40, 1.0, [40, 40, 10]),
    (3, 40, 10, 100, 1.0, [17, 13, 10]),
    (1, 40, 10, 100, 1.0, [40]),
]


@pytest.mark.parametrize("L,T,lo,hi,gamma,expect", PYRAMID_CASES)
def test_pyramid_hand_derived(L, T, lo, hi, gamma, expect):
    assert oracle.pyramid_budgets(L, T, lo, hi, gamma) == expect


@pytest.mark.parametrize("seed", range(20))
def test_pyramid_properties(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(2, 40))
    lo = int(rng.integers(1, 100))
    hi = lo + int(rng.integers(0, 5000))
    T = int(rng.integers(L * lo, (L - 1) * hi + lo + 1))  # the top layer stays at lo
    gamma = float(rng.choice([0.5, 0.8, 1.0, 2.0]))
    b = oracle.pyramid_budgets(L, T, lo, hi, gamma)
    assert sum(b) == T and all(lo <= x <= hi for x in b)
    assert all(b[i] >= b[i + 1] for i in range(L - 1))  # non-increasing with depth
    if L * lo < T and b[0] < hi:
        assert b[-1] == lo  # the top layer sits at C_min unless every layer is clipped


def test_pyramid_infeasible():
    with pytest.raises(ValueError):
        oracle.pyramid_budgets(4, 30, 10, 100, 1.0)
    with pytest.raises(ValueError):
        oracle.pyramid_budgets(4, 500, 10, 100, 1.0)
    with pytest.raises(ValueError):  # above (L-1)*hi + lo: the top layer cannot leave lo
        oracle.pyramid_budgets(4, 311, 10, 100, 1.0)
    assert oracle.pyramid_budgets(4, 310, 10, 100, 1.0) == [100, 100, 100, 10]
