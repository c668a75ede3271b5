"""Pins for the oracle's max-pool + sink selection (CPU only).

DropKV page, "Methodology in Plain English": a max-pool over neighbouring scores and
the recent w tokens always retained, after SnapKV (kernel size 11 in its experiments);
"Preserve Attention Sinks": the first tokens are always kept. The pooled key is checked
against two library routines that compute a windowed maximum with -inf padding
(scipy.ndimage.maximum_filter1d and torch's max_pool1d, SnapKV's own call form), and
the kept set against an exchange-optimality check that needs no sort.
"""
import numpy as np
import pytest
import scipy.ndimage
import torch

import oracle


def _scores(rng, n, ties=False):
    if ties:
        return rng.integers(0, 6, size=n).astype(np.float64)
    return rng.gamma(1.0, 1.0, size=n)


@pytest.mark.parametrize("pool", [1, 3, 11, 13, 25])
@pytest.mark.parametrize("seed", range(4))
def test_pool_matches_scipy_and_torch(pool, seed):
    rng = np.random.default_rng(seed)
    cand = int(rng.integers(1, 300))
    sc = _scores(rng, cand + 5, ties=seed % 2 == 1)
    got = oracle.pooled_scores(sc, cand, pool)
    ref_scipy = scipy.ndimage.maximum_filter1d(sc[:cand], size=pool, mode="constant", cval=-np.inf)
    np.testing.assert_array_equal(got, ref_scipy)
    x = torch.tensor(sc[:cand], dtype=torch.float64)[None, None]
    ref_torch = torch.nn.functional.max_pool1d(x, pool, stride=1, padding=pool // 2)[0, 0].numpy()
    np.testing.assert_array_equal(got, ref_torch)


def test_pool_rejects_even_and_zero():
    with pytest.raises(ValueError):
        oracle.pooled_scores(np.ones(5), 5, 4)
    with pytest.raises(ValueError):
        oracle.pooled_scores(np.ones(5), 5, 0)


@pytest.mark.parametrize("seed", range(12))
def test_pooled_selection_exchange_optimal(seed):
    rng = np.random.default_rng(100 + seed)
    W = int(rng.integers(1, 9))
    n = W + int(rng.integers(1, 200))
    cand = n - W
    n_sink = int(rng.integers(0, 6))
    ns = min(n_sink, cand)
    pool = int(rng.choice([1, 3, 5, 11]))
    b = int(rng.integers(W + ns, n + 1))
    sc = _scores(rng, n, ties=seed % 3 == 0)
    kept = oracle.kept_positions(sc, n, W, b, pool=pool, n_sink=n_sink)
    assert len(kept) == b and (np.diff(kept) > 0).all()
    ks = set(kept.tolist())
    assert set(range(ns)) <= ks and set(range(cand, n)) <= ks
    key = scipy.ndimage.maximum_filter1d(sc[:cand], size=pool, mode="constant", cval=-np.inf)
    comp_kept = [j for j in range(ns, cand) if j in ks]
    comp_out = [j for j in range(ns, cand) if j not in ks]
    for j in comp_kept:  # every kept competitor beats every dropped one (key, then lower position)
        for i in comp_out:
            assert key[j] > key[i] or (key[j] == key[i] and j < i)


def test_wide_pool_keeps_the_first_competitors():
    # a pool wider than the prefix gives every token the prefix maximum: all tie, so the
    # k lowest competitors are kept
    rng = np.random.default_rng(7)
    n, W, b, ns = 120, 8, 40, 3
    sc = _scores(rng, n)
    kept = oracle.kept_positions(sc, n, W, b, pool=2 * n + 1, n_sink=ns)
    k = b - W - ns
    expect = list(range(ns)) + list(range(ns, ns + k)) + list(range(n - W, n))
    assert kept.tolist() == expect


def test_no_pool_no_sinks_is_the_plain_selection():
    rng = np.random.default_rng(3)
    n, W, b = 300, 16, 80
    sc = _scores(rng, n)
    plain = np.sort(np.concatenate([np.argsort(-sc[: n - W], kind="stable")[: b - W], np.arange(n - W, n)]))
    np.testing.assert_array_equal(oracle.kept_positions(sc, n, W, b, pool=1, n_sink=0), plain)


def test_sinks_larger_than_the_prefix_and_budget_errors():
    sc = np.arange(10, dtype=np.float64)
    kept = oracle.kept_positions(sc, 10, 4, 10, pool=3, n_sink=50)  # ns = cand = 6: everything kept
    assert kept.tolist() == list(range(10))
    with pytest.raises(ValueError):
        oracle.kept_positions(sc, 10, 4, 6, n_sink=3)  # b < W + ns


# ---- head budgets chosen jointly over a layer's KV heads (AdaDropKV reading)
def _heads_by_repeated_max(score_heads, n, W, b, ns):
    """A different selection: repeatedly take the best remaining (key, -head, -position)."""
    H, cand = len(score_heads), n - W
    left = {(g, j) for g in range(H) for j in range(ns, cand)}
    chosen = [[] for _ in range(H)]
    for _ in range(min(H * (b - W - ns), len(left))):
        g, j = max(left, key=lambda t: (float(score_heads[t[0]][t[1]]), -t[0], -t[1]))
        left.remove((g, j))
        chosen[g].append(j)
    return [sorted(list(range(ns)) + chosen[g] + list(range(cand, n))) for g in range(H)]


def test_heads_single_head_is_the_per_unit_selection():
    rng = np.random.default_rng(31)
    for _ in range(20):
        n, W = int(rng.integers(10, 200)), int(rng.integers(1, 8))
        ns = int(rng.integers(0, 4))
        b = int(rng.integers(W + min(ns, n - W), n + 1))
        sc = rng.standard_normal(n)
        for pool in (1, 3):
            assert oracle.kept_positions_heads([sc], n, W, b, pool, ns)[0].tolist() == \
                oracle.kept_positions(sc, n, W, b, pool, ns).tolist()


def test_heads_joint_selection_matches_repeated_max_and_keeps_the_layer_total():
    rng = np.random.default_rng(32)
    for trial in range(30):
        H = int(rng.integers(1, 5))
        n, W = int(rng.integers(8, 60)), int(rng.integers(1, 6))
        ns = int(rng.integers(0, 3))
        nse = min(ns, n - W)
        b = int(rng.integers(W + nse, n + 1))
        sc = [np.round(rng.standard_normal(n), 1) for _ in range(H)]  # coarse: many ties
        got = oracle.kept_positions_heads(sc, n, W, b, 1, ns)
        assert [g.tolist() for g in got] == _heads_by_repeated_max(sc, n, W, b, nse)
        assert sum(len(g) for g in got) == H * b
        kept = {(h, j) for h in range(H) for j in got[h] if nse <= j < n - W}
        out = {(h, j) for h in range(H) for j in range(nse, n - W)} - kept
        if kept and out:
            assert min(sc[h][j] for h, j in kept) >= max(sc[h][j] for h, j in out)
