"""GPU parity: the HIP pipeline (through the C ABI) against the fp64 oracle.

Workloads 1 and 2 are checked on every unit; 3, 4 and 5 at full size on one unit per
layer (every layer, KV-head and sequence index covered), every output of each, plus the
selection and compaction of every unit on the GPU's own scores.
Edge cases cover one candidate, empty and full selections, G = 1 / W = 1, d = 64,
ragged sequences, more than 256 rows per unit (several query tiles), one sequence of a
million tokens, 65,280 units (near the launch grids' 65,535 limit), token-major strides,
ties, and run-to-run determinism.
"""
import numpy as np
import pytest
import torch

import oracle

from kv_cache_eviction_kvscore_amd import api, pipeline, synth
from kv_cache_eviction_kvscore_amd.configs import WORKLOADS, Workload, small_variant

from parity import check_selection_every_unit, check_unit, cover_units, run_gpu, sample_units, say

pytestmark = pytest.mark.gpu


def _check_all(w, units, mode=api.MODE_L2, **kw):  # kw: data, k_layout, pool, n_sink
    say(f"[parity] {w.name} mode={mode} units={units} {({k: x for k, x in kw.items() if k != 'data'})}")
    run = run_gpu(w, mode, **kw)
    rep = {}
    for u in units:
        check_unit(w, run, u, mode, rep)
    say(f"[parity] {w.name}: max rel score err {max(rep['max_rel']):.2e}, pmax {max(rep['pmax']):.6f}, "
        f"band sizes {rep['band']}")
    return run


def test_workload1_all_units_l2():
    _check_all(WORKLOADS[1], [0])


def test_workload1_squared_mode():
    _check_all(WORKLOADS[1], [0], mode=api.MODE_SQ)


def test_workload2_all_units():
    w = WORKLOADS[2]
    _check_all(w, list(range(w.num_kv_heads)))


@pytest.mark.parametrize("wid", [3, 4, 5])
def test_full_workloads_every_layer_and_head(wid):
    """Workloads 3-5 at full size: every output of one unit per layer (covering every
    KV-head index and, for the ragged batch, every sequence) against the fp64 oracle, and
    the selection and compaction of every unit on the GPU's own scores."""
    w = WORKLOADS[wid]
    run = _check_all(w, cover_units(w))
    say(f"[parity] {w.name}: selection and compaction of all {check_selection_every_unit(w, run)} units exact")


EDGE = [
    # one candidate token (n = W + 1), budget keeps only the window (k = 0)
    Workload("edge_one_cand_k0", 10, 1, 4, 2, 128, (65,), 64, (0,), "fixed", 64),
    # one candidate, budget keeps everything (k = n - W)
    Workload("edge_one_cand_all", 11, 1, 4, 2, 128, (65,), 64, (0,), "fixed", 65),
    # G = 1, W = 1, d = 64
    Workload("edge_g1_w1_d64", 12, 2, 2, 2, 64, (300,), 1, (5,), "fixed", 40),
    # ragged, odd lengths, d = 64, 24 rows per unit
    Workload("edge_ragged_d64", 13, 2, 6, 2, 64, (100, 1000, 77), 8, (3, 10, 2), "profile", 0.3, ratio=2.5),
    # 448 rows per unit (two query tiles), chunked keys
    Workload("edge_rows448", 14, 1, 28, 4, 128, (5000, 300), 64, (20, 3), "uniform", 0.25),
    # 1024 rows per unit (four query tiles)
    Workload("edge_rows1024", 15, 1, 8, 1, 128, (700,), 128, (4,), "fixed", 300),
    # no sink, no heavy keys: a diffuse softmax
    Workload("edge_diffuse", 16, 1, 8, 2, 128, (3000,), 32, None, "uniform", 0.1, sink=False),
]


@pytest.mark.parametrize("w", EDGE, ids=[e.name for e in EDGE])
def test_edge_cases(w):
    U = w.num_layers * w.num_seqs * w.num_kv_heads
    _check_all(w, list(range(U)))


def test_one_sequence_of_a_million_tokens():
    """One unit with 2^20 + 37 cached tokens: the forward and the score pass split its keys into
    many chunks (the forward's combine runs), the selection has ~1M competitors (more than its
    LDS bitmasks hold, so the ordered-compaction path runs), every output against the fp64
    oracle."""
    w = Workload("long_1m", 31, 1, 4, 1, 128, (1048613,), 64, (2000,), "uniform", 0.05)
    _check_all(w, [0])


def test_units_near_the_grid_limit():
    """65,280 units (255 layers, 4 short sequences, 64 KV heads; the launch grids carry the
    unit count in a dimension capped at 65,535): a spread of units against the oracle, plus
    the selection and compaction of every unit on the GPU's own scores."""
    w = Workload("units_65280", 32, 255, 64, 64, 64, (70, 97, 66, 128), 64, None, "fixed", 66)
    L, S, H, d, W, N = w.num_layers, w.num_seqs, w.num_q_heads, w.head_dim, w.window, w.total_tokens
    gen = torch.Generator(device="cuda").manual_seed(w.seed)  # plain Gaussians: 65,280 per-unit draws would be slow
    data = {"q": torch.randn((L, S, H, W, d), generator=gen, device="cuda").to(torch.bfloat16),
            "k": torch.randn((L, H, N, d), generator=gen, device="cuda").to(torch.bfloat16),
            "v": torch.randn((L, H, N, d), generator=gen, device="cuda").to(torch.bfloat16)}
    _check_all(w, sample_units(w, 12), data=data)


def test_dominant_sink_one_row():
    """One window row per head, the sink aligned with the query: p* is 1 - O(1e-19), so the
    argmax pair's term rests on the rest sums alone (the isolated path in the forward; the
    oracle's removal form)."""
    w = Workload("dominant_sink_w1", 1040805, 3, 2, 2, 128, (3469, 4821, 3375), 1, (16, 28, 17), "fixed", 2104,
                 sink=True)
    _check_all(w, list(range(w.num_layers * w.num_seqs * w.num_kv_heads)), n_sink=4)


def test_squared_mode_one_row_seven_heads():
    """Mode SQ with W = 1 and 7 query heads per KV head, d = 64: few pairs per token, so one
    pair's term can carry a token's score and its distance error is not averaged (a bf16
    A_hat operand missed the bar here)."""
    w = Workload("sq_w1_g7_d64", 672914, 1, 14, 2, 64, (638, 4339, 4170), 1, (26, 0, 2), "uniform", 0.452,
                 sink=True)
    _check_all(w, list(range(w.num_layers * w.num_seqs * w.num_kv_heads)), mode=1, pool=11, n_sink=4)


def test_token_major_strides():
    w = small_variant(WORKLOADS[2], name="tokmajor", seqlens=(4096,), heavy_count=(20,))
    _check_all(w, [0, 3, 7], k_layout="token_major")


def _expansion_floor(w, run, u):
    """Absolute error bound of the score when the true distances vanish.

    The kernel forms D = ||a_hat||^2 + ||v||^2 - 2 a_hat.v (the expansion the DropKV
    page's engineering paragraph describes; a_hat = a rounded to fp16) from fp32 sums of
    at most 2d + 16 products,
    so |dD| <= 2 gamma (||a_hat||^2 + ||v||^2) with gamma = m u / (1 - m u), u = 2^-24,
    m = 2d + 16 (the textbook bound for a floating-point dot product). Since
    |sqrt(x) - sqrt(y)| <= sqrt(|x - y|), token j's score moves by at most
    sum_i c_ij sqrt(2 gamma (||a_hat_i||^2 + ||v_j||^2)), c_ij = p_ij / (1 - p_ij) over
    the pairs the score sums. Returns the largest such bound over the unit's tokens.
    """
    from parity import bits_f64, oracle_unit

    ref = oracle_unit(w, run, u, api.MODE_L2)
    n, W, G, d = w.seqlens[0], w.window, w.group, w.head_dim
    m = 2 * d + 16
    gamma = m * 2.0 ** -24 / (1 - m * 2.0 ** -24)
    ahat = torch.from_numpy(ref["a"]).float().half().double().numpy()
    na = (ahat ** 2).sum(1)
    vf = bits_f64(ref["v"])
    nv = (vf ** 2).sum(1)
    logits = bits_f64(ref["q"]) @ bits_f64(ref["k"]).T / np.sqrt(d)
    p = np.exp(logits - ref["lse"][:, None])
    R = G * W
    pos = n - W + np.arange(R) % W
    mask = np.arange(n)[None, :] <= pos[:, None]
    mask[np.arange(R), ref["jstar"]] = False
    c = np.where(mask, p / (1 - np.where(mask, p, 0)), 0)
    return float((c * np.sqrt(2 * gamma * (na[:, None] + nv[None, :]))).sum(0).max())


def test_ties_constant_values():
    w = Workload("ties", 17, 1, 4, 1, 128, (500,), 16, None, "fixed", 100, sink=False)
    data = synth.generate(w, "cuda")
    data["v"][:] = data["v"][0, 0, 0]  # every value row equal: all true scores are 0
    run = run_gpu(w, data=data)
    # exact zeros are out of reach of the expanded distance in fp32; the absolute floor is
    # the rounding bound of that expansion
    floor = _expansion_floor(w, run, 0)
    say(f"[parity] ties: expansion floor {floor:.3e}")
    check_unit(w, run, 0, atol=floor)


@pytest.mark.parametrize("ratio", [3, 10, 30])
def test_values_with_a_common_offset(ratio):
    """Value rows sharing a large offset: v_j = mu + e_j with e_j ~ N(0, 1) and
    ||mu|| = ratio * sqrt(d), so every a_i lies near mu and ||a_i - v_j|| is small next to
    ||a_i|| and ||v_j||. The expanded distance ||a||^2 - 2 a.v + ||v||^2 then cancels, and
    the fp16 rounding of a weighs ratio times more against the distance; the scores are
    held to the same 1e-3 relative bar with the default absolute floor (DropKV page,
    "Methodology in Plain English": the expanded squared distance)."""
    w = Workload(f"offset{ratio}", 19, 1, 8, 2, 128, (4096,), 32, (20,), "uniform", 0.1)
    data = synth.generate(w, "cuda")
    g = torch.Generator().manual_seed(1000 + ratio)
    mu = torch.randn(w.head_dim, generator=g, dtype=torch.float64)
    mu = mu / mu.norm() * ratio * np.sqrt(w.head_dim)
    data["v"] = (data["v"].double() + mu.to("cuda")).to(torch.bfloat16)
    say(f"[parity] common value offset, ||mu|| / sqrt(d) = {ratio}")
    _check_all(w, list(range(w.num_layers * w.num_seqs * w.num_kv_heads)), data=data)


def test_pyramid_budgets_end_to_end():
    """Layer budgets from kvscore_budget_pyramid (PyramidKV page, "Layer-Adaptive Dynamic
    Budget Allocation": the uniform total reallocated, most to the lowest layer) drive the
    selection and compaction: the library's integers equal the oracle's, and every unit's
    outputs match the oracle with those budgets."""
    w = small_variant(WORKLOADS[3], name="pyramid8", num_layers=8, seqlens=(8192,), heavy_count=(16,))
    L, n, W = w.num_layers, w.seqlens[0], w.window
    total = int(0.1 * n) * L
    b = api.budget_pyramid(L, 1.0, total, W, n)
    assert b.tolist() == oracle.pyramid_budgets(L, total, W, n, 1.0)
    assert b.sum() == total and b[0] > b[L // 2] > b[-1] == W
    say(f"[parity] pyramid budgets {b.tolist()}")
    run = run_gpu(w, budgets=b[None, :].astype(np.int32))
    rep = {}
    for u in range(L * w.num_kv_heads):
        check_unit(w, run, u, api.MODE_L2, rep)
    say(f"[parity] pyramid: max rel score err {max(rep['max_rel']):.2e}")


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_deterministic_bitwise():
    w = small_variant(WORKLOADS[3], name="det", num_layers=2, seqlens=(20000,))
    say("[parity] determinism")
    data = synth.generate(w, "cuda")
    r1 = run_gpu(w, data=data)
    first = {k: _bits(v).clone() for k, v in r1["out"].items() if isinstance(v, torch.Tensor)}
    r1["pipe"].run(data["q"], data["k"], data["v"])
    torch.cuda.synchronize()
    for k, v in r1["pipe"].outputs().items():
        if isinstance(v, torch.Tensor):
            assert torch.equal(_bits(v), first[k]), k


def test_merge_in_place_matches_separate_buffers():
    """With one query tile the pipeline merges in the partial buffer itself; a merge into a
    buffer of its own must give the same bits."""
    w = small_variant(WORKLOADS[3], name="inplace", num_layers=2, seqlens=(20000,))
    data = synth.generate(w, "cuda")
    run = run_gpu(w, data=data)
    pipe, prob = run["pipe"], run["prob"]
    assert pipe.tq == 1 and pipe.score.data_ptr() == pipe.partial.data_ptr()
    partial = torch.empty_like(pipe.partial)
    score = torch.full_like(pipe.score, float("nan"))
    api.score(prob, data["q"], data["k"], data["v"], pipe.a, pipe.lse, pipe.jstar, partial, pipe.ws_score)
    api.merge(prob, partial, pipe.jstar, pipe.dom, score)
    torch.cuda.synchronize()
    assert torch.equal(_bits(score), _bits(pipe.score))


def test_softmax_scale_override():
    w = WORKLOADS[1]
    data = synth.generate(w, "cuda")
    prob = api.Problem.for_tensors(data["k"], data["v"], num_q_heads=w.num_q_heads, window=w.window,
                                   cu_seqlens=w.cu_seqlens(), softmax_scale=0.125)
    pipe = pipeline.Pipeline(prob, pipeline.workload_budgets(w))
    pipe.run(data["q"], data["k"], data["v"])
    prob2 = pipeline.problem_for(w, data["k"], data["v"])  # default 1/sqrt(64) = 0.125
    pipe2 = pipeline.Pipeline(prob2, pipeline.workload_budgets(w))
    pipe2.run(data["q"], data["k"], data["v"])
    torch.cuda.synchronize()
    assert torch.equal(pipe.score, pipe2.score)


# ---- max-pooled ranking key and attention sinks (DropKV page: max-pool over neighbouring
# scores, kernel 11 in its experiments; "Preserve Attention Sinks": the first 4 tokens)


def test_pool11_sinks4_workload2_all_units():
    w = WORKLOADS[2]
    _check_all(w, list(range(w.num_layers * w.num_seqs * w.num_kv_heads)), pool=11, n_sink=4)


def test_pool13_sinks4_ragged_workload5_sampled():
    w = WORKLOADS[5]
    _check_all(w, sample_units(w, 6), pool=13, n_sink=4)


@pytest.mark.parametrize("pool,n_sink,budget", [(255, 0, 120), (3, 40, 120), (1, 4, 120), (11, 1000, 200)])
def test_pool_and_sink_edges(pool, n_sink, budget):
    # pool wider than the prefix, sinks filling much of a short prefix, sinks without pooling,
    # more sinks than candidates (everything kept)
    w = Workload(f"pool{pool}_sink{n_sink}", 18, 1, 4, 2, 64, (200,), 32, (6,), "fixed", budget)
    _check_all(w, [0], pool=pool, n_sink=n_sink)


# ---- attention-sum mode (PyramidKV page, "Observation Window and Aggregated Attention
# Eviction": S_j = sum over the window rows and heads of A_{h,w,j}; SnapKV's ranking)


def test_attention_sum_workload1():
    _check_all(WORKLOADS[1], [0], mode=api.MODE_ATTN)


def test_attention_sum_workload2_all_units():
    w = WORKLOADS[2]
    _check_all(w, list(range(w.num_layers * w.num_seqs * w.num_kv_heads)), mode=api.MODE_ATTN)


def test_attention_sum_ragged_d64_and_pooled_workload5():
    _check_all(EDGE[3], list(range(EDGE[3].num_layers * EDGE[3].num_seqs * EDGE[3].num_kv_heads)),
               mode=api.MODE_ATTN)
    w = WORKLOADS[5]
    _check_all(w, sample_units(w, 4), mode=api.MODE_ATTN, pool=13, n_sink=4)
