"""The C ABI without a GPU: the library loads, exports what include/kvscore.h declares,
validates arguments on the host, and its host-only budget map agrees with the oracle."""
import ctypes
import math
from fractions import Fraction
import os
import re
import subprocess

import numpy as np
import pytest

from kv_cache_eviction_kvscore_amd import api
from kv_cache_eviction_kvscore_amd.configs import WORKLOADS

import oracle

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvscore.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvscore_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = api.load()
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", api.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kvscore_\w+)", out))
    assert set(names) <= exported
    assert set(api.EXPORTS) == set(names)
    assert api.version() >= 100


def make_problem(**kw):
    base = dict(num_seqs=1, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128, window=16,
                cu_seqlens=[0, 100], k_strides=(2 * 100 * 128, 100 * 128, 128), v_strides=(2 * 100 * 128, 100 * 128, 128))
    base.update(kw)
    return api.Problem(**base)


BAD = [
    dict(head_dim=96),
    dict(num_q_heads=6, num_kv_heads=4),
    dict(window=0),
    dict(window=100),  # sequence not longer than the window
    dict(cu_seqlens=[5, 100]),
    dict(mode=3),
    dict(k_strides=(2 * 100 * 128, 100 * 128, 4)),
    dict(v_strides=(2 * 100 * 128, 100 * 128 + 3, 128)),
    dict(num_q_heads=1024 * 2, num_kv_heads=1, window=2),
    dict(num_seqs=0, cu_seqlens=[0]),
    dict(softmax_scale=float("inf")),
    dict(softmax_scale=float("nan")),
    # units (L*S*Hkv) index a launch grid dimension: at most 65535
    dict(num_layers=32768, num_q_heads=8, num_kv_heads=2),
    dict(num_layers=1366, num_seqs=3, cu_seqlens=[0, 100, 200, 300], num_q_heads=32, num_kv_heads=16),
]


@pytest.mark.parametrize("kw", BAD, ids=[str(b) for b in BAD])
def test_invalid_problems_are_rejected_before_any_launch(kw):
    p = make_problem(**kw)
    assert p.workspace_size(api.WS_ATTN_FWD) == 0
    with pytest.raises(api.KvscoreError) as e:
        # NULL tensors: only host validation can run, nothing is launched
        api.load()
        api._check(api.load().kvscore_attn_fwd(p.ref, None, None, None, None, None, None, None, None, 0, None))
    assert e.value.code == 1


def test_null_tensors_and_small_workspace_rejected():
    p = make_problem()
    lib = api.load()
    with pytest.raises(api.KvscoreError) as e:
        api._check(lib.kvscore_score(p.ref, None, None, None, None, None, None, None, None, 0, None))
    assert e.value.code == 1
    # every sequence in one key chunk: the forward needs no workspace
    assert p.workspace_size(api.WS_ATTN_FWD) == 0
    # one layer of 8 heads over 32K tokens is split into key chunks: then it needs records
    n, Hkv = 32768, 8
    pc = make_problem(num_layers=1, num_q_heads=4 * Hkv, num_kv_heads=Hkv, window=64, cu_seqlens=[0, n],
                      k_strides=(Hkv * n * 128, n * 128, 128), v_strides=(Hkv * n * 128, n * 128, 128))
    need = pc.workspace_size(api.WS_ATTN_FWD)
    assert need > 0
    fake = 1 << 20  # a non-null, aligned address that is never dereferenced
    rc = lib.kvscore_attn_fwd(pc.ref, fake, fake, fake, fake, fake, fake, fake, fake, need - 1, None)
    assert rc == 2 and b"need" in lib.kvscore_last_error()
    rc = lib.kvscore_attn_fwd(pc.ref, fake, fake, fake, fake, fake, fake, fake, None, need, None)
    assert rc == 2 and b"NULL" in lib.kvscore_last_error()
    rc = lib.kvscore_attn_fwd(pc.ref, fake + 8, fake, fake, fake, fake, fake, fake, fake, need, None)
    assert rc == 1  # q not 16-byte aligned


def test_merge_in_place_only_with_one_query_tile():
    """partial and score may be one buffer only when there is one query tile (then the layouts
    agree); with two tiles that is rejected before any launch."""
    p2 = make_problem(num_q_heads=28, num_kv_heads=4, window=64)  # 448 rows -> 2 tiles
    lib = api.load()
    fake = 1 << 20
    rc = lib.kvscore_merge(p2.ref, fake, fake + 4096, fake + 8192, fake, None)
    assert rc == api.EINVAL and b"one query tile" in lib.kvscore_last_error()


def test_query_tiles_and_workspace_sizes():
    p = make_problem()  # G*W = 64 rows
    assert p.num_query_tiles() == 1
    p2 = make_problem(num_q_heads=28, num_kv_heads=4, window=64)  # 448 rows -> 2 tiles
    assert p2.num_query_tiles() == 2
    assert p2.workspace_size(api.WS_SCORE) == p2.rows * 128 * 2 + p2.rows * 8
    # the pooled ranking keys: one fp32 per (layer, KV head, token)
    assert p2.workspace_size(api.WS_TOPK) == p2.num_layers * p2.num_kv_heads * p2.total_tokens * 4


def test_forward_chunks_follow_the_makespan_estimate():
    # the forward workspace holds one record block (196 RT floats at d = 128) per (unit,
    # query tile, key chunk); the chunk is picked per problem, so its size shows the pick
    block = 196 * 256 * 4

    def fwd_chunks(L, Hkv, seqlens):
        n = max(seqlens)
        cu = [0] + list(np.cumsum(seqlens))
        p = make_problem(num_layers=L, num_q_heads=4 * Hkv, num_kv_heads=Hkv, window=64, num_seqs=len(seqlens),
                         cu_seqlens=cu, k_strides=(Hkv * cu[-1] * 128, cu[-1] * 128, 128),
                         v_strides=(Hkv * cu[-1] * 128, cu[-1] * 128, 128))
        U = L * len(seqlens) * Hkv
        ws = p.workspace_size(api.WS_ATTN_FWD)
        assert ws % (U * block) == 0
        # no records at all when every sequence is one chunk (the pass writes its outputs)
        return (ws // (U * block) if ws else 1), n

    # 32 layers x 8 KV heads of 128K tokens: 256 units for 256 CUs, one chunk each
    assert fwd_chunks(32, 8, [131072]) == (1, 131072)
    # one layer x 8 heads of 32K: 8 units, so 1024-key chunks spread them over the CUs
    assert fwd_chunks(1, 8, [32768])[0] == 32
    # ragged lengths: shorter chunks than the longest sequence
    assert fwd_chunks(28, 4, [131072, 65536, 40000, 12345])[0] == 4


def test_segment_offsets_layout_and_budget_validation():
    p = make_problem(num_seqs=2, cu_seqlens=[0, 100, 150])
    b = np.array([[20, 30], [16, 50]], dtype=np.int32)  # [S][L]
    off = api.segment_offsets(p, b)
    # unit u = (l*S + s)*Hkv + g, Hkv = 2
    lens = [b[(u // 2) % 2][u // 4] for u in range(8)]
    assert list(np.diff(off)) == lens and off[0] == 0
    with pytest.raises(api.KvscoreError) as e:
        api.segment_offsets(p, np.array([[20, 30], [15, 50]], dtype=np.int32))  # below the window
    assert e.value.code == 3
    with pytest.raises(api.KvscoreError):
        api.segment_offsets(p, np.array([[20, 101], [16, 50]], dtype=np.int32))  # above n


# ------------------------------------------------------------------ budgets: library vs oracle
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload_budgets_match_oracle(cid):
    w = WORKLOADS[cid]
    for s in range(w.num_seqs):
        prof, r, g, tot = w.budget_request(s)
        got = api.budget(prof, r, g, tot, w.window, w.seqlens[s])
        ref = oracle.layer_budgets(prof, r, g, tot, w.window, w.seqlens[s])
        assert list(got) == ref
        assert got.sum() == tot


def test_workload_budget_values():
    w3 = WORKLOADS[3]
    b3 = api.budget(*w3.budget_request(0), w3.window, w3.seqlens[0])
    assert b3.sum() == 104857 and b3.max() / b3.min() < 2.0 + 1e-9 and len(set(b3)) > 5
    w4 = WORKLOADS[4]
    assert list(api.budget(*w4.budget_request(0), 64, 131072)) == [6553] * 32
    w2 = WORKLOADS[2]
    assert list(api.budget(*w2.budget_request(0), 64, 32768)) == [1638]


@pytest.mark.parametrize("seed", range(40))
def test_random_budgets_match_oracle(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 64))
    s = rng.normal(size=L) * rng.uniform(0.01, 5)
    if seed % 5 == 0:
        s[:] = 1.25  # constant profile
    r = float(rng.uniform(1.0, 6.0))
    gamma = math.inf if seed % 3 else float(rng.uniform(1.0, 3.0))
    lo = int(rng.integers(0, 100))
    hi = lo + int(rng.integers(1, 20000))
    total = int(rng.integers(L * lo, L * hi + 1))
    got = api.budget(s, r, gamma, total, lo, hi)
    ref = oracle.layer_budgets(s, r, gamma, total, lo, hi)
    assert list(got) == ref


def test_random_budgets_match_oracle_bulk():
    """1000 random requests, all layers' integers equal to the oracle's (exact rationals)."""
    rng = np.random.default_rng(7)
    for i in range(1000):
        L = int(rng.integers(1, 48))
        s = rng.normal(size=L) * rng.uniform(0.01, 5)
        if i % 7 == 0:
            s[:] = 0.5  # constant profile
        if i % 11 == 0:
            s = np.round(s, 1)  # repeated values: equal multipliers, equal remainders
        r = float(rng.choice([1.0, 2.0, 3.0, float(rng.uniform(1.0, 8.0))]))
        gamma = math.inf if i % 3 else float(rng.uniform(1.0, 3.0))
        lo = int(rng.integers(0, 80))
        hi = lo + int(rng.integers(0, 5000))
        total = int(rng.integers(L * lo, L * hi + 1))
        got = api.budget(s, r, gamma, total, lo, hi)
        ref = oracle.layer_budgets(s, r, gamma, total, lo, hi)
        assert list(got) == ref, (i, L, r, gamma, lo, hi, total)
        assert got.sum() == total and got.min() >= lo and got.max() <= hi


def test_budget_near_tie_pin():
    """Two remainders 1e-10 apart (RippleKV Eq. 12 rounded under Eq. 5): the larger one
    takes the extra slot. With sens = (0, 1) the multipliers are (1, r) (Eq. 9-10), so
    x = 3 (1, r) / (1 + r); r = 1 + 4e-10/3 puts x near 1.5 - 5e-11 and 1.5 + 5e-11.
    Rounding the remainders to 1e-9 before ordering them would tie them and hand the slot
    to layer 0."""
    r = 1.0 + 4e-10 / 3
    w = [Fraction(1.0), Fraction(math.exp(math.log(r) * 1.0))]
    x = [3 * wl / sum(w) for wl in w]
    rem = [xi - math.floor(xi) for xi in x]
    assert 0 < rem[1] - rem[0] < Fraction(1, 10 ** 9)
    assert list(api.budget([0.0, 1.0], r, math.inf, 3, 0, 3)) == [1, 2]
    assert oracle.layer_budgets([0.0, 1.0], r, math.inf, 3, 0, 3) == [1, 2]
    # the same near-tie between the first and the last of four layers, with a clip active
    sens = [0.0, 0.3, 0.3, 1.0]
    for total in (10, 11, 13):
        assert list(api.budget(sens, r, math.inf, total, 2, 6)) == oracle.layer_budgets(sens, r, math.inf, total, 2, 6)


def test_pyramid_budget_integer_gamma_against_oracle():
    """Integer exponents: the curve is rational and both sides take it exactly."""
    rng = np.random.default_rng(99)
    for _ in range(300):
        L = int(rng.integers(1, 40))
        lo = int(rng.integers(0, 100))
        hi = lo + int(rng.integers(0, 3000))
        gamma = float(rng.integers(0, 13))
        f = [1.0] if L == 1 else [(1 - l / (L - 1)) ** gamma for l in range(L)]
        T = int(rng.integers(L * lo, sum(hi if x > 0 else lo for x in f) + 1))
        assert api.budget_pyramid(L, gamma, T, lo, hi).tolist() == oracle.pyramid_budgets(L, T, lo, hi, gamma)


@pytest.mark.parametrize("case", [dict(ratio=0.5), dict(gamma=0.5), dict(lo=-1), dict(total=10 ** 9)])
def test_budget_errors(case):
    args = dict(sens=[0.0, 1.0, 2.0], ratio=2.0, gamma=math.inf, total=30, lo=1, hi=100)
    args.update(case)
    with pytest.raises(api.KvscoreError):
        api.budget(**args)


def _topk_rc(p, budgets, pool, n_sink, ws_bytes=0):
    """Calls kvscore_topk with placeholder device pointers: every case here fails validation,
    which happens before any launch, so the pointers are never used."""
    lib = api.load()
    b = np.ascontiguousarray(np.asarray(budgets, dtype=np.int32))
    fake = ctypes.c_void_p(0x1000)
    return lib.kvscore_topk(p.ref, fake, ctypes.c_void_p(b.ctypes.data), fake, fake, pool, n_sink,
                            fake if ws_bytes else None, ws_bytes, None)


def test_topk_pool_and_sink_validation():
    p = make_problem(num_seqs=2, cu_seqlens=[0, 100, 150])  # W = 16, L = 2
    good = np.array([[40, 40], [30, 30]], dtype=np.int32)
    assert _topk_rc(p, good, 4, 0) == api.EINVAL  # even pool
    assert _topk_rc(p, good, 0, 0) == api.EINVAL
    assert _topk_rc(p, good, 257, 0) == api.EINVAL  # beyond the largest pool
    assert _topk_rc(p, good, 1, -1) == api.EINVAL
    assert _topk_rc(p, np.array([[40, 40], [30, 19]], dtype=np.int32), 1, 4) == api.EBUDGET  # 19 < 16 + 4
    assert "window + sinks" in api.load().kvscore_last_error().decode()
    assert _topk_rc(p, good, 11, 4) == api.EWORKSPACE  # pooling needs the workspace
    assert _topk_rc(p, good, 11, 4, ws_bytes=16) == api.EWORKSPACE  # too small


@pytest.mark.parametrize("L,gamma,T,lo,hi", [(5, 1.0, 100, 10, 1000), (3, 2.0, 44, 8, 1000), (3, 1.0, 90, 10, 40),
                                             (3, 1.0, 40, 10, 100), (1, 1.0, 40, 10, 100),
                                             (32, 0.8, 32 * 6553, 64, 131072), (28, 1.0, 183500, 64, 131072)])
def test_pyramid_budget_matches_oracle(L, gamma, T, lo, hi):
    assert api.budget_pyramid(L, gamma, T, lo, hi).tolist() == oracle.pyramid_budgets(L, T, lo, hi, gamma)


def test_pyramid_budget_random_against_oracle():
    rng = np.random.default_rng(2024)
    for _ in range(500):
        L = int(rng.integers(1, 60))
        lo = int(rng.integers(0, 200))
        hi = lo + int(rng.integers(0, 10000))
        gamma = float(rng.choice([0.0, 0.5, 0.8, 1.0, 1.5, 2.0, 3.7]))
        f = [1.0] if L == 1 else [(1 - l / (L - 1)) ** gamma for l in range(L)]
        T = int(rng.integers(L * lo, sum(hi if x > 0 else lo for x in f) + 1))
        assert api.budget_pyramid(L, gamma, T, lo, hi).tolist() == oracle.pyramid_budgets(L, T, lo, hi, gamma)


def test_pyramid_budget_errors():
    with pytest.raises(api.KvscoreError) as e:
        api.budget_pyramid(4, 1.0, 311, 10, 100)  # the top layer cannot leave lo
    assert e.value.code == api.EBUDGET
    with pytest.raises(api.KvscoreError):
        api.budget_pyramid(4, -1.0, 100, 10, 100)
    with pytest.raises(api.KvscoreError):
        api.budget_pyramid(0, 1.0, 100, 10, 100)


def _decode_rc(p, off, *, q=0x1000, k=0x1000, v=0x1000, out=0x1000, lse=0x1000, ws_bytes=None):
    lib = api.load()
    off = np.ascontiguousarray(np.asarray(off, dtype=np.int64))
    need = int(lib.kvscore_decode_workspace_size(p.ref, ctypes.c_void_p(off.ctypes.data)))
    fake = ctypes.c_void_p(0x1000)
    vp = lambda a: None if a is None else ctypes.c_void_p(a)
    return lib.kvscore_decode_attn(p.ref, vp(q), vp(k), vp(v), ctypes.c_void_p(off.ctypes.data), fake, vp(out), vp(lse),
                                   fake, need if ws_bytes is None else ws_bytes, None)


def test_decode_workspace_size():
    p = make_problem()  # L = 2, S = 1, Hkv = 2, G = 4, d = 128: four segments
    off = np.array([0, 100, 200, 300, 400], dtype=np.int64)
    # 100 keys per segment: one split per segment; records of (m, l, acc[d]) per query head
    assert api.decode_workspace_size(p, off) == 4 * 1 * 4 * (128 + 2) * 4
    long = np.array([0, 100000, 100001, 100002, 100003], dtype=np.int64)
    ws = api.decode_workspace_size(p, long)
    assert ws % (4 * 4 * 130 * 4) == 0 and ws > 4 * 4 * 130 * 4  # the long segment is split


def test_decode_validation():
    p = make_problem()
    good = [0, 10, 20, 30, 40]
    assert _decode_rc(p, good, ws_bytes=0) == api.EWORKSPACE
    assert _decode_rc(p, [0, 10, 10, 30, 40]) == api.EINVAL  # empty segment
    assert "empty" in api.load().kvscore_last_error().decode()
    assert _decode_rc(p, [0, 10, 5, 30, 40]) == api.EINVAL  # decreasing
    assert _decode_rc(p, [1, 10, 20, 30, 40]) == api.EINVAL  # must start at 0
    assert _decode_rc(p, good, q=None) == api.EINVAL
    assert _decode_rc(p, good, lse=None) == api.EINVAL
    assert _decode_rc(p, good, k=0x1008) == api.EINVAL  # not 16-byte aligned
    assert _decode_rc(p, good, out=0x1002) == api.EINVAL
    assert _decode_rc(make_problem(num_q_heads=18, num_kv_heads=2), good) == api.EINVAL  # G = 9 > 8
    assert "at most 8" in api.load().kvscore_last_error().decode()
    assert _decode_rc(make_problem(head_dim=96), good) == api.EINVAL
    assert _decode_rc(make_problem(softmax_scale=float("inf")), good) == api.EINVAL
    with pytest.raises(api.KvscoreError):
        api.decode_attn(p, None, None, None, [0, 10, 10, 30, 40], None, None, None, None)


def test_token_stride_limit():
    big = 1 << 22
    p = make_problem(k_strides=(2 * 100 * big, 100 * big, big))
    assert p.workspace_size(api.WS_SCORE) == 0
    assert "2^22" in api.load().kvscore_last_error().decode()
    p = make_problem(v_strides=(2 * 100 * 128, 100 * 128, big - 8))
    assert p.workspace_size(api.WS_SCORE) > 0


def test_topk_heads_and_compact_heads_validation():
    lib = api.load()
    p = make_problem(num_seqs=2, cu_seqlens=[0, 100, 150])  # W = 16, L = 2
    good = np.array([[40, 40], [30, 30]], dtype=np.int32)
    fake = ctypes.c_void_p(0x1000)
    bp = ctypes.c_void_p(good.ctypes.data)

    def rc(pool=1, n_sink=0, head=fake, budgets=bp):
        return lib.kvscore_topk_heads(p.ref, fake, budgets, fake, head, fake, pool, n_sink, None, 0, None)

    assert rc(head=None) == api.EINVAL
    assert rc(pool=2) == api.EINVAL
    assert rc(n_sink=-1) == api.EINVAL
    bad = np.array([[40, 40], [30, 19]], dtype=np.int32)
    assert rc(n_sink=4, budgets=ctypes.c_void_p(bad.ctypes.data)) == api.EBUDGET
    assert rc(pool=11) == api.EWORKSPACE
    assert lib.kvscore_compact_heads(p.ref, fake, fake, bp, None, fake, fake, fake, None) == api.EINVAL
    assert lib.kvscore_compact_heads(p.ref, fake, fake, bp, fake, fake, ctypes.c_void_p(0x1004), fake,
                                     None) == api.EINVAL  # k_out misaligned


def test_unit_limit_boundary():
    """65535 units are accepted, one more is rejected with a message naming the limit."""
    ok = make_problem(num_layers=65535 // 5, num_q_heads=5, num_kv_heads=5,
                      k_strides=(5 * 100 * 128, 100 * 128, 128), v_strides=(5 * 100 * 128, 100 * 128, 128))
    assert ok.workspace_size(api.WS_SCORE) > 0
    bad = make_problem(num_layers=65536 // 4, num_q_heads=4, num_kv_heads=4)
    assert bad.workspace_size(api.WS_SCORE) == 0
    assert "65535" in api.load().kvscore_last_error().decode()


def test_decode_noalloc_rejects_scratch_beyond_its_array():
    """kvscore_decode_attn_noalloc: segments whose split records exceed the fixed array
    (KVSCORE_DECODE_SCRATCH_BYTES) are rejected with EWORKSPACE before any HIP call, so the
    placeholder pointers are never used."""
    L, Hkv, Hq, d = 1100, 8, 64, 128  # 8800 one-row segments x 8 heads x 130 floats > 32 MiB
    p = api.Problem(num_seqs=1, num_layers=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, window=1,
                    cu_seqlens=[0, 2], k_strides=(Hkv * 2 * d, 2 * d, d), v_strides=(Hkv * 2 * d, 2 * d, d))
    off = np.arange(0, L * Hkv + 1, dtype=np.int64)
    assert api.decode_workspace_size(p, off) > api.DECODE_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    lib = api.load()
    rc = lib.kvscore_decode_attn_noalloc(p.ref, fake, fake, fake, ctypes.c_void_p(off.ctypes.data), fake, fake, fake,
                                         None)
    assert rc == api.EWORKSPACE
    assert "scratch" in lib.kvscore_last_error().decode()
    assert lib.kvscore_decode_attn_noalloc(p.ref, None, fake, fake, ctypes.c_void_p(off.ctypes.data), fake, fake,
                                           fake, None) == api.EINVAL
