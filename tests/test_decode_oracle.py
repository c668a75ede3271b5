"""Pins for the oracle's decode attention over the packed ragged cache.

RippleKV page, "Problem Formulation": during decoding each new query attends to the
cached states; with compression those are the retained (k, v) pairs of Eq. 4. GraceKV
page, physical cache packing: every (layer, KV head) gets a cache of its own length.

The oracle is checked against closed forms (one key; a zero query), against torch's
scaled-dot-product attention in fp64, against the C oracle's attention forward (a
decode query over the uncompressed cache is the last window row of the prefill
forward, which sees every key), and against invariances that a wrong segment or row
index would break.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f64(bits):
    return (np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ragged(rng, L, S, Hq, Hkv, d, lens, qscale=1.0):
    U = L * S * Hkv
    assert len(lens) == U
    off = np.zeros(U + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    q = bf16_bits(rng.standard_normal((L, S, Hq, d)) * qscale)
    k = bf16_bits(rng.standard_normal((int(off[-1]), d)))
    v = bf16_bits(rng.standard_normal((int(off[-1]), d)))
    return q, k, v, off


def test_single_key_segments_return_that_value_row():
    rng = np.random.default_rng(1)
    L, S, Hq, Hkv, d = 2, 2, 4, 2, 16
    q, k, v, off = ragged(rng, L, S, Hq, Hkv, d, [1] * (L * S * Hkv))
    out, lse = oracle.decode_attention(q, k, v, off, num_layers=L, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv)
    G = Hq // Hkv
    kf, vf, qf = f64(k), f64(v), f64(q).reshape(L, S, Hq, d)
    for l in range(L):
        for s in range(S):
            for h in range(Hq):
                u = (l * S + s) * Hkv + h // G
                assert np.array_equal(out[l, s, h], vf[u])  # weight exactly 1
                assert lse[l, s, h] == pytest.approx(float(kf[u] @ qf[l, s, h]) / math.sqrt(d), rel=1e-15, abs=1e-15)


def test_zero_query_averages_the_segment():
    rng = np.random.default_rng(2)
    L, S, Hq, Hkv, d = 1, 3, 2, 1, 8
    lens = [5, 1, 12]
    q, k, v, off = ragged(rng, L, S, Hq, Hkv, d, lens)
    q[:] = 0
    out, lse = oracle.decode_attention(q, k, v, off, num_layers=L, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv)
    vf = f64(v)
    for s in range(S):
        seg = vf[off[s]:off[s + 1]]
        for h in range(Hq):
            np.testing.assert_allclose(out[0, s, h], seg.mean(axis=0), rtol=1e-14, atol=1e-15)
            assert lse[0, s, h] == pytest.approx(math.log(lens[s]), rel=1e-14)


@pytest.mark.parametrize("G,d", [(4, 128), (7, 64), (1, 64)])
def test_matches_torch_sdpa_fp64(G, d):
    rng = np.random.default_rng(3 + G)
    L, S, Hkv = 2, 2, 2
    Hq = G * Hkv
    lens = list(rng.integers(1, 300, size=L * S * Hkv))
    q, k, v, off = ragged(rng, L, S, Hq, Hkv, d, lens, qscale=2.0)
    scale = 0.37
    out, lse = oracle.decode_attention(q, k, v, off, num_layers=L, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv,
                                       scale=scale)
    qf = torch.from_numpy(f64(q).reshape(L, S, Hq, d))
    kf, vf = torch.from_numpy(f64(k)), torch.from_numpy(f64(v))
    for l in range(L):
        for s in range(S):
            for g in range(Hkv):
                u = (l * S + s) * Hkv + g
                K, V = kf[off[u]:off[u + 1]], vf[off[u]:off[u + 1]]
                qq = qf[l, s, g * G:(g + 1) * G]  # [G, d]
                ref = torch.nn.functional.scaled_dot_product_attention(qq[None], K[None], V[None], scale=scale)[0]
                np.testing.assert_allclose(out[l, s, g * G:(g + 1) * G], ref.numpy(), rtol=1e-12, atol=1e-13)
                ref_lse = torch.logsumexp(scale * (qq @ K.T), dim=1)
                np.testing.assert_allclose(lse[l, s, g * G:(g + 1) * G], ref_lse.numpy(), rtol=1e-13, atol=1e-13)


def test_uncompressed_cache_reproduces_the_prefill_forward_last_row():
    # The C oracle's attention forward is an independent implementation. Its last window
    # row (position n - 1) sees every key, so a decode query equal to that row over the
    # full, uncompressed cache must give the same output and logsumexp.
    rng = np.random.default_rng(4)
    L, S, Hq, Hkv, d, W = 2, 2, 8, 2, 64, 4
    lens = [37, 90]
    cu = np.array([0, lens[0], lens[0] + lens[1]], dtype=np.int64)
    N = int(cu[-1])
    qw = bf16_bits(rng.standard_normal((L, S, Hq, W, d)) * 1.5)
    k = bf16_bits(rng.standard_normal((L, Hkv, N, d)))
    v = bf16_bits(rng.standard_normal((L, Hkv, N, d)))
    ref = oracle.scores(qw, k, v, num_seqs=S, num_layers=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, window=W,
                        cu_seqlens=cu, want_rows=True)
    # packed cache holding every position, segment order u = (l*S + s)*Hkv + g
    rows_k, rows_v, off = [], [], [0]
    for l in range(L):
        for s in range(S):
            for g in range(Hkv):
                rows_k.append(k[l, g, cu[s]:cu[s + 1]])
                rows_v.append(v[l, g, cu[s]:cu[s + 1]])
                off.append(off[-1] + lens[s])
    kc, vc = np.concatenate(rows_k), np.concatenate(rows_v)
    qd = np.ascontiguousarray(qw[:, :, :, W - 1, :])
    out, lse = oracle.decode_attention(qd, kc, vc, np.array(off), num_layers=L, num_seqs=S, num_q_heads=Hq,
                                       num_kv_heads=Hkv)
    a = ref["a"].reshape(L, S, Hq, W, d)[:, :, :, W - 1]
    rl = ref["lse"].reshape(L, S, Hq, W)[:, :, :, W - 1]
    np.testing.assert_allclose(out, a, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


def test_row_order_within_a_segment_and_segment_placement_do_not_matter():
    rng = np.random.default_rng(5)
    L, S, Hq, Hkv, d = 2, 1, 6, 3, 32
    lens = [4, 9, 1, 30, 7, 2]
    q, k, v, off = ragged(rng, L, S, Hq, Hkv, d, lens)
    kw = dict(num_layers=L, num_seqs=S, num_q_heads=Hq, num_kv_heads=Hkv)
    out, lse = oracle.decode_attention(q, k, v, off, **kw)
    # shuffle rows inside every segment
    perm = np.concatenate([off[u] + rng.permutation(lens[u]) for u in range(len(lens))])
    out2, lse2 = oracle.decode_attention(q, k[perm], v[perm], off, **kw)
    np.testing.assert_allclose(out2, out, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14, atol=1e-14)
    # a different query head's output changes when its own segment changes, no other does
    k3 = k.copy()
    k3[off[4]:off[5]] = bf16_bits(rng.standard_normal((lens[4], d)))
    out3, _ = oracle.decode_attention(q, k3, v, off, **kw)
    G = Hq // Hkv
    changed = [(l, h) for l in range(L) for h in range(Hq) if not np.array_equal(out3[l, 0, h], out[l, 0, h])]
    assert changed == [(1, h) for h in range(1 * G, 2 * G)]  # unit 4 = layer 1, KV head 1


def test_empty_segment_is_rejected():
    q = np.zeros((1, 1, 1, 8), dtype=np.uint16)
    k = np.zeros((0, 8), dtype=np.uint16)
    with pytest.raises(ValueError):
        oracle.decode_attention(q, k, k, np.array([0, 0]), num_layers=1, num_seqs=1, num_q_heads=1, num_kv_heads=1)
