"""Calls on separate streams: the library keeps no state between calls (every buffer is the
caller's), so two pipelines enqueued on two streams at once must give the same bits as the
same pipelines run one after the other on the default stream (every sum has a fixed order).
Both streams have the default priority."""
import numpy as np
import pytest
import torch

from kv_cache_eviction_kvscore_amd import pipeline, synth
from kv_cache_eviction_kvscore_amd.configs import WORKLOADS, small_variant

from parity import say

pytestmark = pytest.mark.gpu

KEYS = ("a", "lse", "jstar", "dom", "score", "kept", "k_out", "v_out")


def _setup(w):
    data = synth.generate(w, "cuda")
    prob = pipeline.problem_for(w, data["k"], data["v"])
    return data, prob, pipeline.workload_budgets(w)


def _bits(t):
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().copy()


def _snapshot(pipe):
    out = pipe.outputs()
    return {k: _bits(out[k]) for k in KEYS}


def _same(x, y, what):
    for k in KEYS:
        assert x[k].dtype == y[k].dtype and x[k].shape == y[k].shape, (what, k)
        assert np.array_equal(x[k].view(np.uint8), y[k].view(np.uint8)), f"{what}: {k} differs"


def test_two_problems_on_two_streams():
    wa = WORKLOADS[2]
    wb = small_variant(WORKLOADS[5], num_layers=2, seqlens=(9000, 4100, 2000, 1500))
    say(f"[streams] {wa.name} and {wb.name}")
    (da, pa, ba), (db, pb, bb) = _setup(wa), _setup(wb)
    torch.cuda.synchronize()
    # one after the other, default stream
    ref_a = pipeline.Pipeline(pa, ba)
    ref_a.run(da["q"], da["k"], da["v"])
    ref_b = pipeline.Pipeline(pb, bb)
    ref_b.run(db["q"], db["k"], db["v"])
    torch.cuda.synchronize()
    want_a, want_b = _snapshot(ref_a), _snapshot(ref_b)
    # at once: each call of one pipeline enqueued between the calls of the other
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    pa2, pb2 = pipeline.Pipeline(pa, ba), pipeline.Pipeline(pb, bb)
    torch.cuda.synchronize()
    pa2.attn(da["q"], da["k"], da["v"], sa)
    pb2.attn(db["q"], db["k"], db["v"], sb)
    pa2.scores(da["q"], da["k"], da["v"], sa)
    pb2.scores(db["q"], db["k"], db["v"], sb)
    pb2.select(db["k"], db["v"], sb)
    pa2.select(da["k"], da["v"], sa)
    torch.cuda.synchronize()
    _same(_snapshot(pa2), want_a, wa.name)
    _same(_snapshot(pb2), want_b, wb.name)


def test_one_problem_twice_at_once():
    w = small_variant(WORKLOADS[3], num_layers=4)
    data, prob, budgets = _setup(w)
    torch.cuda.synchronize()
    ref = pipeline.Pipeline(prob, budgets)
    ref.run(data["q"], data["k"], data["v"])
    torch.cuda.synchronize()
    want = _snapshot(ref)
    streams = [torch.cuda.Stream() for _ in range(3)]
    pipes = [pipeline.Pipeline(prob, budgets) for _ in streams]
    torch.cuda.synchronize()
    for p, s in zip(pipes, streams):
        p.run(data["q"], data["k"], data["v"], s)
    torch.cuda.synchronize()
    for i, p in enumerate(pipes):
        _same(_snapshot(p), want, f"{w.name} copy {i}")
    say(f"[streams] {w.name}: three concurrent runs equal the sequential one bit for bit")
