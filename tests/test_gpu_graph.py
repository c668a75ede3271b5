"""The whole pipeline captured in a HIP graph: the library's calls only launch kernels on the
given stream (no allocation, copy, fill or synchronisation), so one step can be captured once
and replayed. Every replay, with eager work and synchronisations between the replays, must
give the bits of an eager run, and a replay after the inputs are rewritten in place must
follow the new inputs."""
import numpy as np
import pytest
import torch

from kv_cache_eviction_kvscore_amd import pipeline, synth
from kv_cache_eviction_kvscore_amd.configs import WORKLOADS, small_variant

from parity import say

pytestmark = pytest.mark.gpu

KEYS = ("a", "lse", "jstar", "dom", "score", "kept", "k_out", "v_out")


def _snapshot(pipe):
    out = pipe.outputs()
    snap = {}
    for k in KEYS:
        t = out[k].detach().contiguous()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        snap[k] = t.cpu().numpy().copy()
    return snap


def _same(x, y, what):
    for k in KEYS:
        assert np.array_equal(x[k].view(np.uint8), y[k].view(np.uint8)), f"{what}: {k} differs"


def _eager(prob, budgets, q, k, v, heads=False):
    p = pipeline.Pipeline(prob, budgets, heads=heads)
    p.run(q, k, v)
    torch.cuda.synchronize()
    return _snapshot(p)


# the joint head select (heads=True) keeps a counter and lists in its workspace: every replay
# must start them afresh
@pytest.mark.parametrize("wid,heads", [(2, False), (5, False), (2, True)])
def test_pipeline_graph_replays(wid, heads):
    w = WORKLOADS[wid] if wid == 2 else small_variant(WORKLOADS[5], num_layers=2, seqlens=(6000, 3000, 1500, 1300))
    data = synth.generate(w, "cuda")
    q, k, v = data["q"], data["k"], data["v"]
    prob = pipeline.problem_for(w, k, v)
    budgets = pipeline.workload_budgets(w)
    torch.cuda.synchronize()
    want = _eager(prob, budgets, q, k, v, heads)

    pipe = pipeline.Pipeline(prob, budgets, heads=heads)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one run off the capture, as torch recommends before capturing
        pipe.run(q, k, v)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pipe.run(q, k, v)
    torch.cuda.synchronize()
    for rep in range(3):
        for key in ("score", "k_out", "kept"):  # clear outputs eagerly so a replay must rewrite them
            pipe.outputs()[key].zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(_snapshot(pipe), want, f"{w.name} replay {rep}")
        _eager(prob, budgets, q, k, v, heads)  # eager work between the replays

    # new inputs written into the captured tensors: the replay follows them
    q2 = (torch.randn(q.shape, generator=torch.Generator(device="cuda").manual_seed(7), device="cuda") * 1.5)
    q.copy_(q2.to(torch.bfloat16))
    torch.cuda.synchronize()
    want2 = _eager(prob, budgets, q, k, v, heads)
    graph.replay()
    torch.cuda.synchronize()
    _same(_snapshot(pipe), want2, f"{w.name} replay with new queries")
    say(f"[graph] {w.name}: 4 replays equal eager runs bit for bit")
