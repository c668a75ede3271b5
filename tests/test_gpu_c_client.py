"""The C ABI from plain C: tests/c_client/kvscore_c_client (C99, built with gcc against
include/kvscore.h and the HIP runtime's C API, no torch) runs the whole path on inputs this
test writes, in a child process. Its budgets, segment offsets, scores, kept positions and
packed cache must equal, bit for bit, what the Python binding gives on the same inputs."""
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

from kv_cache_eviction_kvscore_amd import api, pipeline, synth
from kv_cache_eviction_kvscore_amd.configs import WORKLOADS, small_variant

from parity import say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "kvscore_c_client")


def _python_path(w, data, ratio, frac, mode):
    prob = api.Problem.for_tensors(data["k"], data["v"], num_q_heads=w.num_q_heads, window=w.window,
                                   cu_seqlens=w.cu_seqlens(), mode=mode)
    L = w.num_layers
    budgets = np.stack([api.budget(np.zeros(L), ratio, float("inf"), int(np.floor(frac * L * n)), w.window, n)
                        for n in w.seqlens]).astype(np.int32)
    pipe = pipeline.Pipeline(prob, budgets)
    pipe.run(data["q"], data["k"], data["v"])
    torch.cuda.synchronize()
    return budgets, pipe.outputs()


@pytest.mark.parametrize("mode", [api.MODE_L2, api.MODE_SQ])
def test_c_client_matches_python(tmp_path, mode):
    assert os.path.exists(EXE), "tests/c_client/kvscore_c_client is not built (run the repository's build step)"
    w = small_variant(WORKLOADS[5], num_layers=2, seqlens=(3000, 1200, 700))
    data = synth.generate(w, "cuda")
    ratio, frac = 2.0, 0.2
    S, L, Hq, Hkv, d, W = w.num_seqs, w.num_layers, w.num_q_heads, w.num_kv_heads, w.head_dim, w.window
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(struct.pack("<7i", S, L, Hq, Hkv, d, W, mode))
        f.write(np.asarray(w.cu_seqlens(), dtype="<i8").tobytes())
        f.write(struct.pack("<2d", ratio, frac))
        for t in ("q", "k", "v"):
            f.write(synth.bf16_bits(data[t]).tobytes())
    say(f"[c client] {w.name} mode={mode}")
    r = subprocess.run([EXE, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"client failed ({r.returncode}): {r.stderr}"

    budgets, out = _python_path(w, data, ratio, frac, mode)
    U, N = L * S * Hkv, w.total_tokens
    raw = open(outp, "rb").read()
    pos = 0

    def take(dtype, count):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dtype, count=count, offset=pos)
        pos += a.nbytes
        return a

    c_budgets = take("<i4", S * L).reshape(S, L)
    c_off = take("<i8", U + 1)
    R = int(c_off[-1])
    c_score = take("<f4", L * Hkv * N)
    c_kept = take("<i4", R)
    c_k = take("<u2", R * d)
    c_v = take("<u2", R * d)
    assert pos == len(raw)
    assert np.array_equal(c_budgets, budgets)
    assert np.array_equal(c_off, out["seg_off"])
    assert np.array_equal(c_score.view(np.uint32), out["score"].cpu().numpy().reshape(-1).view(np.uint32))
    assert np.array_equal(c_kept, out["kept"].cpu().numpy())
    assert np.array_equal(c_k, synth.bf16_bits(out["k_out"]).reshape(-1))
    assert np.array_equal(c_v, synth.bf16_bits(out["v_out"]).reshape(-1))
    say(f"[c client] {w.name}: {R} kept rows, every output equal to the Python path's")
