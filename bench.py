"""Benchmark: the whole eviction-scoring hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--no-cpu-baseline]

One step = kvscore_attn_fwd + kvscore_score + kvscore_merge + kvscore_topk +
kvscore_compact over every (layer, KV head) of the workload, inputs already resident in
HBM. The layer budgets (host map, O(L)) depend only on the profile and total, so they
are computed once before timing and their host time is reported separately. Prints one
JSON line (rank 0): whole-job scored prompt tokens/s, a roofline entry for the dominant
kernel, per-call timings, and the CPU oracle timed on a bounded sample of units of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "scored prompt tokens/sec (score+top-k+compact) at n=128K; % bf16 MFMA / HBM peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
CALLS = ("attn_fwd", "score", "merge", "topk", "compact")
# the kernel files whose counters a committed traffic record describes
KERNEL_SOURCES = {"score": "score.hip", "attn_fwd": "attn_fwd.hip", "compact": "compact.hip",
                  "topk": "topk.hip", "merge": "merge.hip", "decode": "decode.hip"}
# the kernels (by name fragment) that make up each call, for counter records
CALL_KERNELS = {"attn_fwd": ("fwd_partial_kernel", "fwd_combine_kernel"), "score": ("score_prep_kernel", "score_kernel"),
                "merge": ("merge_sum_kernel", "merge_isolated_kernel"), "topk": ("topk_kernel",), "compact": ("compact_kernel",),
                "decode": ("decode_partial_kernel", "decode_combine_kernel")}


def bound_of(work: dict) -> str:
    """The roofline that binds a call: HBM when its algorithmic bytes take longer at peak bandwidth
    than its FLOP at the bf16 matrix peak (arithmetic intensity below the ~312 FLOP/B ridge)."""
    if not work["flop"]:
        return "hbm"
    return "hbm" if work["bytes"] / PEAK_HBM_GBS / 1e9 >= work["flop"] / PEAK_BF16_TFLOPS / 1e12 else "mfma"


def algorithmic_work(w, budgets_rows: int, tq: int):
    """Per-call algorithmic FLOP and HBM bytes for one step (the method's own work)."""
    L, Hkv, G, d, W = w.num_layers, w.num_kv_heads, w.group, w.head_dim, w.window
    # (row, key) pairs with the key visible to the row: row i of a unit sees n - W + i + 1 keys
    pairs = sum(L * Hkv * G * (W * (n - W) + W * (W + 1) // 2) for n in w.seqlens)
    N = w.total_tokens
    rows = L * w.num_seqs * w.num_q_heads * W
    kv = 2 * L * Hkv * N * d * 2  # K and V, bf16
    q = rows * d * 2
    th = L * Hkv * N  # (token, KV head, layer) triples
    return {
        "attn_fwd": {"flop": 4 * d * pairs, "bytes": kv + q + rows * (d * 4 + 12)},
        "score": {"flop": 4 * d * pairs, "bytes": kv + q + rows * (d * 2 + 12) + 4 * tq * th},
        # one query tile: merged in place, only the isolated terms (read j*, dom; one score
        # read and written per row); else the tile rows are summed into the score rows
        "merge": {"flop": 0, "bytes": (4 * tq * th + 4 * th + rows * 8) if tq > 1 else rows * 16},
        "topk": {"flop": 0, "bytes": 4 * th + 4 * budgets_rows},
        "compact": {"flop": 0, "bytes": budgets_rows * (2 * 2 * d * 2 + 4)},
        "pairs": pairs,
    }


def source_digest(name: str) -> str:
    path = os.path.join(ROOT, "kv_cache_eviction_kvscore_amd", "csrc", KERNEL_SOURCES[name])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def committed_traffic(name: str, workload: str):
    """HBM traffic per launch from the committed counter record, if it still describes this kernel."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    ent = rec.get(workload, {}).get(name)
    if not ent or ent.get("source_sha256_16") != source_digest(name):
        return None
    return ent.get("bytes_per_launch")


def traffic_from(fetch_dir: str, write_dir: str, out_path: str, workload: str, copy_mib: int) -> dict:
    """HBM bytes per launch of each call from two rocprofv3 --pmc runs of this script (one with
    FETCH_SIZE, one with WRITE_SIZE, both with --calibrate-copy-mib). Each counter is scaled by what it
    reads for the calibration kernel (torch.neg over copy_mib MiB: that many bytes read and written)."""
    import csv
    import glob

    def per_dispatch(d: str, counter: str) -> dict:
        acc = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                if row["Counter_Name"] != counter:
                    continue
                name = row["Kernel_Name"]
                key = "neg" if "neg_kernel" in name else next(
                    (k for ks in CALL_KERNELS.values() for k in ks if k in name), None)
                if key is None:
                    continue
                acc.setdefault(key, {}).setdefault(row["Dispatch_Id"], 0.0)
                acc[key][row["Dispatch_Id"]] += float(row["Counter_Value"])
        return {k: sum(v.values()) / len(v) for k, v in acc.items()}  # KiB per dispatch

    fetch, write = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")
    nbytes = copy_mib * (1 << 20)
    fs, ws = nbytes / (fetch["neg"] * 1024), nbytes / (write["neg"] * 1024)
    rec = {}
    for call, ks in CALL_KERNELS.items():
        fb = fs * 1024 * sum(fetch.get(k, 0.0) for k in ks)
        wb = ws * 1024 * sum(write.get(k, 0.0) for k in ks)
        rec[call] = {"source_sha256_16": source_digest(call), "fetch_bytes": round(fb), "write_bytes": round(wb),
                     "bytes_per_launch": round(fb + wb), "fetch_scale": round(fs, 4), "write_scale": round(ws, 4)}
    allrec = {}
    if os.path.exists(out_path):
        with open(out_path) as f:
            allrec = json.load(f)
    allrec[workload] = rec
    with open(out_path, "w") as f:
        json.dump(allrec, f, indent=1)
    return rec


def counters_from(dirs, kernels=("score_kernel", "fwd_partial_kernel")) -> dict:
    """Per-dispatch means of rocprofv3 --pmc counters (csv output folders of runs of this script),
    for each kernel whose name contains one of ``kernels``, plus derived figures. SQ time counters
    are in quad-cycles summed over the SIMDs' waves; GRBM_GUI_ACTIVE is summed over the 8 XCDs;
    SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES are cycles summed over the 1024 SIMDs.
    The dispatches' start and end timestamps give their mean duration, and with GRBM_GUI_ACTIVE
    the mean shader clock over the kernel (cycles / duration)."""
    import csv
    import glob
    acc, dur = {}, {}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for row in csv.DictReader(open(f)):
                key = next((k for k in kernels if k in row["Kernel_Name"]), None)
                if key is None:
                    continue
                ent = acc.setdefault(key, {}).setdefault(row["Counter_Name"], {})
                did = (d, row["Dispatch_Id"])  # a counter collected in several runs is averaged over them
                ent[did] = ent.get(did, 0.0) + float(row["Counter_Value"])
                dur.setdefault(key, {})[did] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
    out = {}
    for key, cs in acc.items():
        mean = {c: sum(v.values()) / len(v) for c, v in cs.items()}
        simds, xcds = 1024, 8
        der = {}
        cyc = mean.get("GRBM_GUI_ACTIVE", 0) / xcds  # kernel duration in cycles
        if cyc:
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                der["mfma_busy_frac"] = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / simds / cyc
            if "SQ_ACTIVE_INST_VALU" in mean:
                der["valu_active_frac"] = 4 * mean["SQ_ACTIVE_INST_VALU"] / simds / cyc
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in mean:
                der["coexec_frac"] = mean["SQ_VALU_MFMA_COEXEC_CYCLES"] / simds / cyc
            clk = [cs["GRBM_GUI_ACTIVE"][k] / xcds / t for k, t in dur[key].items()
                   if k in cs["GRBM_GUI_ACTIVE"] and t > 0]
            if clk:
                der["clock_ghz"] = sum(clk) / len(clk) * 1e-9
                der["duration_ms"] = sum(dur[key].values()) / len(dur[key]) * 1e3
        if "SQ_INSTS_VALU" in mean and "SQ_INSTS_MFMA" in mean:
            der["valu_non_mfma_insts"] = mean["SQ_INSTS_VALU"] - mean["SQ_INSTS_MFMA"]
        out[key] = {"counters": mean, "derived": der, "dispatches": max(len(v) for v in cs.values())}
    return out


def cpu_model() -> str:
    """The host CPU's model name (first entry of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, data, budgets, target_s: float, max_units: int):
    """The oracle (as it stands) on a bounded sample of units: score + top-k + gather."""
    import numpy as np
    import oracle
    from kv_cache_eviction_kvscore_amd import synth
    cu = w.cu_seqlens()
    U = w.num_layers * w.num_seqs * w.num_kv_heads
    G, W, d = w.group, w.window, w.head_dim
    R = G * W
    rng = np.random.default_rng(12345)
    order = rng.permutation(U)
    spent, done, tokens_equiv = 0.0, 0, 0.0
    for u in order[:max_units]:
        g = u % w.num_kv_heads
        s = (u // w.num_kv_heads) % w.num_seqs
        l = u // (w.num_kv_heads * w.num_seqs)
        n = w.seqlens[s]
        q = synth.bf16_bits(data["q"].reshape(-1, d)[u * R:(u + 1) * R]).reshape(1, 1, G, W, d)
        k = synth.bf16_bits(data["k"][l, g, cu[s]:cu[s + 1]]).reshape(1, 1, n, d)
        v = synth.bf16_bits(data["v"][l, g, cu[s]:cu[s + 1]]).reshape(1, 1, n, d)
        t0 = time.perf_counter()
        sc = oracle.scores(q, k, v, num_seqs=1, num_layers=1, num_q_heads=G, num_kv_heads=1, head_dim=d,
                           window=W, cu_seqlens=[0, n])["score"][0, 0]
        kept = oracle.kept_positions(sc, n, W, int(budgets[s][l]))
        oracle.gather(k.reshape(n, d), v.reshape(n, d), kept)
        spent += time.perf_counter() - t0
        done += 1
        # this unit's share of the whole job's prompt tokens
        tokens_equiv += n / (w.num_layers * w.num_kv_heads)
        if spent >= target_s:
            break
    threads = oracle.num_threads()
    return {"value": tokens_equiv / spent, "unit": "tokens/s", "cores": threads, "threads": threads,
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} of {U} (layer, sequence, KV head) units of {w.name}, fp64 oracle score + full-sort "
                      f"top-k + gather, {spent:.1f} s; tokens/s = the units' share of the prompt tokens / time"}


def time_decode(w, prob, pipe, steps: int) -> dict:
    """Decode attention of one new token per query head over the packed ragged cache the step
    just compacted (not part of the step). Algorithmic bytes: every packed K and V row once,
    the queries, the fp32 outputs and logsumexps."""
    import numpy as np
    import torch
    from kv_cache_eviction_kvscore_amd import api
    L, S, Hq, d = w.num_layers, w.num_seqs, w.num_q_heads, w.head_dim
    g = torch.Generator().manual_seed(2024)
    q = torch.randn((L, S, Hq, d), generator=g).to(torch.bfloat16).cuda()
    out = torch.empty((L, S, Hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((L, S, Hq), dtype=torch.float32, device="cuda")
    off_dev = pipe.head_off if pipe.heads else pipe.seg_off  # the heads' own segments in --heads mode
    off = off_dev.cpu().numpy()
    ws = torch.empty(api.decode_workspace_size(prob, off), dtype=torch.uint8, device="cuda")
    k_out, v_out = pipe.k_out[:pipe.kept_rows], pipe.v_out[:pipe.kept_rows]

    def run():
        api.decode_attn(prob, q, k_out, v_out, off, off_dev, out, lse, ws)

    for _ in range(3):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nq = L * S * Hq
    nbytes = 2 * pipe.kept_rows * d * 2 + nq * d * 2 + nq * (d + 1) * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "cache_rows": pipe.kept_rows, "bytes": nbytes, "gbs": round(gbs, 1),
            "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bound": "hbm",
            "what": "one new token per query head over the packed ragged cache the step compacted "
                    "(kvscore_decode_attn, partial + combine), mean of the timed launches"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the decode-attention measurement over the step's packed cache")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="also run a plain elementwise kernel (torch.neg) over this many MiB of fp32, three "
                         "times: it reads and writes exactly that many bytes, which calibrates HBM counters")
    ap.add_argument("--mode", choices=("l2", "sq", "attn"), default="l2",
                    help="score: DropKV L2 shift (default), its squared variant, or the attention sum")
    ap.add_argument("--pool", type=int, default=1,
                    help="rank candidates by the score max-pooled over this odd window (1 = off)")
    ap.add_argument("--sinks", type=int, default=0, help="first tokens always kept (attention sinks)")
    ap.add_argument("--heads", action="store_true",
                    help="head budgets chosen jointly over each layer's KV heads (kvscore_topk_heads)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no run: turn two rocprofv3 --pmc output folders (FETCH_SIZE, WRITE_SIZE) of this script "
                         "into HBM bytes per launch, written to --traffic-out")
    ap.add_argument("--traffic-out", default=os.path.join(ROOT, "profiles", "traffic.json"))
    ap.add_argument("--counters-from", nargs="+", metavar="DIR",
                    help="no run: per-dispatch means and derived figures of rocprofv3 --pmc output folders "
                         "(csv) of this script, for the score, forward, top-k and compaction kernels")
    args = ap.parse_args()
    if args.counters_from:
        print(json.dumps(counters_from(args.counters_from, ("score_kernel", "fwd_partial_kernel", "topk_kernel",
                                                            "compact_kernel")), indent=1))
        return
    if args.traffic_from:
        from kv_cache_eviction_kvscore_amd.configs import WORKLOADS
        rec = traffic_from(args.traffic_from[0], args.traffic_from[1], args.traffic_out, WORKLOADS[args.workload].name,
                           args.calibrate_copy_mib or 1024)
        print(json.dumps(rec, indent=1))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the path shards by (layer, KV head) units "
                                   "with no communication, but multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    from kv_cache_eviction_kvscore_amd import api, pipeline, synth
    from kv_cache_eviction_kvscore_amd.configs import WORKLOADS

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    w = WORKLOADS[args.workload]
    print(f"[bench] generating {w.name} ({w.kv_bytes() / 1e9:.2f} GB of K/V)", file=sys.stderr, flush=True)
    data = synth.generate(w, "cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    budgets = pipeline.workload_budgets(w, args.sinks)
    budget_us = (time.perf_counter() - t0) * 1e6
    mode = {"l2": api.MODE_L2, "sq": api.MODE_SQ, "attn": api.MODE_ATTN}[args.mode]
    prob = pipeline.problem_for(w, data["k"], data["v"], mode)
    pipe = pipeline.Pipeline(prob, budgets, pool=args.pool, n_sink=args.sinks, heads=args.heads)
    q, k, v = data["q"], data["k"], data["v"]
    calls = [lambda: pipe.attn(q, k, v),
             lambda: api.score(prob, q, k, v, pipe.a, pipe.lse, pipe.jstar, pipe.partial, pipe.ws_score),
             lambda: api.merge(prob, pipe.partial, pipe.jstar, pipe.dom, pipe.score),
             lambda: api.topk(prob, pipe.score, pipe.budgets, pipe.seg_off, pipe.kept, pool=args.pool,
                              n_sink=args.sinks, ws=pipe.ws_topk),
             lambda: api.compact(prob, k, v, pipe.budgets, pipe.seg_off, pipe.kept, pipe.k_out, pipe.v_out)]
    if args.heads:
        calls[3] = lambda: api.topk_heads(prob, pipe.score, pipe.budgets, pipe.seg_off, pipe.head_off, pipe.kept,
                                          pool=args.pool, n_sink=args.sinks, ws=pipe.ws_topk)
        calls[4] = lambda: api.compact_heads(prob, k, v, pipe.budgets, pipe.head_off, pipe.kept, pipe.k_out,
                                             pipe.v_out)

    if args.calibrate_copy_mib:
        src = torch.randn(args.calibrate_copy_mib * (1 << 18), device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        for j, c in enumerate(calls):
            c()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    per_call = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(args.steps)]))
                for j, name in enumerate(CALLS)}
    step_ms = float(np.mean([ev[i][0].elapsed_time(ev[i][-1]) for i in range(args.steps)]))
    ms_per_step = wall * 1e3 / args.steps
    tokens = w.total_tokens
    value = tokens / (ms_per_step / 1e3)

    work = algorithmic_work(w, pipe.kept_rows, pipe.tq)
    if args.mode == "attn":  # the attention sum streams K only and has one GEMM
        kv = w.num_layers * w.num_kv_heads * w.total_tokens * w.head_dim * 2
        work["score"]["bytes"] -= kv
        work["score"]["flop"] //= 2
    if args.pool > 1:  # the pooled keys: one more read of the scores and a write of the keys
        work["topk"]["bytes"] += 8 * w.num_layers * w.num_kv_heads * w.total_tokens
    kernels = {}
    for name in CALLS:
        ms = per_call[name]
        ent = {"ms": round(ms, 4)}
        if work[name]["flop"]:
            tf = work[name]["flop"] / (ms * 1e-3) / 1e12
            ent.update(tflops=round(tf, 1), frac_bf16_mfma=round(tf / PEAK_BF16_TFLOPS, 4))
        gbs = work[name]["bytes"] / (ms * 1e-3) / 1e9
        ent.update(gbs=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM_GBS, 4))
        kernels[name] = ent
    dom_name = max(CALLS, key=lambda n: per_call[n])
    if bound_of(work[dom_name]) == "mfma":
        ach = work[dom_name]["flop"] / (per_call[dom_name] * 1e-3) / 1e12
        roof = {"kernel": dom_name, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    else:
        ach = work[dom_name]["bytes"] / (per_call[dom_name] * 1e-3) / 1e9
        roof = {"kernel": dom_name, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    roof["traffic"] = committed_traffic(dom_name, w.name)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "seqlens": list(w.seqlens),
                   "num_layers": w.num_layers, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
                   "head_dim": w.head_dim, "window": w.window, "kept_rows": pipe.kept_rows,
                   "mode": args.mode.upper(), "pool": args.pool, "n_sink": args.sinks,
                   "head_budgets": "joint per layer" if args.heads else "uniform", "parallelism": "single GPU"},
        "roofline": roof,
        "kernels": kernels,
        "event_ms_per_step": round(step_ms, 4),
        # scored (token, KV head, layer) triples per second, and the rate of a caller whose prefill
        # already produced a and lse (every call but the forward)
        "triples_per_s": round(w.num_layers * w.num_kv_heads * w.total_tokens / (ms_per_step / 1e3), 1),
        "value_without_attn_fwd": round(tokens / ((step_ms - per_call["attn_fwd"]) / 1e3), 1),
        "budget_host_us": round(budget_us, 1),
        "pairs_per_step": work["pairs"],
    }
    if not args.no_decode:
        out["decode"] = time_decode(w, prob, pipe, args.steps)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on a sample of units)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, data, budgets, args.cpu_seconds, max_units=16)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
