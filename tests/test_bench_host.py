"""Host-side logic of bench.py, on the CPU: the algorithmic work figures its roofline entry is
built from, the bound it picks, and the summaries it makes of rocprofv3 counter output
(per-dispatch means, shader clock, HBM bytes per launch), on synthetic counter files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from kv_cache_eviction_kvscore_amd.configs import WORKLOADS, small_variant  # noqa: E402


def _visible_pairs_brute(w):
    """(row, key) pairs by enumeration: row t of the window (t = 0 .. W-1) of a sequence of n
    tokens attends to keys 0 .. n - W + t, for every query head of every layer."""
    total = 0
    for n in w.seqlens:
        for t in range(w.window):
            total += n - w.window + t + 1
    return total * w.num_layers * w.num_q_heads


@pytest.mark.parametrize("wid", [1, 2, 5])
def test_pairs_match_enumeration(wid):
    w = WORKLOADS[wid]
    if wid == 5:  # keep the enumeration small: same structure, shorter sequences
        w = small_variant(w, num_layers=2, seqlens=(700, 333, 64, 65))
    assert bench.algorithmic_work(w, 0, 1)["pairs"] == _visible_pairs_brute(w)


def test_headline_workload_figures():
    """llama8b_32layer_n128k: 8.59e9 visible pairs, 4d bytes of K and V per (token, KV head,
    layer) triple and 4d FLOP per pair for each MFMA pass."""
    w = WORKLOADS[4]
    work = bench.algorithmic_work(w, budgets_rows=0, tq=1)
    pairs = work["pairs"]
    assert pairs == 32 * 32 * (64 * (131072 - 64) + 64 * 65 // 2)
    triples = 32 * 8 * 131072
    rows = 32 * 32 * 64
    assert work["attn_fwd"]["flop"] == 4 * 128 * pairs
    assert work["attn_fwd"]["bytes"] == 4 * 128 * triples + rows * 128 * 2 + rows * (128 * 4 + 12)
    assert work["score"]["bytes"] == 4 * 128 * triples + rows * 128 * 2 + rows * (128 * 2 + 12) + 4 * triples
    assert work["topk"]["bytes"] == 4 * triples


def test_bound_of_follows_the_ridge():
    ridge = bench.PEAK_BF16_TFLOPS * 1e12 / (bench.PEAK_HBM_GBS * 1e9)  # FLOP per byte
    assert bench.bound_of({"flop": 0, "bytes": 10}) == "hbm"
    assert bench.bound_of({"flop": int(0.9 * ridge * 1e6), "bytes": int(1e6)}) == "hbm"
    assert bench.bound_of({"flop": int(1.1 * ridge * 1e6), "bytes": int(1e6)}) == "mfma"
    # the two MFMA passes of the headline workload sit just below the ridge
    work = bench.algorithmic_work(WORKLOADS[4], 0, 1)
    assert bench.bound_of(work["score"]) == "hbm" and bench.bound_of(work["attn_fwd"]) == "hbm"


FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_counters(folder, rows):
    """rows: (dispatch id, kernel name, counter, value, start ns, end ns)"""
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "pmc_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=FIELDS)
        wr.writeheader()
        for did, name, counter, value, t0, t1 in rows:
            wr.writerow({k: 0 for k in FIELDS} | {"Correlation_Id": did, "Dispatch_Id": did, "Kernel_Name": name,
                                                   "Counter_Name": counter, "Counter_Value": value,
                                                   "Start_Timestamp": t0, "End_Timestamp": t1})


def test_counters_summary_and_clock(tmp_path):
    k = "void kvs::(anonymous namespace)::score_kernel<128, 0, 1>(kvs::Dev, ...)"
    # two dispatches: 1.0e6 and 1.2e6 cycles (x 8 XCDs) over 0.5 ms and 0.6 ms: 2.0 GHz each
    rows = []
    for did, cyc, t0, dur in ((10, 1.0e6, 1_000_000, 500_000), (20, 1.2e6, 9_000_000, 600_000)):
        rows.append((did, k, "GRBM_GUI_ACTIVE", 8 * cyc, t0, t0 + dur))
        rows.append((did, k, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 0.4 * cyc, t0, t0 + dur))
        rows.append((did, k, "SQ_ACTIVE_INST_VALU", 1024 * 0.6 * cyc / 4, t0, t0 + dur))
        rows.append((did, k, "SQ_INSTS_VALU", 500.0, t0, t0 + dur))
        rows.append((did, k, "SQ_INSTS_MFMA", 100.0, t0, t0 + dur))
    rows.append((30, "other_kernel", "GRBM_GUI_ACTIVE", 1.0, 0, 10))  # not a kernel asked for
    _write_counters(str(tmp_path / "a"), rows)
    out = bench.counters_from([str(tmp_path / "a")])
    assert set(out) == {"score_kernel"}
    s = out["score_kernel"]
    assert s["dispatches"] == 2
    assert s["counters"]["GRBM_GUI_ACTIVE"] == pytest.approx(8 * 1.1e6)
    d = s["derived"]
    assert d["clock_ghz"] == pytest.approx(2.0)
    assert d["duration_ms"] == pytest.approx(0.55)
    assert d["mfma_busy_frac"] == pytest.approx(0.4)
    assert d["valu_active_frac"] == pytest.approx(0.6)
    assert d["valu_non_mfma_insts"] == pytest.approx(400.0)


def test_traffic_scaled_by_the_copy_kernel(tmp_path):
    """Counter KiB are scaled by the copy's known bytes: here the copy of 64 MiB reads 32 MiB of
    FETCH_SIZE and 64 MiB of WRITE_SIZE, so fetch counts twice and write once."""
    neg = "void at::native::vectorized_elementwise_kernel<neg_kernel...>"
    sk = "void kvs::(anonymous namespace)::score_kernel<128, 0, 1>(kvs::Dev, ...)"
    sp = "void kvs::(anonymous namespace)::score_prep_kernel<128>(...)"
    _write_counters(str(tmp_path / "f"), [(1, neg, "FETCH_SIZE", 32 * 1024, 0, 1), (2, sk, "FETCH_SIZE", 1000.0, 0, 1),
                                          (3, sp, "FETCH_SIZE", 24.0, 0, 1)])
    _write_counters(str(tmp_path / "w"), [(1, neg, "WRITE_SIZE", 64 * 1024, 0, 1), (2, sk, "WRITE_SIZE", 10.0, 0, 1),
                                          (3, sp, "WRITE_SIZE", 6.0, 0, 1)])
    out = str(tmp_path / "traffic.json")
    rec = bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"), out, "wl", 64)
    assert rec["score"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["score"]["write_scale"] == pytest.approx(1.0)
    assert rec["score"]["fetch_bytes"] == 2 * 1024 * (1000 + 24)
    assert rec["score"]["write_bytes"] == 1024 * (10 + 6)
    assert rec["score"]["bytes_per_launch"] == rec["score"]["fetch_bytes"] + rec["score"]["write_bytes"]
    assert rec["topk"]["bytes_per_launch"] == 0
    with open(out) as f:
        assert json.load(f)["wl"]["score"] == rec["score"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
