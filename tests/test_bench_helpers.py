"""bench.py's host-side helpers on the CPU: nearest-rank percentiles, the measured-traffic
lookup that is dropped once the gather's source changes, workload descriptions, and the
one-GPU guard.  No GPU, no torch import."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from kv_cache_eviction_05_amd import configs  # noqa: E402


def test_percentiles_nearest_rank():
    xs = [5.0, 1.0, 4.0, 2.0, 3.0, 10.0, 7.0, 6.0, 9.0, 8.0, 11.0]
    p = bench.percentiles(xs)
    assert (p["p10"], p["p50"], p["p90"]) == (2.0, 6.0, 10.0)
    assert bench.percentiles([3.0]) == {"p10": 3.0, "p50": 3.0, "p90": 3.0}


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    good = tmp_path / "traffic.json"
    entry = {"source_sha256_16": bench.source_hash(bench.COMPACT_SRC), "bytes_per_launch": 123.0}
    good.write_text(json.dumps({"workloads": {"batch": entry}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.traffic_for("batch") == 123.0
    assert bench.traffic_for("paged") is None          # not measured
    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps({"workloads": {"batch": dict(entry, source_sha256_16="0" * 16)}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.traffic_for("batch") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for("batch") is None


def write_counters(path, counter, rows):
    """A rocprofv3 counter_collection.csv with (dispatch, kernel, KiB) rows."""
    head = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,"
            "Kernel_Id,Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,"
            "Accum_VGPR_Count,SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp")
    lines = [head] + [f'{d},{d},"Agent 1",1,1,1,256,1,"{k}",256,0,0,8,0,8,"{counter}",{v},0,1'
                      for d, k, v in rows]
    path.write_text("\n".join(lines) + "\n")


def test_summarize_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    """The copy's counters give the scale factors (4 GiB copied: FETCH reads half, WRITE all);
    a workload's gather bytes per launch are the mean over its gather dispatches, scaled, and
    other kernels of the run are left out."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "t.json"))
    gib4 = 4 * 1024 * 1024  # KiB
    f, w = tmp_path / "cf.csv", tmp_path / "cw.csv"
    write_counters(f, "FETCH_SIZE", [(d, "__amd_rocclr_copyBuffer", gib4 / 2) for d in (1, 2, 3)] +
                   [(9, "__amd_rocclr_copyBuffer", 100.0)])   # a small set-up fill, ignored
    write_counters(w, "WRITE_SIZE", [(d, "__amd_rocclr_copyBuffer", gib4) for d in (1, 2, 3)])
    bench.summarize_traffic("copy", str(f), str(w))
    cal = json.load(open(tmp_path / "t.json"))["copy_calibration"]
    assert abs(cal["fetch_scale"] - 2.0) < 1e-12 and abs(cal["write_scale"] - 1.0) < 1e-12
    write_counters(f, "FETCH_SIZE", [(3, "void kvevict::compact_list_kernel<16>(x)", 1000.0),
                                     (5, "void kvevict::compact_list_kernel<16>(x)", 1002.0),
                                     (4, "draw_select_kernel", 7.0)])
    write_counters(w, "WRITE_SIZE", [(3, "void kvevict::compact_list_kernel<16>(x)", 2000.0),
                                     (5, "void kvevict::compact_list_kernel<16>(x)", 2000.0)])
    bench.summarize_traffic("batch", str(f), str(w))
    e = json.load(open(tmp_path / "t.json"))["workloads"]["batch"]
    assert e["dispatches"] == [2, 2]
    assert e["bytes_per_launch"] == 1024 * (2.0 * 1001.0 + 2000.0)
    assert bench.traffic_for("batch") == e["bytes_per_launch"]


def test_every_workload_is_described_with_its_sizes():
    for name, cfg in configs.ALL.items():
        text = bench.describe(cfg)
        assert text.startswith(name + ":"), text
        assert f"n={cfg.n}" in text and f"D={cfg.D}" in text, text


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
