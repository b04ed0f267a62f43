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
    good.write_text(json.dumps({"source_sha256_16": bench.source_hash(bench.COMPACT_SRC),
                                "bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.traffic_for(1) == 123.0
    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps({"source_sha256_16": "0" * 16, "bytes_per_launch": 123.0}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.traffic_for(1) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_for(1) is None


def test_every_workload_is_described_with_its_sizes():
    for name, cfg in configs.ALL.items():
        text = bench.describe(cfg)
        assert text.startswith(name + ":"), text
        assert f"n={cfg.n}" in text and f"D={cfg.D}" in text, text


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
