"""bench.py on the CPU: the one-GPU refusal and the traffic summaries' source-hash check."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_used_only_for_the_current_sources(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "a" * 16)
    assert bench.load_traffic("some_workload") is None                      # no summary
    path = tmp_path / "profiles" / "tree_attention_some_workload_traffic.json"
    rec = {"workload": "some_workload", "source_hash": "0" * 16, "bytes_per_launch": 123}
    path.write_text(json.dumps(rec))
    assert bench.load_traffic("some_workload") is None                      # taken on other sources
    rec["source_hash"] = "a" * 16
    path.write_text(json.dumps(rec))
    assert bench.load_traffic("some_workload")["bytes_per_launch"] == 123
