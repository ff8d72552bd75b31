"""Host-side contract of bench.py (no GPU): the one-GPU refusal, the traffic entry keyed on the
kernel source, and the CPU-baseline record."""

import json
import os
import subprocess
import sys

import bench
from synth import make_inputs, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_entry_follows_the_kernel_source(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_entry() is None  # no counter summary
    f.write_text(json.dumps({"kernel_source_hash": bench.kernel_source_hash(), "hbm_bytes_per_launch": 123.0}))
    assert bench.traffic_entry() == 123.0
    f.write_text(json.dumps({"kernel_source_hash": "0" * 16, "hbm_bytes_per_launch": 123.0}))
    assert bench.traffic_entry() is None  # counters taken on another kernel source


def test_cpu_baseline_record():
    w = workload("tiny")
    qb, kb, vb = make_inputs(w)
    rec = bench.cpu_baseline(w, qb, kb, vb, 0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s" and rec["cores"] >= 1
    assert rec["value"] > 0 and rec["seconds"] >= 0.2
    assert "query rows" in rec["sample"] and w.name in rec["sample"]
