"""Host-side checks of bench.py's contract (no GPU): the one-GPU refusal and
the committed traffic record's guard."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode != 0
    line = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert line and "one GPU" in json.loads(line[0])["error"]


def test_traffic_record_matches_only_its_workload_and_source():
    rec = json.load(open(os.path.join(ROOT, "profiles", "gate_up_gemm_1024_traffic.json")))
    got = bench.recorded_traffic("1024")
    # the record is either current (its value) or stale (None): never another number
    assert got in (None, rec["traffic_bytes_per_launch"])
    assert bench.recorded_traffic("2048") is None
    assert bench.recorded_traffic("512") is None


def test_traffic_record_is_dropped_when_the_kernel_source_changes(tmp_path, monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "gate_up_gemm_1024_traffic.json")))
    fake = tmp_path / "profiles"
    fake.mkdir()
    src = tmp_path / "k.hip"
    src.write_text("// not the recorded source\\n")
    rec = dict(rec, kernel_source="k.hip")
    (fake / "gate_up_gemm_1024_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("1024") is None
