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


def test_traffic_record_matches_only_its_workload_form_and_sources():
    rec = json.load(open(os.path.join(ROOT, "profiles", "gate_up_gemm_1024_lo4_traffic.json")))
    got = bench.recorded_traffic("1024", "lo4")
    # the record is either current (its value) or stale (None): never another number
    assert got in (None, rec["traffic_bytes_per_launch"])
    assert bench.recorded_traffic("2048", "lo4") is None
    assert bench.recorded_traffic("512", "lo4") is None
    for ffn in ("f16", "lo8", "pair"):  # no record for these forms
        assert bench.recorded_traffic("1024", ffn) is None


def test_traffic_record_is_dropped_when_a_kernel_source_changes(tmp_path, monkeypatch):
    rec = json.load(open(os.path.join(ROOT, "profiles", "gate_up_gemm_1024_lo4_traffic.json")))
    fake = tmp_path / "profiles"
    fake.mkdir()
    srcs = {}
    for name, sha in rec["kernel_sources"].items():
        f = tmp_path / os.path.basename(name)
        f.write_bytes(open(os.path.join(ROOT, name), "rb").read())
        srcs[os.path.basename(name)] = sha
    (fake / "gate_up_gemm_1024_lo4_traffic.json").write_text(json.dumps(dict(rec, kernel_sources=srcs)))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    current = bench.recorded_traffic("1024", "lo4")
    (tmp_path / "lores.h").write_text("// not the recorded source\n")  # one of the sources changes
    assert bench.recorded_traffic("1024", "lo4") is None
    assert current in (None, rec["traffic_bytes_per_launch"])
