"""bench.py on the CPU: it measures one GPU and refuses any other count before
it touches a device; its traffic lookup reports bytes only for the kernel
sources the counters were taken on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr + r.stdout
    assert not r.stdout.strip().startswith("{")  # no benchmark line


def test_traffic_lookup_follows_the_source_hash(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    stored = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    kind = "qgemm_q4k_160x24576x4096"
    monkeypatch.setattr(bench, "source_hash", lambda: stored[kind]["source_hash"])
    assert bench.stored_traffic(kind) == stored[kind]["bytes_per_launch"]
    monkeypatch.setattr(bench, "source_hash", lambda: "0" * 16)
    assert bench.stored_traffic(kind) is None
    assert bench.stored_traffic("no such kernel") is None
