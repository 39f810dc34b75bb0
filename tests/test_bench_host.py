"""Host-side contract of bench.py (CPU): one GPU only, and the roofline/traffic helpers."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_follow_the_formats():
    """Packed bytes per token and KV head: 50 (turbo3), 66 (turbo4), 256 (fp16 K) per side."""
    sys.path.insert(0, ROOT)
    import bench
    from synth import get_workload
    from synth.gen import context_lengths
    w = get_workload(1)                                  # turbo3 / turbo3, 8192 tokens, 4 KV heads
    assert bench.algorithmic_bytes(w, context_lengths(w, 0)) == 8192 * 4 * 100
    w = get_workload(2)                                  # fp16 K + turbo4 V, 16384 tokens, 4 KV heads
    assert bench.algorithmic_bytes(w, context_lengths(w, 0)) == 16384 * 4 * (256 + 66)


def test_recorded_traffic_is_keyed_to_the_kernel_sources(tmp_path, monkeypatch):
    """The committed counters are reported only while the decode/merge sources hash as recorded."""
    sys.path.insert(0, ROOT)
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    name = next(iter(rec["workloads"]))
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
    assert bench.recorded_traffic(name) == rec["workloads"][name]["bytes_per_call"]
    stale = dict(rec, kernel_source_sha256="0" * 64)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.recorded_traffic(name) is None
