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
    """Recorded counters are reported only while the decode/merge sources and the split planner
    hash as they did when the counters were taken."""
    sys.path.insert(0, ROOT)
    import bench
    assert "quantized_kv_cache_decode_amd/csrc/api.hip" in bench.KERNEL_SOURCES      # the split plan
    rec = {"kernel_source_sha256": bench.kernel_source_hash(),
           "workloads": {"w": {"bytes_per_call": 12345}}}
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.recorded_traffic("w") == 12345
    assert bench.recorded_traffic("other") is None
    p.write_text(json.dumps(dict(rec, kernel_source_sha256="0" * 64)))
    assert bench.recorded_traffic("w") is None


def test_committed_traffic_record_names_its_sources():
    """The committed record carries the source hash it was taken under (reported only while
    that hash is current)."""
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    assert len(rec["kernel_source_sha256"]) == 64
    for name, r in rec["workloads"].items():
        assert r["bytes_per_call"] >= r["algorithmic_bytes"] * 0.9, name


def test_bench_arguments_default_to_one_gpu_and_whole_counts():
    sys.path.insert(0, ROOT)
    import bench
    a = bench.parse([])
    assert a.gpus == 1 and a.workload == 1 and a.path == "step" and a.steps >= 1 and a.warmup >= 0
    a = bench.parse(["--steps", "20", "--warmup", "5"])
    assert (a.steps, a.warmup) == (20, 5)
