"""Host-side parts of bench.py: the one-GPU guard and the lookup of recorded HBM traffic."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_before_touching_a_device():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr)


def test_recorded_traffic_is_reported_only_for_the_sources_it_was_taken_on():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    for key in ("prefill_bf16_kernel", "decode_bf16_kernel"):
        e = t[key]
        assert e["bytes_per_launch"] == e["bytes_read"] + e["bytes_written"] or \
            abs(e["bytes_per_launch"] - e["bytes_read"] - e["bytes_written"]) <= 1
        assert bench.traffic_for(key, e["source_sha256"]) == e["bytes_per_launch"]
        assert bench.traffic_for(key, "0" * 64) is None
    assert bench.traffic_for("no_such_kernel", "0" * 64) is None


def test_source_hash_covers_the_kernel_sources():
    h = bench.source_hash(bench.PREFILL_SOURCES)
    assert len(h) == 64 and h != bench.source_hash(bench.DECODE_SOURCES)
