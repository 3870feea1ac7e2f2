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
    keys = [k for k in t if not k.startswith("_")]
    assert keys
    for key in keys:
        kernel, workload = key.split("/")
        e = t[key]
        assert abs(e["bytes_per_launch"] - e["bytes_read"] - e["bytes_written"]) <= 1
        assert bench.traffic_for(kernel, workload, e["source_sha256"]) == e["bytes_per_launch"]
        assert bench.traffic_for(kernel, workload, "0" * 64) is None
        assert bench.traffic_for(kernel, "no_such_workload", e["source_sha256"]) is None
    assert bench.traffic_for("no_such_kernel", "qwen25_7b", "0" * 64) is None


def test_source_hash_covers_the_kernel_and_its_item_order():
    h = bench.source_hash(bench.PREFILL_SOURCES)
    assert len(h) == 64 and h != bench.source_hash(bench.DECODE_SOURCES)
    # the work-list pass and the call decide the prefill's item order, hence its HBM bytes
    assert "kev_schedule.hip" in bench.PREFILL_SOURCES and "kev_api.hip" in bench.PREFILL_SOURCES


def test_oracle_row_sample_counts_effective_flops():
    import numpy as np
    from segment_isolated_packed_amd import workloads as W
    case = W.make_prefill([3, 5], 2, 1, 16, W.F32, seed=0)
    rows, heads, f = bench._sample_pairs(case, np.random.default_rng(0), 50)
    keys = [(r - (0 if r < 3 else 3)) + 1 for r in rows]
    assert f == 4 * 16 * sum(keys)
    assert ((heads >= 0) & (heads < 2)).all()
