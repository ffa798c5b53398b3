"""Host-side checks of bench.py's contract (no GPU): it refuses more than one
GPU before touching a device, and the counter-derived traffic it reports is
taken only from a profile of the current kernel source."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_traffic_record_follows_the_source():
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        recs = json.load(f)
    key = next(iter(recs))
    kernel, workload = key.rsplit(":", 1)
    rec = recs[key]
    assert bench.traffic_record(kernel, workload, rec["source_sha"]) == rec["bytes_per_launch"]
    assert bench.traffic_record(kernel, workload, "0" * 16) is None
    assert bench.traffic_record(kernel, "no_such_workload", rec["source_sha"]) is None


def test_source_sha_changes_with_the_text():
    a = bench.source_sha(["prefill.hip", "common.hpp", "args.hpp"])
    b = bench.source_sha(["prefill.hip", "common.hpp"])
    assert len(a) == 16 and a != b


def test_head_split_flop_count_matches_the_oracle_pairs():
    # the bench's closed-form pair count (its FLOP numerator) against the
    # oracle's count of each query's visible set
    import oracle
    for n, s, w in ((1, 4, 8), (300, 4, 64), (513, 0, 1), (200, 250, 0), (1000, 4, 1024)):
        assert bench.head_split_pairs(n, True, s, w) == oracle.visible_pairs(n, 0, s, w)
        assert bench.head_split_pairs(n, False, s, w) == oracle.visible_pairs(n, 1, s, w)
