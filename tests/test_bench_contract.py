"""Host-side checks of bench.py that need no GPU: it refuses more than one GPU
with a message, every --op is a known choice, its algorithmic byte counts
follow the rows each request must read, and the committed traffic counters
are tied to the current kernel sources."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from rejection_sampling_verify_scaled_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_ops_listed_in_help():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for op in ("verify", "draft", "commit", "early-exit", "tree", "greedy"):
        assert op in r.stdout


def test_algorithmic_bytes_count_needed_rows():
    b = W.make_custom_batch(np.random.default_rng(0), W.DTYPE_BF16, 100, [2, 0, 3],
                            [1.0, 1.0, 0.0])
    # sampled: 2K + 1 rows, greedy: K + 1 rows
    assert bench.algorithmic_bytes(b) == (5 + 1 + 4) * 100 * 2


def test_early_exit_bytes_count_rows_up_to_the_stop():
    b = W.make_custom_batch(np.random.default_rng(0), W.DTYPE_F32, 10, [3, 3, 3, 0],
                            [1.0, 1.0, 0.0, 1.0])
    # sampled, stop at 1: rows 0..1 of both; sampled, all 3 accepted: 2*3 + 1;
    # greedy, stop at 2: target rows 0..2; sampled K = 0: the bonus row only
    acc = np.array([1, 3, 2, 0])
    assert bench.early_exit_bytes(b, acc) == (4 + 7 + 3 + 1) * 10 * 4


@pytest.mark.parametrize("name,sources", [("sv_verify", None),
                                          ("sv_verify_ee", bench.EE_KERNEL_SOURCES)])
def test_committed_traffic_is_tied_to_sources(name, sources):
    """A committed traffic record names the sources it was measured on and its
    summary; bench.py reports it only while those sources are unchanged (a
    stale record gives "traffic": null rather than a figure from another kernel)."""
    paths = [p for p in os.listdir(os.path.join(ROOT, "profiles"))
             if p.startswith(f"traffic_{name}_workload")]
    assert paths
    for p in paths:
        with open(os.path.join(ROOT, "profiles", p)) as f:
            rec = json.load(f)
        assert rec["kernel"] == name
        assert os.path.exists(os.path.join(ROOT, rec["summary"]))
        fresh = rec["source_sha256"] == bench.kernel_source_sha256(sources)
        got = bench.traffic_record(rec["workload"], kernel=name, sources=sources)
        if fresh:
            assert got == rec["hbm_bytes_per_launch"]
        else:
            assert got is None, f"{p} is stale but bench.py would report it"
