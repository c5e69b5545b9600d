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


def test_stream_profile_counts_block_bytes():
    """The stage trace's stream table from a synthetic trace (one tick = 1 us):
    a sampled request's 36 blocks (9 rows) store at 3 us, a greedy request's
    20 blocks with rows (5 rows; its 16 surplus groups hold none) at 5 us, a
    race workgroup lives from 0 to 9 us.  Blocks of a row add up to the row."""
    full = W.make_batch(2, 0)
    batch = W.subset_requests(full, [0, 40])  # request 0 sampled, request 40 greedy
    assert batch.temperature[0] > 0 and batch.temperature[1] == 0
    rows = []
    for b, stored in ((0, 3), (1, 5)):
        for grp in range(36):
            r = np.zeros(10, dtype=np.uint64)
            r[0] = 1 | (b << 8) | (grp << 32)
            r[1], r[2], r[3] = 100, 101, 100 + stored  # start, scalars loaded, partial stored
            rows.append(r)
    race = np.zeros(10, dtype=np.uint64)
    race[0] = 2 | (0 << 8)
    race[1], race[9] = 100, 109
    rows.append(race)
    prof = bench.stream_profile(np.stack(rows), batch, 1.0, n_windows=5)
    row_mb = batch.V * 2 / 1e6
    w = bench.STREAM_WINDOW_US
    assert prof[1, 0] == pytest.approx(9 * row_mb / w)   # [2, 4): the sampled request's rows
    assert prof[2, 0] == pytest.approx(5 * row_mb / w)   # [4, 6): the greedy request's rows
    assert prof[1, 1] == pytest.approx(14 * row_mb)      # both in flight at 2 us
    assert prof[2, 1] == pytest.approx(5 * row_mb)       # the greedy one at 4 us
    assert prof[0, 3] == 72 and prof[1, 3] == 0          # all wait for scalars at 0 us
    assert prof[1, 2] == 1 and prof[4, 2] == 1           # the race workgroup at 2 and 8 us
    ragged = W.make_batch(5, 0)
    assert bench.stream_profile(np.stack(rows), ragged, 1.0) is None  # column grouping
