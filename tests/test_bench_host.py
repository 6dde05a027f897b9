"""Host logic of bench.py (no GPU): the single-GPU contract, the traffic record built from
rocprofv3 counter files, and the row counts the algorithmic bytes come from."""
import csv
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for k, v in rows:
            w.writerow({"Kernel_Name": k, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_record_scales_by_the_copy(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    copy_kib = bench.COPY_MIB * 1024
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    # FETCH_SIZE reads half the copy's bytes, WRITE_SIZE all of them
    _counter_csv(f, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", copy_kib / 2), ("void sv::pass1_kernel<x>", 1000.0),
                                   ("void sv::pass1_kernel<x>", 3000.0), ("void sv::pass2_kernel<x>", 500.0)])
    _counter_csv(w, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", copy_kib), ("void sv::pass1_kernel<x>", 10.0),
                                   ("void sv::pass2_kernel<x>", 20.0)])
    bench.write_traffic(str(f), str(w))
    rec = json.load(open(out))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["kernels"]["pass1_kernel"]["hbm_bytes_per_launch"] == int(2000 * 1024 * 2 + 10 * 1024)
    assert rec["kernels"]["pass2_kernel"]["hbm_bytes_per_launch"] == int(500 * 1024 * 2 + 20 * 1024)
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()


class _W:
    def __init__(self, ro, dt, V, temperature):
        self.row_offsets = np.asarray(ro)
        self.draft_tokens = np.asarray(dt)
        self.V = V
        self.B = len(ro) - 1
        self.temperature = np.asarray(temperature)


def test_row_counts():
    # request 0: 4 rows, all with proposals; request 1: 3 rows, a -1 at its second row
    w = _W([0, 4, 7], [1, 2, 3, 0, 5, -1, 2], 8, [1.0, 1.0])
    assert bench.proposal_rows(w) == 3 + 1
    # accepted 1 draft in request 0 (rows 0 and 1 read), bonus at row 1 of request 1 (row 0 read)
    assert bench.tested_rows(w, np.array([1, 1])) == 2 + 1
    # all three drafts of request 0 accepted: its three proposal rows were read
    assert bench.tested_rows(w, np.array([3, -1])) == 3
    # final-row bytes: request 0 stops at a residual row (both arrays), request 1 at a bonus row
    assert bench.pass2_bytes(w, np.array([1, 1]), 2) == 2 * 8 * 2 + 8 * 2


def test_filtered_row_counts():
    # three requests of 2, 3 and 1 rows; request 1 is greedy (its filters never apply)
    w = _W([0, 2, 5, 6], [1, -1, 2, 3, -1, -1], 10, [1.0, 0.0, 0.7])
    k = np.array([3, 3, 0], dtype=np.int32)
    tp = np.array([1.0, 1.0, 1.0], dtype=np.float32)
    mp = np.array([0.0, 0.0, 0.0], dtype=np.float32)
    assert bench.filtered_rows(w, (k, tp, mp)) == 2            # top-k on request 0 only
    mp[2] = 0.05
    assert bench.filtered_rows(w, (k, tp, mp)) == 3            # min-p turns request 2 on
    k[0] = 10                                                  # k >= V is off
    assert bench.filtered_rows(w, (k, tp, mp)) == 1
    tp[0] = 0.9
    assert bench.filtered_rows(w, (k, tp, mp)) == 3


def test_sampler_filter_recipe():
    from lossless_rejection_sampling_row_amd import workloads as wl
    t1, d1 = wl.sampler_filters(64, rng_seed=7)
    t2, d2 = wl.sampler_filters(64, rng_seed=7)
    for a, b in zip(t1 + d1, t2 + d2):
        assert np.array_equal(a, b)
    for k, tp, mp in (t1, d1):
        assert k.dtype == np.int32 and tp.dtype == np.float32 and mp.dtype == np.float32
        assert set(k.tolist()) <= {0, 20, 50} and set(tp.tolist()) <= {1.0, np.float32(0.9), np.float32(0.95)}
        assert set(mp.tolist()) <= {0.0, np.float32(0.05)}
    assert not all(np.array_equal(a, b) for a, b in zip(t1, d1))  # the two sides are drawn apart
