#!/usr/bin/env python3
"""Throughput of the verify sampler on one MI355X.

One step is one full verify call (both kernels) over one batch of synthetic
logits already resident in HBM. The default workload is the gated batch B=64,
T=4 (+1 bonus row), V=151936, bf16 logits. Four distinct input sets rotate,
so that repeated steps read HBM, not the 256 MB Infinity Cache.

It prints ONE JSON line on stdout with:
* verified rows/s (value);
* the whole step's algorithmic bytes per second;
* a roofline entry for the dominant kernel (the one with the longer mean
  launch, with the other beside it), timed with HIP events recorded on the
  launch stream around each kernel (a second run of the same steps, so that
  the events do not slow the timed steps), and its HBM traffic from the
  counter record in profiles/ while the kernel sources match it;
* the CPU oracle timed on a bounded sample of the same workload on this
  host's cores.

--row-sums, --lazy and --filtered time the acceptance sums, the lazy verify
and the filtered verify instead, each printing its own line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified rows/sec + achieved HBM GB/s (% of peak), B=64 T=4 V=151936 bf16"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_pass1_pass2_gated_B64_T4_V151936_bf16.json")
KERNEL_SOURCES = [os.path.join(ROOT, "lossless_rejection_sampling_row_amd", "csrc", f)
                  for f in ("sv_kernels.hip", "sv_device.h", "sv_plan.h")]
DEFAULT_SETS = {1: 2, 2: 8, 3: 4, 4: 2, 5: 2}
COPY_MIB = 384  # calibration copy: larger than the 256 MB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code: comments and blank space are dropped first, so that an
    edit of a comment does not void counters taken on the same code."""
    import re
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def proposal_rows(w, requests=None) -> int:
    """Rows pass 1 streams: every row before a request's first no-proposal row and before its
    last row (of the given requests, default all)."""
    ro, dt, V = w.row_offsets, w.draft_tokens, w.V
    n = 0
    for b in (range(w.B) if requests is None else requests):
        lo, hi = int(ro[b]), int(ro[b + 1])
        for r in range(lo, hi - 1):
            if not (0 <= dt[r] < V):
                break
            n += 1
    return n


def pass2_bytes(w, accept_len: np.ndarray, esize: int) -> int:
    """Bytes the method must read to draw each request's last token."""
    ro, dt, V = w.row_offsets, w.draft_tokens, w.V
    tot = 0
    for b in range(w.B):
        k = int(accept_len[b])
        if k < 0:
            continue
        lo, hi = int(ro[b]), int(ro[b + 1])
        r = lo + k
        bonus = (r == hi - 1) or not (0 <= dt[r] < V)
        greedy = w.temperature[b] == 0
        if bonus:
            tot += V * esize                    # race (or argmax) over p
        elif not greedy:
            tot += 2 * V * esize                # race over (p - mu)+
    return tot


def tested_rows(w, accept_len: np.ndarray) -> int:
    """Rows the lazy verify streams: each request's rows up to its stop (the stop row included
    when it is a proposal row), as given by its accept length."""
    ro, dt, V = w.row_offsets, w.draft_tokens, w.V
    n = 0
    for b in range(w.B):
        k = int(accept_len[b])
        if k < 0:
            continue
        lo, hi = int(ro[b]), int(ro[b + 1])
        nprop = 0
        for r in range(lo, hi - 1):
            if not (0 <= dt[r] < V):
                break
            nprop += 1
        n += min(k + 1, nprop)
    return n


POOL_CAP = 16  # a one-GPU machine's share of host cores, whatever the affinity mask shows
_POOL_W = None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _pool_init(cfg: int) -> None:
    global _POOL_W
    from lossless_rejection_sampling_row_amd import workloads as wl
    _POOL_W = wl.config(cfg)


def _pool_ready(_: int) -> int:
    time.sleep(0.2)  # keep this worker busy so that every worker takes one
    return os.getpid()


def _pool_task(seed: int, b0: int, b1: int) -> int:
    """The oracle on requests b0 .. b1-1 of the worker's batch; returns the rows it verified."""
    from oracle import verify as ov
    w = _POOL_W
    ov.verify_batch(w.target, w.draft, w.draft_tokens, w.row_offsets, w.temperature, w.tau, seed, w.dtype,
                    requests=range(b0, b1))
    return int(w.row_offsets[b1] - w.row_offsets[b0])


def _single_leg(w, budget_s: float):
    from oracle import verify as ov
    rows = calls = 0
    t0 = time.perf_counter()
    while True:
        ov.verify_batch(w.target, w.draft, w.draft_tokens, w.row_offsets, w.temperature, w.tau, calls, w.dtype)
        rows += w.R
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": rows / el, "unit": "rows/s", "cores": 1,
            "sample": f"{calls} full batches (seeds 0..{calls - 1}), {rows} rows in {el:.1f} s, one process"}


def _pool_leg(cfg: int, w, budget_s: float):
    import multiprocessing as mp
    from concurrent.futures import FIRST_COMPLETED, ProcessPoolExecutor, wait
    avail = len(os.sched_getaffinity(0))
    n = max(1, min(avail, POOL_CAP))
    chunk = max(1, min(4, w.B))
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=_pool_init,
                             initargs=(cfg,)) as pool:
        for f in [pool.submit(_pool_ready, i) for i in range(n)]:
            f.result()  # every worker has built the batch before the clock starts
        jobs = ((seed, b, min(b + chunk, w.B)) for seed in range(1 << 30) for b in range(0, w.B, chunk))
        rows = tasks = 0
        t0 = time.perf_counter()
        live = {pool.submit(_pool_task, *next(jobs)) for _ in range(2 * n)}
        while live:
            done, live = wait(live, return_when=FIRST_COMPLETED)
            for f in done:
                rows += f.result()
                tasks += 1
            if time.perf_counter() - t0 < budget_s:
                live |= {pool.submit(_pool_task, *next(jobs)) for _ in done}
        el = time.perf_counter() - t0
    return {"value": rows / el, "unit": "rows/s", "cores": n,
            "sample": f"{tasks} tasks of {chunk} requests over seeds 0.., {rows} rows in {el:.1f} s, "
                      f"a pool of {n} processes ({avail} cores in the affinity mask, at most {POOL_CAP} used)"}


def cpu_baseline(cfg: int, w, budget_s: float):
    """Time the oracle as it stands on this host: one process over whole batches of the workload,
    then a spawn pool of processes over its requests on the cores this process may use."""
    one = _single_leg(w, budget_s / 2)
    many = _pool_leg(cfg, w, budget_s / 2)
    model = cpu_model()
    return {"value": many["value"], "unit": "rows/s", "cores": many["cores"], "kind": "oracle",
            "sample": many["sample"], "cpu_model": model,
            "legs": [dict(one, cpu_model=model), dict(many, cpu_model=model)]}


def _counter_means(path, counter):
    """Mean counter value per dispatch, per kernel name, from a rocprofv3 counter_collection.csv."""
    import csv
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return acc


def write_traffic(fetch_csv: str, write_csv: str) -> None:
    """HBM bytes per launch of each verify kernel from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by the same counter on the calibration copy: its largest dispatch moved COPY_MIB
    MiB each way."""
    fetch = _counter_means(fetch_csv, "FETCH_SIZE")
    write = _counter_means(write_csv, "WRITE_SIZE")

    def pick(d, key):
        return [v for k, vs in d.items() if key(k) for v in vs]

    cf = max(pick(fetch, lambda k: "copy" in k.lower()))
    cw = max(pick(write, lambda k: "copy" in k.lower()))
    copy_bytes = COPY_MIB * 1024 * 1024
    f_fetch = copy_bytes / (cf * 1024.0)
    f_write = copy_bytes / (cw * 1024.0)
    kernels = {}
    for name in ("pass1_kernel", "pass2_kernel"):
        kf = pick(fetch, lambda k: name in k)
        kw = pick(write, lambda k: name in k)
        fetch_kib = sum(kf) / len(kf)
        write_kib = sum(kw) / len(kw)
        kernels[name] = {
            "dispatches": len(kf),
            "fetch_kib_per_dispatch": round(fetch_kib, 1),
            "write_kib_per_dispatch": round(write_kib, 1),
            "hbm_bytes_per_launch": int(fetch_kib * 1024 * f_fetch + write_kib * 1024 * f_write),
        }
    rec = {
        "workload": "gated B=64 T=4 V=151936 bf16",
        "kernel_source_hash": kernel_source_hash(),
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": cf,
        "copy_write_kib": cw,
        "fetch_scale": round(f_fetch, 4),
        "write_scale": round(f_write, 4),
        "kernels": kernels,
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o f -- python3 bench.py --steps 8 --warmup 2 "
            f"--cpu-budget 0 --copy-calibration {COPY_MIB}",
            f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o w -- python3 bench.py --steps 8 --warmup 2 "
            f"--cpu-budget 0 --copy-calibration {COPY_MIB}",
            "python3 bench.py --write-traffic <dir>/f_counter_collection.csv <dir>/w_counter_collection.csv",
        ],
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def bench_lazy(args, binding, torch, sets, ws, stream):
    """K lazy verify calls over the rotating input sets. Algorithmic bytes: the rows each request
    must read up to its stop, its final row's bytes, and the small arrays."""
    from lossless_rejection_sampling_row_amd import workloads as wl
    K, W = args.steps, args.warmup
    nsets = len(sets)
    w0 = sets[0][0]
    B, R, V = w0.B, w0.R, w0.V
    esize = 2 if w0.dtype == "bf16" else 4
    max_rows = int(np.diff(w0.row_offsets).max())
    out_tok = torch.empty((K, R), dtype=torch.int32, device=stream.device)
    out_len = torch.empty((K, B), dtype=torch.int32, device=stream.device)

    def call(i, tok, ln):
        _, g = sets[i % nsets]
        binding.verify_batch(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"], g["temperature"],
                             g["tau"], 1_000_003 * i + 17, out_tokens=tok, out_accept_len=ln, workspace=ws,
                             stream=stream, lazy_max_rows=max_rows)

    for i in range(W):
        call(i, out_tok[0], out_len[0])
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(K):
        call(i, out_tok[i], out_len[i])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    lens = out_len.cpu().numpy()
    alg = np.array([tested_rows(sets[i % nsets][0], lens[i]) * V * 2 * esize
                    + pass2_bytes(sets[i % nsets][0], lens[i], esize) + 16 * R + 8 * B for i in range(K)],
                   dtype=np.float64)
    rows_read = np.mean([tested_rows(sets[i % nsets][0], lens[i]) for i in range(K)])
    gbps = alg.mean() / (ms / 1e3) / 1e9
    log(f"[bench] lazy: {ms * 1e3:.1f} us/step, {rows_read:.1f} of {proposal_rows(w0)} proposal rows read, "
        f"{gbps:.0f} GB/s of algorithmic bytes")
    line = {
        "metric": "verified rows/sec, lazy position-serial verify (reads rows up to each request's first rejection)",
        "value": round(R / (ms / 1e3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.CONFIG_NAMES[args.config], "B": B, "rows": R, "V": V, "logits": w0.dtype,
                   "input_sets": nsets, "max_rows": max_rows, "rows_read_per_step": round(float(rows_read), 1)},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": f"{max(1, max_rows - 1)} x lazy_rows_kernel + pass2_kernel (one call)",
                     "launch_us": round(ms * 1e3, 2), "alg_bytes_per_launch": int(alg.mean())},
    }
    print(json.dumps(line), flush=True)


def filter_active(w, filt) -> np.ndarray:
    """Per request: T > 0 and a filter that removes something."""
    k, tp, mp = filt
    return (w.temperature > 0) & (((k > 0) & (k < w.V)) | (tp < 1.0) | (mp > 0.0))


def filtered_rows(w, filt, draft_side=None) -> int:
    """Rows the thresholds chain reads on one side: every row of a request with T > 0 and an
    active filter on that side (sv_filter_thresholds). With draft_side set, only the rows the
    verify reads on that side: a request's rows up to its first row without a proposal, less
    that row on the draft side."""
    ro = w.row_offsets.astype(np.int64)
    act = filter_active(w, filt)
    if draft_side is None:
        return int(np.sum(np.diff(ro)[act]))
    dt = w.draft_tokens
    n = 0
    for b in np.flatnonzero(act):
        d = dt[ro[b]:ro[b + 1]]
        f = int(np.flatnonzero((d < 0) | (d >= w.V))[0])  # the last row has none
        n += f if draft_side else f + 1
    return n


def bench_filtered(args, binding, torch, sets, ws, stream):
    """K filtered verify calls (top-k / top-p / min-p on both sides), and K calls of the
    thresholds chain alone (sv_filter_thresholds: seg_records_kernel, then
    thresholds_finish_kernel). The chain's algorithmic bytes are one read of every row it
    filters; the whole call's are one read of each filtered row side the verify reads, plus
    pass 1's and pass 2's bytes."""
    from lossless_rejection_sampling_row_amd import workloads as wl
    K, W = args.steps, args.warmup
    nsets = len(sets)
    w0 = sets[0][0]
    B, R, V = w0.B, w0.R, w0.V
    esize = 2 if w0.dtype == "bf16" else 4
    filts = []
    for i in range(nsets):
        tf, df = wl.sampler_filters(B, rng_seed=4242 + i)
        dev = stream.device
        to_t = lambda f: tuple(torch.from_numpy(a).to(dev) for a in f)  # noqa: E731
        filts.append(((tf, df), (to_t(tf), to_t(df))))
    out_tok = torch.empty((K, R), dtype=torch.int32, device=stream.device)
    out_len = torch.empty((K, B), dtype=torch.int32, device=stream.device)
    theta = torch.empty((R, 2), dtype=torch.float32, device=stream.device)

    def call(i, tok, ln):
        _, g = sets[i % nsets]
        _, (tf, df) = filts[i % nsets]
        binding.verify_batch(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"], g["temperature"],
                             g["tau"], 1_000_003 * i + 17, out_tokens=tok, out_accept_len=ln, workspace=ws,
                             stream=stream, target_filter=tf, draft_filter=df)

    def thresholds(i):
        _, g = sets[i % nsets]
        _, (tf, df) = filts[i % nsets]
        binding.filter_thresholds(g["target"], g["draft"], g["row_offsets"], g["temperature"], target_filter=tf,
                                  draft_filter=df, out_theta=theta, workspace=ws, stream=stream)

    def timed(fn):
        for i in range(W):
            fn(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(K):
            fn(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / K

    ms = timed(lambda i: call(i, out_tok[i], out_len[i]))
    ms_th = timed(thresholds)
    lens = out_len.cpu().numpy()
    th_bytes = np.array([(filtered_rows(sets[i % nsets][0], filts[i % nsets][0][0])
                          + filtered_rows(sets[i % nsets][0], filts[i % nsets][0][1])) * V * esize
                         for i in range(K)], dtype=np.float64)
    # Pass 1 must read only the unfiltered sides of the proposal rows: the chain read the others.
    def pair_bytes(i):
        w, (tf, df) = sets[i % nsets][0], filts[i % nsets][0]
        rows = sum(proposal_rows(w, np.flatnonzero(~filter_active(w, f))) for f in (tf, df))
        return rows * V * esize + pass2_bytes(w, lens[i], esize)
    pair = np.array([pair_bytes(i) for i in range(K)], dtype=np.float64)
    used_bytes = np.array([(filtered_rows(sets[i % nsets][0], filts[i % nsets][0][0], draft_side=False)
                            + filtered_rows(sets[i % nsets][0], filts[i % nsets][0][1], draft_side=True)) * V * esize
                           for i in range(K)], dtype=np.float64)
    th_gbps = th_bytes.mean() / (ms_th / 1e3) / 1e9
    gbps = (used_bytes.mean() + pair.mean()) / (ms / 1e3) / 1e9
    log(f"[bench] filtered verify: {ms * 1e3:.1f} us/step ({gbps:.0f} GB/s of algorithmic bytes); thresholds chain "
        f"alone {ms_th * 1e3:.1f} us ({th_gbps:.0f} GB/s, one read of each filtered row)")
    line = {
        "metric": "verified rows/sec, filtered verify (top-k / top-p / min-p on p and q)",
        "value": round(R / (ms / 1e3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.CONFIG_NAMES[args.config] + ", sampler filters on both sides", "B": B, "rows": R,
                   "V": V, "logits": w0.dtype, "input_sets": nsets,
                   "filters": "per request: top_k {0,20,50}, top_p {1,0.9,0.95}, min_p {0,0.05}, each side"},
        "thresholds_us": round(ms_th * 1e3, 2),
        "roofline": {"bound": "hbm", "achieved": round(th_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(th_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "seg_records_kernel + thresholds_finish_kernel (one sv_filter_thresholds call)",
                     "launch_us": round(ms_th * 1e3, 2), "alg_bytes_per_launch": int(th_bytes.mean())},
        "whole_call": {"achieved": round(gbps, 1), "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                       "alg_bytes_per_call": int(used_bytes.mean() + pair.mean())},
    }
    print(json.dumps(line), flush=True)


def bench_row_sums(args, binding, torch, sets, ws, stream):
    """K calls of sv_row_acceptance over the rotating input sets. The two-pass method reads every
    proposal row twice (statistics, then the sums), so its algorithmic bytes are twice pass 1's."""
    from lossless_rejection_sampling_row_amd import workloads as wl
    K, W = args.steps, args.warmup
    nsets = len(sets)
    w0 = sets[0][0]
    R, V = w0.R, w0.V
    esize = 2 if w0.dtype == "bf16" else 4
    smin = torch.empty(R, dtype=torch.float32, device=stream.device)
    spq = torch.empty(R, dtype=torch.float32, device=stream.device)

    def call(i):
        _, g = sets[i % nsets]
        binding.row_acceptance(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"], g["temperature"],
                               g["tau"], out_sum_min=smin, out_sum_pq=spq, workspace=ws, stream=stream)

    for i in range(W):
        call(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(K):
        call(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    prop = np.array([proposal_rows(sets[i % nsets][0]) for i in range(K)], dtype=np.float64)
    alg = 2.0 * prop * V * 2 * esize
    gbps = alg.mean() / (ms / 1e3) / 1e9
    log(f"[bench] row sums: {ms * 1e3:.1f} us/call, {gbps:.0f} GB/s of algorithmic bytes")
    line = {
        "metric": "per-row acceptance sums (sum min(p, mu), sum p q): rows/s and algorithmic GB/s",
        "value": round(R / (ms / 1e3), 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.CONFIG_NAMES[args.config], "rows": R, "V": V, "logits": w0.dtype,
                   "input_sets": nsets},
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "pass1_kernel + sums_kernel + merge_sums_kernel (one call)",
                     "launch_us": round(ms * 1e3, 2), "alg_bytes_per_launch": int(alg.mean())},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--sets", type=int, default=None, help="distinct input sets rotated through")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle timing, split between the one-process and pool legs (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the steps, copy a MIB-MiB device buffer three times (a plain copy of known size "
                         "whose FETCH_SIZE / WRITE_SIZE scale the counters of the verify kernels)")
    ap.add_argument("--row-sums", action="store_true",
                    help="time the per-row acceptance sums (sv_row_acceptance) on the same inputs instead of the "
                         "verify call, and print their own JSON line")
    ap.add_argument("--filtered", action="store_true",
                    help="time the filtered verify (sampler filters on both sides) and its thresholds chain")
    ap.add_argument("--lazy", action="store_true",
                    help="time the lazy position-serial verify (sv_verify_batch_lazy) instead, and print its own "
                         "JSON line; its algorithmic bytes count only the rows it must read")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 counter_collection.csv files (FETCH_SIZE, WRITE_SIZE runs "
                         "with --copy-calibration) into the traffic record the roofline entry reads")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): this verify "
              f"path is measured on a single MI355X; requests shard across GPUs with no "
              f"exchange, so more GPUs are not run here.", file=sys.stderr)
        sys.exit(2)

    import torch
    from lossless_rejection_sampling_row_amd import binding
    from lossless_rejection_sampling_row_amd import workloads as wl

    binding.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nsets = args.sets or DEFAULT_SETS[args.config]
    log(f"[bench] generating {nsets} input sets of {wl.CONFIG_NAMES[args.config]}")
    sets = []
    for i in range(nsets):
        w = wl.config(args.config, rng_seed=wl.CONFIGS[args.config].rng_seed + 7919 * i)
        esize = 2 if w.dtype == "bf16" else 4
        if w.dtype == "bf16":
            tgt = torch.from_numpy(w.target.view(np.int16)).view(torch.bfloat16).to(dev)
            dft = torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16).to(dev)
        else:
            tgt = torch.from_numpy(w.target).to(dev)
            dft = torch.from_numpy(w.draft).to(dev)
        g = dict(target=tgt, draft=dft,
                 draft_tokens=torch.from_numpy(w.draft_tokens).to(dev),
                 row_offsets=torch.from_numpy(w.row_offsets).to(dev),
                 temperature=torch.from_numpy(w.temperature).to(dev),
                 tau=torch.from_numpy(w.tau).to(dev))
        sets.append((w, g))
    w0 = sets[0][0]
    B, R, V = w0.B, w0.R, w0.V
    K, W = args.steps, args.warmup
    ws = torch.zeros(binding.workspace_bytes(B, R, V, sets[0][1]["target"].dtype), dtype=torch.uint8, device=dev)
    out_tok = torch.empty((K, R), dtype=torch.int32, device=dev)
    out_len = torch.empty((K, B), dtype=torch.int32, device=dev)
    scratch_tok = torch.empty(R, dtype=torch.int32, device=dev)
    scratch_len = torch.empty(B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    if args.row_sums:
        bench_row_sums(args, binding, torch, sets, ws, stream)
        return
    if args.lazy:
        bench_lazy(args, binding, torch, sets, ws, stream)
        return
    if args.filtered:
        bench_filtered(args, binding, torch, sets, ws, stream)
        return
    ev = binding.HipEvents(3 * K)

    def step(i, timed, events=False):
        w, g = sets[i % nsets]
        kw = dict(workspace=ws, stream=stream)
        if timed:
            kw.update(out_tokens=out_tok[i], out_accept_len=out_len[i])
        else:
            kw.update(out_tokens=scratch_tok, out_accept_len=scratch_len)
        if events:
            kw.update(events=ev.handles[3 * i:3 * i + 3])
        binding.verify_batch(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"],
                             g["temperature"], g["tau"], 1_000_003 * i + 17, **kw)

    log(f"[bench] warmup {W} steps")
    for i in range(W):
        step(i, False)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # The step time comes from K back-to-back calls with nothing recorded between them.
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(K):
        step(i, True)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # The per-kernel durations come from the same K steps run again with HIP events recorded
    # on the launch stream around each kernel (events between kernels slow the step a little).
    log(f"[bench] timing each kernel over {K} more steps")
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    e_start.record(stream)
    for i in range(K):
        step(i, True, events=True)
    e_end.record(stream)
    torch.cuda.synchronize()
    evented_ms = e_start.elapsed_time(e_end) / K
    p1_ms = np.array([ev.elapsed_ms(3 * i, 3 * i + 1) for i in range(K)])
    p2_ms = np.array([ev.elapsed_ms(3 * i + 1, 3 * i + 2) for i in range(K)])
    lens = out_len.cpu().numpy()
    ev.close()

    esize = 2 if w0.dtype == "bf16" else 4
    prop = [proposal_rows(w) for w, _ in sets]
    p1_bytes = np.array([prop[i % nsets] * V * 2 * esize for i in range(K)], dtype=np.float64)
    p2_bytes = np.array([pass2_bytes(sets[i % nsets][0], lens[i], esize) for i in range(K)], dtype=np.float64)
    small = 16 * R + 8 * B
    alg = p1_bytes + p2_bytes + small
    ms_per_step = total_ms / K
    rows_per_s = R * K / (total_ms / 1e3)
    step_gbps = alg.sum() / (total_ms / 1e3) / 1e9
    p1_gbps = p1_bytes.mean() / (p1_ms.mean() / 1e3) / 1e9
    log(f"[bench] {ms_per_step * 1e3:.1f} us/step ({evented_ms * 1e3:.1f} with kernel events); "
        f"pass1 {p1_ms.mean() * 1e3:.1f} us ({p1_gbps:.0f} GB/s); pass2 {p2_ms.mean() * 1e3:.1f} us; "
        f"step {step_gbps:.0f} GB/s")

    traffic = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash() and args.config == 3:
            traffic = {k: v.get("hbm_bytes_per_launch") for k, v in tr.get("kernels", {}).items()}

    def roof(name, nbytes, ms):
        gbps = nbytes.mean() / (ms.mean() / 1e3) / 1e9
        return {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic.get(name),
                "kernel": name, "launch_us": round(float(ms.mean()) * 1e3, 2),
                "alg_bytes_per_launch": int(nbytes.mean())}

    # The entry for the kernel with the longer average launch leads; the other follows.
    roofs = [roof("pass1_kernel", p1_bytes, p1_ms), roof("pass2_kernel", p2_bytes, p2_ms)]
    roofs.sort(key=lambda r: -r["launch_us"])
    roofline = roofs[0]

    if args.copy_calibration:
        n = args.copy_calibration * 1024 * 1024
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_budget > 0:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_budget:.0f} s")
        cpu = cpu_baseline(args.config, w0, args.cpu_budget)

    line = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.CONFIG_NAMES[args.config], "B": B, "rows": R, "V": V,
                   "logits": w0.dtype, "input_sets": nsets},
        "achieved_gbps": round(step_gbps, 1),
        "hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "pass2_us": round(float(p2_ms.mean()) * 1e3, 2),
        "us_per_step_with_kernel_events": round(evented_ms * 1e3, 2),
        "roofline": roofline,
        "roofline_other_kernel": roofs[1],
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
