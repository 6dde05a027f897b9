"""Shared machinery for the GPU parity tests: upload a batch, run the HIP path, compare with the oracle."""
from __future__ import annotations

import sys
from dataclasses import dataclass

import numpy as np

from oracle import verify as ov

P_RTOL = 1e-5           # p(D), q(D), mu(D): relative
RESID_RTOL = 1e-5       # residual mass: max(RESID_RTOL * R, RESID_ATOL)
RESID_ATOL = 2e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def as_batch(w):
    """A workloads.Workload or a helpers.batch_from_rows dict -> dict."""
    if isinstance(w, dict):
        return w
    return dict(target=w.target, draft=w.draft, draft_tokens=w.draft_tokens, row_offsets=w.row_offsets,
                temperature=w.temperature, tau=w.tau, seed=w.seed, dtype=w.dtype)


def upload(batch, device="cuda"):
    import torch
    dt = torch.bfloat16 if batch["dtype"] == "bf16" else torch.float32
    if batch["dtype"] == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(batch["target"]).view(np.int16)).view(torch.bfloat16)
        d = torch.from_numpy(np.ascontiguousarray(batch["draft"]).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(batch["target"], dtype=np.float32))
        d = torch.from_numpy(np.ascontiguousarray(batch["draft"], dtype=np.float32))
    assert t.dtype == dt
    g = dict(
        target=t.to(device), draft=d.to(device),
        draft_tokens=torch.from_numpy(np.ascontiguousarray(batch["draft_tokens"], dtype=np.int32)).to(device),
        row_offsets=torch.from_numpy(np.ascontiguousarray(batch["row_offsets"], dtype=np.int32)).to(device),
        temperature=torch.from_numpy(np.ascontiguousarray(batch["temperature"], dtype=np.float32)).to(device),
        tau=torch.from_numpy(np.ascontiguousarray(batch["tau"], dtype=np.float32)).to(device),
    )
    for key in ("tau_step", "min_cum"):  # optional gate schedule and cumulative floor
        if batch.get(key) is not None:
            g[key] = torch.from_numpy(np.ascontiguousarray(batch[key], dtype=np.float32)).to(device)
    for key in ("target_filter", "draft_filter"):  # optional (top_k, top_p, min_p) triples
        f = batch.get(key)
        if f is not None:
            g[key] = tuple(None if a is None else
                           torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32 if i == 0 else np.float32)).to(device)
                           for i, a in enumerate(f))
    return g


@dataclass
class GpuResult:
    out_tokens: np.ndarray
    out_accept_len: np.ndarray
    p_D: np.ndarray
    q_D: np.ndarray
    mu_D: np.ndarray
    u: np.ndarray
    resid_mass: np.ndarray
    verdict: np.ndarray
    stats: np.ndarray


def run_gpu(batch, seed=None, gpu=None, diag=True):
    import torch
    from lossless_rejection_sampling_row_amd import binding
    g = gpu if gpu is not None else upload(batch)
    R = int(g["target"].shape[0])
    row_diag = torch.full((R, 8), -7, dtype=torch.int32, device="cuda") if diag else None
    stats = torch.full((binding.STATS_FIELDS,), -7, dtype=torch.int64, device="cuda") if diag else None
    toks, lens = binding.verify_batch(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"],
                                      g["temperature"], g["tau"], batch["seed"] if seed is None else seed,
                                      row_diag=row_diag, stats=stats, tau_step=g.get("tau_step"),
                                      min_cum=g.get("min_cum"), target_filter=g.get("target_filter"),
                                      draft_filter=g.get("draft_filter"))
    torch.cuda.synchronize()
    if diag:
        p, q, mu, u, rm, v = binding.split_row_diag(row_diag)
        return GpuResult(toks.cpu().numpy(), lens.cpu().numpy(), p.cpu().numpy().astype(np.float64),
                         q.cpu().numpy().astype(np.float64), mu.cpu().numpy().astype(np.float64),
                         u.cpu().numpy().astype(np.float64), rm.cpu().numpy().astype(np.float64),
                         v.cpu().numpy(), stats.cpu().numpy())
    return GpuResult(toks.cpu().numpy(), lens.cpu().numpy(), None, None, None, None, None, None, None)


def run_oracle(batch, seed=None, requests=None):
    return ov.verify_batch(batch["target"], batch["draft"], batch["draft_tokens"], batch["row_offsets"],
                           batch["temperature"], batch["tau"], batch["seed"] if seed is None else seed,
                           batch["dtype"], requests=requests, tau_step=batch.get("tau_step"),
                           min_cum=batch.get("min_cum"), target_filter=batch.get("target_filter"),
                           draft_filter=batch.get("draft_filter"))


@dataclass
class Parity:
    requests: int = 0
    rows: int = 0
    flagged_requests: int = 0
    flagged_rows: int = 0
    max_p_rel: float = 0.0
    max_mu_rel: float = 0.0
    max_resid_abs: float = 0.0

    def add(self, other: "Parity"):
        for k in self.__dataclass_fields__:
            if k.startswith("max_"):
                setattr(self, k, max(getattr(self, k), getattr(other, k)))
            else:
                setattr(self, k, getattr(self, k) + getattr(other, k))


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.maximum(np.abs(b), 1e-300)
    return np.where(a == b, 0.0, np.abs(a - b) / den)


def compare(batch, gpu: GpuResult, ora, requests=None, check_diag=True) -> Parity:
    """Assert parity request by request; flagged requests are counted and skipped."""
    ro = np.asarray(batch["row_offsets"], dtype=np.int64)
    temp = np.asarray(batch["temperature"], dtype=np.float32)
    B = ro.size - 1
    par = Parity()
    todo = range(B) if requests is None else requests
    for b in todo:
        lo, hi = int(ro[b]), int(ro[b + 1])
        par.requests += 1
        par.rows += hi - lo
        if ora.flags[b]:
            par.flagged_requests += 1
            par.flagged_rows += hi - lo
            continue
        ctx = f"request {b} (rows {lo}..{hi - 1}, T={temp[b]}, flags={ora.flags[b]})"
        assert gpu.out_accept_len[b] == ora.out_accept_len[b], \
            f"{ctx}: accept_len gpu {gpu.out_accept_len[b]} oracle {ora.out_accept_len[b]}"
        assert np.array_equal(gpu.out_tokens[lo:hi], ora.out_tokens[lo:hi]), \
            f"{ctx}: tokens gpu {gpu.out_tokens[lo:hi]} oracle {ora.out_tokens[lo:hi]}"
        if not check_diag or gpu.verdict is None or ora.out_accept_len[b] < 0:
            continue
        k = int(ora.out_accept_len[b])
        rows = np.arange(lo, lo + k + 1)
        assert np.array_equal(gpu.verdict[rows], ora.verdict[rows]), \
            f"{ctx}: verdicts gpu {gpu.verdict[rows]} oracle {ora.verdict[rows]}"
        assert np.all(gpu.verdict[lo + k + 1:hi] == 0), f"{ctx}: rows after the stop must be untested"
        tested = rows[(ora.verdict[rows] == ov.ACCEPT) | (ora.verdict[rows] == ov.REJECT) |
                      (ora.verdict[rows] == ov.NULL)]
        if tested.size:
            pr = _rel(gpu.p_D[tested], ora.p_D[tested])
            qr = _rel(gpu.q_D[tested], ora.q_D[tested])
            mr = _rel(gpu.mu_D[tested], ora.mu_D[tested])
            par.max_p_rel = max(par.max_p_rel, float(pr.max()), float(qr.max()))
            par.max_mu_rel = max(par.max_mu_rel, float(mr.max()))
            assert np.all(pr <= P_RTOL), f"{ctx}: p(D) gpu {gpu.p_D[tested]} oracle {ora.p_D[tested]}"
            assert np.all(qr <= P_RTOL), f"{ctx}: q(D) gpu {gpu.q_D[tested]} oracle {ora.q_D[tested]}"
            assert np.all(mr <= P_RTOL), f"{ctx}: mu(D) gpu {gpu.mu_D[tested]} oracle {ora.mu_D[tested]}"
            if temp[b] > 0:
                offered = tested[ora.verdict[tested] != ov.NULL]
                assert np.array_equal(gpu.u[offered], ora.u[offered]), f"{ctx}: accept uniforms differ"
        fr = lo + k
        if ora.verdict[fr] in (ov.REJECT, ov.NULL) and temp[b] > 0:
            R = ora.resid_mass[fr]
            err = abs(gpu.resid_mass[fr] - R)
            par.max_resid_abs = max(par.max_resid_abs, err)
            assert err <= max(RESID_RTOL * R, RESID_ATOL), f"{ctx}: residual mass gpu {gpu.resid_mass[fr]} oracle {R}"
    return par


def check_properties(batch, gpu: GpuResult):
    """Invariants that hold for every request at any size (used where the oracle samples a subset)."""
    ro = np.asarray(batch["row_offsets"], dtype=np.int64)
    V = np.asarray(batch["target"]).shape[1]
    dt = np.asarray(batch["draft_tokens"])
    for b in range(ro.size - 1):
        lo, hi = int(ro[b]), int(ro[b + 1])
        k = int(gpu.out_accept_len[b])
        assert -1 <= k <= hi - lo - 1
        if k < 0:
            assert np.all(gpu.out_tokens[lo:hi] == -1)
            continue
        assert np.array_equal(gpu.out_tokens[lo:lo + k], dt[lo:lo + k])
        assert 0 <= gpu.out_tokens[lo + k] < V
        assert np.all(gpu.out_tokens[lo + k + 1:hi] == -1)
