"""A host process pool that runs the oracle over many seeds of a benchmark batch.

Each worker builds the seeded batch itself (once per configuration) instead of receiving
it, so a task is only (configuration, seed, requests). Workers are started with "spawn":
fresh interpreters that never touch the GPU.
"""
import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

_CACHE: dict = {}


def workers(cap: int = 16) -> int:
    """Worker count: the cores this process may run on, at most `cap`."""
    return max(1, min(cap, len(os.sched_getaffinity(0))))


def make_pool(n: int) -> ProcessPoolExecutor:
    return ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"))


def _batch(cfg: int):
    if cfg not in _CACHE:
        from lossless_rejection_sampling_row_amd import workloads as wl
        from tests.gpu_util import as_batch
        _CACHE.clear()
        _CACHE[cfg] = as_batch(wl.config(cfg))
    return _CACHE[cfg]


def oracle_task(cfg: int, seed: int, requests: list, filt_seed=None):
    """The oracle on `requests` of configuration `cfg` at `seed`: (flags, accept_len, tokens).
    With filt_seed, both sides carry the serving-style filters workloads.sampler_filters draws
    from that seed."""
    from tests.gpu_util import run_oracle
    batch = _batch(cfg)
    if filt_seed is not None:
        from lossless_rejection_sampling_row_amd import workloads as wl
        B = len(batch["row_offsets"]) - 1
        batch = dict(batch)
        batch["target_filter"], batch["draft_filter"] = wl.sampler_filters(B, rng_seed=filt_seed)
    o = run_oracle(batch, seed=seed, requests=requests)
    return o.flags, o.out_accept_len, o.out_tokens
