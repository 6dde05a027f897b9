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


def oracle_task(cfg: int, seed: int, requests: list):
    """The oracle on `requests` of configuration `cfg` at `seed`: (flags, accept_len, tokens)."""
    from tests.gpu_util import run_oracle
    o = run_oracle(_batch(cfg), seed=seed, requests=requests)
    return o.flags, o.out_accept_len, o.out_tokens
