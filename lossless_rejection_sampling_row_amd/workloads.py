"""Seeded synthetic inputs for the verify sampler.

Both the HIP path and the CPU oracle are fed from this module. It holds none
of the verify method's arithmetic: it draws logits, rounds them to the storage
type, plays the drafter by drawing one draft token per proposal row, and lays
out the batch. A drafter samples its token from its own distribution q, so
the token here is drawn by Gumbel-max (argmax of draft/T plus Gumbel noise
from numpy's PCG64, in fp32). That is the producer's job. The verifier only reads the
token.

The pages measure on real models that are not available here (Llama-3.1-8B /
Llama-3.2-1B in mlxcel PR #992, section Verifying the gain). These
generators stand in for them with the shapes of the pages' workloads: vocab
32k to 256k, 4 to 8 draft positions, temperature 0.7 to 1.0. The recipe:

* target logits ~ N(0, sigma_t), drawn in float32;
* optionally, ``n_spikes`` distinct tokens per row raised by
  ``spike_sigmas * sigma_t`` (8 tokens at +8 sigma);
* draft logits = target logits (spikes included) + N(0, sigma_d);
* values rounded to bf16 with round-to-nearest-even, or kept in fp32;
* per request: the temperature, the gate threshold tau, and optionally the
  draft noise.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


@dataclass
class Spec:
    """Shape and value distribution of a synthetic verify batch."""
    B: int
    T: int | tuple = 4             # draft positions per request (int, or (lo, hi) inclusive for ragged)
    V: int = 32000
    dtype: str = "bf16"            # "bf16" or "f32"
    sigma_t: float = 3.0
    n_spikes: int = 0
    spike_sigmas: float = 8.0
    sigma_d: float | tuple = 1.0   # draft noise std, or (lo, hi) drawn per request
    temperature: float | tuple = 1.0   # scalar or (lo, hi) drawn per request
    greedy_frac: float = 0.0       # fraction of requests at temperature 0
    tau: float | tuple = 0.0       # scalar, or a tuple of choices drawn per request
    gated_frac: float | None = None  # if set: this fraction of requests gets tau, the rest 0
    noprop_frac: float = 0.0       # each proposal row independently gets draft token -1
    rng_seed: int = 0
    verify_seed: int = 0


@dataclass
class Workload:
    spec: Spec
    target: np.ndarray        # [R, V] uint16 bf16 bit patterns, or float32
    draft: np.ndarray         # same
    draft_tokens: np.ndarray  # [R] int32 (-1 = no proposal; the last row of a request is ignored)
    row_offsets: np.ndarray   # [B+1] int32
    temperature: np.ndarray   # [B] float32
    tau: np.ndarray           # [B] float32
    seed: int                 # Philox key for the verify call
    meta: dict = field(default_factory=dict)

    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def B(self) -> int:
        return int(self.row_offsets.size - 1)

    @property
    def R(self) -> int:
        return int(self.target.shape[0])

    @property
    def V(self) -> int:
        return int(self.target.shape[1])


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _stored(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _as_f32(stored: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(stored) if dtype == "bf16" else stored


def _draw_tokens(rng, draft_f32: np.ndarray, T: float) -> np.ndarray:
    """The drafter's draw D ~ softmax(draft/T) by Gumbel-max (-log of a unit exponential is Gumbel).

    T == 0 takes the argmax.
    """
    if T == 0.0:
        return np.argmax(draft_f32, axis=-1)
    e = rng.standard_exponential(size=draft_f32.shape, dtype=np.float32)
    np.maximum(e, np.float32(1e-30), out=e)   # an exact 0 would give an infinite Gumbel
    return np.argmax(draft_f32 * np.float32(1.0 / T) - np.log(e), axis=-1)


def generate(spec: Spec, row_chunk: int = 256) -> Workload:
    """Build a seeded batch. The same spec always gives the same bits."""
    rng = np.random.Generator(np.random.PCG64(spec.rng_seed))
    B, V = spec.B, spec.V
    if isinstance(spec.T, tuple):
        t_per = rng.integers(spec.T[0], spec.T[1] + 1, size=B)
    else:
        t_per = np.full(B, spec.T, dtype=np.int64)
    n_rows = t_per + 1
    ro = np.zeros(B + 1, dtype=np.int64)
    ro[1:] = np.cumsum(n_rows)
    R = int(ro[-1])

    # Per-request policy.
    if isinstance(spec.temperature, tuple):
        temp = rng.uniform(spec.temperature[0], spec.temperature[1], size=B)
    else:
        temp = np.full(B, spec.temperature)
    if spec.greedy_frac > 0:
        n_g = int(round(spec.greedy_frac * B))
        temp[rng.permutation(B)[:n_g]] = 0.0
    if isinstance(spec.tau, tuple):
        tau = rng.choice(np.asarray(spec.tau, dtype=np.float64), size=B)
    else:
        tau = np.full(B, spec.tau)
    if spec.gated_frac is not None:
        n_gated = int(round(spec.gated_frac * B))
        gated = np.zeros(B, dtype=bool)
        gated[rng.permutation(B)[:n_gated]] = True
        tau = np.where(gated, tau, 0.0)
    if isinstance(spec.sigma_d, tuple):
        sig_d = rng.uniform(spec.sigma_d[0], spec.sigma_d[1], size=B)
    else:
        sig_d = np.full(B, spec.sigma_d)
    temp = temp.astype(np.float32)
    tau = tau.astype(np.float32)

    req_of_row = np.repeat(np.arange(B), n_rows)
    store_dt = np.uint16 if spec.dtype == "bf16" else np.float32
    target = np.empty((R, V), dtype=store_dt)
    draft = np.empty((R, V), dtype=store_dt)
    tokens = np.full(R, -1, dtype=np.int64)
    for r0 in range(0, R, row_chunk):
        r1 = min(R, r0 + row_chunk)
        n = r1 - r0
        t = rng.standard_normal(size=(n, V), dtype=np.float32) * np.float32(spec.sigma_t)
        if spec.n_spikes > 0:
            idx = np.stack([rng.choice(V, size=spec.n_spikes, replace=False) for _ in range(n)])
            np.put_along_axis(t, idx, np.take_along_axis(t, idx, axis=1)
                              + np.float32(spec.spike_sigmas * spec.sigma_t), axis=1)
        noise = rng.standard_normal(size=(n, V), dtype=np.float32)
        d = t + noise * sig_d[req_of_row[r0:r1]].astype(np.float32)[:, None]
        target[r0:r1] = _stored(t, spec.dtype)
        draft[r0:r1] = _stored(d, spec.dtype)
        d_f32 = _as_f32(draft[r0:r1], spec.dtype)
        for i in range(n):
            r = r0 + i
            b = req_of_row[r]
            if r == ro[b + 1] - 1:
                continue  # the bonus row takes no draft token
            tokens[r] = _draw_tokens(rng, d_f32[i], float(temp[b]))
    if spec.noprop_frac > 0:
        prop_rows = np.array([r for r in range(R) if r != ro[req_of_row[r] + 1] - 1], dtype=np.int64)
        mark = rng.random(size=prop_rows.size) < spec.noprop_frac
        tokens[prop_rows[mark]] = -1
    return Workload(spec=spec, target=target, draft=draft, draft_tokens=tokens.astype(np.int32),
                    row_offsets=ro.astype(np.int32), temperature=temp, tau=tau,
                    seed=int(spec.verify_seed))


# The five workloads. Index 0 is the small case the oracle finishes in
# seconds; index 2 is the one throughput is quoted on.
CONFIGS = {
    1: Spec(B=1, T=4, V=32000, dtype="f32", sigma_t=2.0, sigma_d=1.0, temperature=1.0, tau=0.0,
            rng_seed=1001, verify_seed=0),
    2: Spec(B=32, T=4, V=128256, dtype="bf16", sigma_t=3.0, n_spikes=8, sigma_d=1.5,
            temperature=0.7, tau=0.0, rng_seed=1002),
    3: Spec(B=64, T=4, V=151936, dtype="bf16", sigma_t=3.0, n_spikes=8, sigma_d=1.5,
            temperature=1.0, tau=(0.1, 0.3, 0.5), rng_seed=1003),
    4: Spec(B=256, T=8, V=256000, dtype="bf16", sigma_t=3.0, sigma_d=2.0, temperature=0.8,
            tau=0.0, rng_seed=1004),
    5: Spec(B=512, T=4, V=152064, dtype="f32", sigma_t=3.0, n_spikes=8, sigma_d=(0.5, 3.0),
            temperature=(0.5, 1.2), greedy_frac=0.1, tau=0.5, gated_frac=0.25, noprop_frac=0.1,
            rng_seed=1005),
}

CONFIG_NAMES = {
    1: "ungated B=1 T=4 V=32000 fp32",
    2: "ungated B=32 T=4 V=128256 bf16",
    3: "gated B=64 T=4 V=151936 bf16",
    4: "ungated B=256 T=8 V=256000 bf16",
    5: "mixed-policy B=512 T=4 V=152064 fp32",
}


def config(cfg: int, verify_seed: int | None = None, rng_seed: int | None = None) -> Workload:
    """One of the five named workloads, optionally with another verify seed or data seed."""
    spec = CONFIGS[cfg]
    if verify_seed is not None:
        spec = replace(spec, verify_seed=int(verify_seed))
    if rng_seed is not None:
        spec = replace(spec, rng_seed=int(rng_seed))
    return generate(spec)


def sampler_filters(B: int, rng_seed: int = 0):
    """A serving-style sampler configuration per request, for the target and for the draft.

    Each side gets its own (top_k [B] int32, top_p [B] float32, min_p [B] float32), drawn
    from values common in serving: top_k in {0 (off), 20, 50}, top_p in {1 (off), 0.9,
    0.95}, min_p in {0 (off), 0.05}. The drafted tokens stay those of the unfiltered
    drafter.
    """
    rng = np.random.default_rng(rng_seed)

    def side():
        return (rng.choice([0, 20, 50], size=B).astype(np.int32),
                rng.choice([1.0, 0.9, 0.95], size=B).astype(np.float32),
                rng.choice([0.0, 0.05], size=B).astype(np.float32))

    return side(), side()

