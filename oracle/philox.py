"""Philox4x32-10, written out from its published definition (numpy, vectorised).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything under ``oracle/``.
The product path never does.

Source of the definition: J. K. Salmon, M. A. Moraes, R. O. Dror and
D. E. Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11, section on
the Philox family (Philox-4x32 with 10 rounds).

* The state is four 32-bit counter words (c0, c1, c2, c3).
* The key is two 32-bit words (k0, k1).
* One round forms the two 64-bit products M0*c0 and M1*c2. With (hi, lo) the
  halves of each product, the new state is
  (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)).
* Between rounds the key is advanced by the Weyl increments (W0, W1) modulo
  2**32. The first round uses the key unchanged.

The pages fix no generator. Strata PR #3416, section Validation, asks only
that every sampled decision can be rebuilt from captured values and counters.
mlxcel PR #992, section RNG, asks that a seed reproduces a run. A
counter-based generator keyed by (seed, request, position) gives both.

How this library lays out the counter (a reading; the GPU side uses the same
layout, written independently):

    key      = (seed mod 2**32, seed >> 32)
    counter  = (block, tag, j, b)
      tag 0  accept test of row j of request b: block 0, word 0
      tag 1  exponential race of the final row j of request b:
             token x uses block x >> 2, word x & 3
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)
_SHIFT = np.uint64(32)

TAG_ACCEPT = 0
TAG_RACE = 1


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Apply ten Philox-4x32 rounds to counters (c0, c1, c2, c3) under key (k0, k1).

    Counter arguments may be scalars or broadcastable integer arrays. The
    result is a tuple of four ``uint32`` arrays, the output words 0..3.
    """
    shape = np.broadcast(np.asarray(c0), np.asarray(c1), np.asarray(c2), np.asarray(c3)).shape
    x0 = np.broadcast_to(np.asarray(c0, dtype=np.uint64), shape) & _MASK
    x1 = np.broadcast_to(np.asarray(c1, dtype=np.uint64), shape) & _MASK
    x2 = np.broadcast_to(np.asarray(c2, dtype=np.uint64), shape) & _MASK
    x3 = np.broadcast_to(np.asarray(c3, dtype=np.uint64), shape) & _MASK
    key0 = int(k0) & 0xFFFFFFFF
    key1 = int(k1) & 0xFFFFFFFF
    m0 = np.uint64(M0)
    m1 = np.uint64(M1)
    for rnd in range(10):
        if rnd:
            key0 = (key0 + W0) & 0xFFFFFFFF
            key1 = (key1 + W1) & 0xFFFFFFFF
        # Both factors are below 2**32, so each product fits in 64 bits exactly.
        prod0 = m0 * x0
        prod1 = m1 * x2
        hi0, lo0 = prod0 >> _SHIFT, prod0 & _MASK
        hi1, lo1 = prod1 >> _SHIFT, prod1 & _MASK
        x0, x1, x2, x3 = (hi1 ^ x1 ^ np.uint64(key0), lo1,
                          hi0 ^ x3 ^ np.uint64(key1), lo0)
    return tuple(np.asarray(w, dtype=np.uint64).astype(np.uint32) for w in (x0, x1, x2, x3))


def key_of_seed(seed: int) -> tuple[int, int]:
    """Split a 64-bit seed into the two Philox key words (low word first)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32


def u24(word) -> np.ndarray:
    """Uniform on [0, 1): the top 24 bits of a word, times 2**-24 (exact in fp32 and fp64)."""
    w = np.asarray(word, dtype=np.uint64)
    return (w >> np.uint64(8)).astype(np.float64) * 2.0 ** -24


def u23_odd(word) -> np.ndarray:
    """Uniform on the open interval (0, 1): (2*(w >> 9) + 1) * 2**-24.

    Never 0 and never 1, so -ln(u) is finite and positive. Exact in fp32 and fp64.
    """
    w = np.asarray(word, dtype=np.uint64)
    return ((w >> np.uint64(9)) * np.uint64(2) + np.uint64(1)).astype(np.float64) * 2.0 ** -24


def accept_uniform(seed: int, b: int, j: int) -> float:
    """The uniform u for the accept test of row j of request b (tag 0, block 0, word 0)."""
    k0, k1 = key_of_seed(seed)
    w0, _, _, _ = philox4x32_10(0, TAG_ACCEPT, j, b, k0, k1)
    return float(u24(w0))


def race_uniforms(seed: int, b: int, j: int, V: int) -> np.ndarray:
    """Open-interval uniforms for tokens 0..V-1 of the race on row j of request b (tag 1)."""
    k0, k1 = key_of_seed(seed)
    nblk = (int(V) + 3) // 4
    blocks = np.arange(nblk, dtype=np.uint64)
    words = philox4x32_10(blocks, TAG_RACE, j, b, k0, k1)
    flat = np.stack(words, axis=1).reshape(-1)[:V]
    return u23_odd(flat)


def race_exponentials(seed: int, b: int, j: int, V: int) -> np.ndarray:
    """E[x] = -ln(U[x]): i.i.d. unit exponentials, one per token, for the race on row j of request b."""
    return -np.log(race_uniforms(seed, b, j, V))
