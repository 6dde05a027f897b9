"""Pins for the oracle's Philox4x32-10 and its uniform maps.

The generator is checked against two things outside itself:

* the known-answer vectors published with the Random123 library, which
  accompanies the SC'11 paper that defines Philox;
* PyTorch's header-only ``at::philox_engine`` (ATen/core/PhiloxRNGEngine.h),
  an independent implementation. It is compiled here with g++ and fed the
  same (seed, counter) pairs.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import numpy as np
import pytest

from oracle import philox

# Random123 known-answer tests for philox4x32 with 10 rounds:
# (counter words, key words) -> output words.
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF, 0xFFFFFFFF), (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_known_answers(ctr, key, want):
    got = philox.philox4x32_10(*ctr, *key)
    assert tuple(int(w) for w in got) == want


def test_vectorised_matches_scalar():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2**32, size=(4, 64), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9ABCDEF0
    vec = philox.philox4x32_10(c[0], c[1], c[2], c[3], k0, k1)
    for i in range(64):
        one = philox.philox4x32_10(int(c[0, i]), int(c[1, i]), int(c[2, i]), int(c[3, i]), k0, k1)
        assert all(int(vec[w][i]) == int(one[w]) for w in range(4))


_TORCH_PROG = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    at::philox_engine e(seed, sub, off);
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def torch_philox():
    torch = pytest.importorskip("torch")
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if not os.path.exists(os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")):
        pytest.skip("PhiloxRNGEngine.h not shipped with this torch")
    d = tempfile.mkdtemp(prefix="philox_xcheck_")
    src = os.path.join(d, "p.cpp")
    exe = os.path.join(d, "p")
    with open(src, "w") as f:
        f.write(_TORCH_PROG)
    subprocess.run([gxx, "-std=c++17", "-O1", "-I", inc, src, "-o", exe], check=True)

    def run(triples):
        inp = "\n".join(f"{s} {u} {o}" for s, u, o in triples) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return np.array([[int(t) for t in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64)
    yield run
    shutil.rmtree(d, ignore_errors=True)


def test_matches_torch_engine(torch_philox):
    # at::philox_engine(seed, subsequence, offset): key <- seed; counter words
    # 0-1 <- offset; words 2-3 <- subsequence; four calls give words 0..3.
    rng = np.random.default_rng(1234)
    n = 10000
    seeds = rng.integers(0, 2**63, size=n, dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=n, dtype=np.uint64)
    subs = rng.integers(0, 2**63, size=n, dtype=np.uint64)
    offs = rng.integers(0, 2**63, size=n, dtype=np.uint64)
    # include small and all-ones edge counters
    seeds[:3] = [0, 2**64 - 1, 1]
    subs[:3] = [0, 2**64 - 1, 2**32]
    offs[:3] = [0, 2**64 - 1, 2**32 - 1]
    want = torch_philox(list(zip(seeds.tolist(), subs.tolist(), offs.tolist())))
    m = np.uint64(0xFFFFFFFF)
    k0 = seeds & m
    k1 = seeds >> np.uint64(32)
    got = np.empty_like(want)
    # the key differs per case: evaluate one case at a time in chunks of equal keys
    for i in range(n):
        w = philox.philox4x32_10(int(offs[i] & m), int(offs[i] >> np.uint64(32)),
                                 int(subs[i] & m), int(subs[i] >> np.uint64(32)),
                                 int(k0[i]), int(k1[i]))
        got[i] = [int(x) for x in w]
    assert np.array_equal(got, want)


def test_counter_layout_matches_torch_engine(torch_philox):
    """accept_uniform / race_uniforms use counter (block, tag, j, b) under key = seed."""
    cases = [(0, 0, 0), (7, 3, 2), (2**40 + 5, 511, 4), (2**64 - 1, 2**31 - 1, 8)]
    V = 37
    for seed, b, j in cases:
        sub = j | (b << 32)
        want0 = torch_philox([(seed, sub, 0 | (philox.TAG_ACCEPT << 32))])[0, 0]
        assert philox.accept_uniform(seed, b, j) == float(want0 >> 8) * 2.0 ** -24
        blocks = torch_philox([(seed, sub, blk | (philox.TAG_RACE << 32)) for blk in range((V + 3) // 4)])
        words = blocks.reshape(-1)[:V]
        want_u = ((words >> np.uint64(9)) * 2 + 1).astype(np.float64) * 2.0 ** -24
        assert np.array_equal(philox.race_uniforms(seed, b, j, V), want_u)


def test_uniform_maps_exact_and_in_range():
    w = np.array([0, 1, 255, 256, 0x7FFFFFFF, 0xFFFFFFFF], dtype=np.uint64)
    u = philox.u24(w)
    assert u[0] == 0.0 and u[-1] == 1.0 - 2.0 ** -24
    assert np.all((u >= 0) & (u < 1))
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))          # multiples of 2**-24
    assert np.all(u.astype(np.float32).astype(np.float64) == u)  # exact in fp32
    v = philox.u23_odd(w)
    assert v[0] == 2.0 ** -24 and v[-1] == 1.0 - 2.0 ** -24
    assert np.all((v > 0) & (v < 1))
    assert np.all(v.astype(np.float32).astype(np.float64) == v)
    assert np.all(np.isfinite(-np.log(v))) and np.all(-np.log(v) > 0)


def test_race_uniforms_look_uniform():
    # 4 * 2**14 draws: mean 1/2, variance 1/12, no duplicates beyond birthday rate
    u = philox.race_uniforms(99, 3, 1, 4 * 2 ** 14)
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / u.size)
    assert abs(u.var() - 1 / 12) < 0.01
    E = philox.race_exponentials(99, 3, 1, 4 * 2 ** 14)
    assert abs(E.mean() - 1.0) < 5 / np.sqrt(E.size)
