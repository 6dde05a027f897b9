"""CPU oracle for the speculative-decoding verify sampler.

TEST INFRASTRUCTURE, not product code. It is a plain, slow implementation of
what the verify path computes: float64 numpy, one request and one row at a
time. The HIP library is checked against it. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import, call or run anything in this package. The HIP library and its
binding never do, and this package imports nothing from them.

Modules:

* ``philox``: Philox4x32-10 from its published definition, plus the uniform
  maps.
* ``verify``: the sampled verify rule, decision-boundary flags and
  negative-control rules.
* ``exact``: exact rational laws by enumeration (``fractions``).

What pins each function to something other than itself is listed in the
tests (``tests/test_oracle_*.py``). No function here is "parity unpinned".
"""
from . import exact, philox, verify  # noqa: F401
