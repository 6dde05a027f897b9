"""GPU parity of the lazy position-serial verify (sv_verify_batch_lazy) against the oracle.

The lazy call reads each request's rows only up to its first row that is not
accepted. Its outputs are the plain call's, so the bar is the plain call's:
tokens and accept lengths bit-exact on every request the oracle does not flag.
It streams each row with more waves than the data-parallel pass, so its fp32
partial sums round differently, and flagged requests may differ from the
plain call as they may from the oracle.
"""
import numpy as np
import pytest

from lossless_rejection_sampling_row_amd import workloads as wl
from tests.gpu_util import Parity, as_batch, check_properties, compare, run_oracle, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_rejection_sampling_row_amd import binding
    binding.load_library()
    yield


def _lazy(batch, g, seed, max_rows):
    import torch
    from lossless_rejection_sampling_row_amd import binding
    from tests.gpu_util import GpuResult
    toks, lens = binding.verify_batch(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"],
                                      g["temperature"], g["tau"], seed, lazy_max_rows=max_rows)
    torch.cuda.synchronize()
    return GpuResult(toks.cpu().numpy(), lens.cpu().numpy(), None, None, None, None, None, None, None)


def _max_rows(batch):
    return int(np.diff(np.asarray(batch["row_offsets"])).max())


def _parity(batch, seeds, label, requests=None, max_rows=None):
    tot = Parity()
    g = upload(batch)
    mr = max_rows or _max_rows(batch)
    for s in seeds:
        say(f"[lazy] {label} seed={s} max_rows={mr}")
        gpu = _lazy(batch, g, s, mr)
        ora = run_oracle(batch, seed=s, requests=requests)
        tot.add(compare(batch, gpu, ora, requests=requests, check_diag=False))
        check_properties(batch, gpu)
    say(f"[lazy] {label}: {tot}")
    return tot


@pytest.mark.parametrize("V,dtype", [(1, "f32"), (7, "bf16"), (64, "f32"), (4097, "bf16"), (16384, "f32"),
                                     (40000, "bf16")])
def test_micro_batches(V, dtype):
    spec = wl.Spec(B=24, T=(0, 6), V=V, dtype=dtype, sigma_t=2.5, n_spikes=min(8, V // 4), sigma_d=(0.3, 2.5),
                   temperature=(0.4, 1.3), greedy_frac=0.15, tau=(0.0, 0.05, 0.3, 0.6), noprop_frac=0.1,
                   rng_seed=9700 + V, verify_seed=V)
    batch = as_batch(wl.generate(spec))
    tot = _parity(batch, range(8), f"micro V={V} {dtype}")
    assert tot.flagged_rows <= 1e-4 * tot.rows + 5
    # a looser bound on rows changes nothing
    _parity(batch, (3,), f"micro V={V} {dtype}, max_rows + 5", max_rows=_max_rows(batch) + 5)


@pytest.mark.parametrize("cfg,seeds", [(1, range(20)), (2, (0, 1)), (3, (0, 1))])
def test_full_config(cfg, seeds):
    _parity(as_batch(wl.config(cfg)), seeds, wl.CONFIG_NAMES[cfg])


def test_low_acceptance_batch_sampled():
    batch = as_batch(wl.config(4))
    reqs = list(range(0, 256, 17))
    _parity(batch, (0,), wl.CONFIG_NAMES[4], requests=reqs)


def test_rows_beyond_max_rows_fail_the_batch():
    spec = wl.Spec(B=8, T=(2, 5), V=512, dtype="f32", sigma_t=2.0, rng_seed=5, verify_seed=1)
    batch = as_batch(wl.generate(spec))
    g = upload(batch)
    gpu = _lazy(batch, g, 3, _max_rows(batch) - 1)
    assert np.all(gpu.out_accept_len == -1) and np.all(gpu.out_tokens == -1)


def test_bad_max_rows_is_a_host_error():
    import torch
    from lossless_rejection_sampling_row_amd import binding
    spec = wl.Spec(B=2, T=2, V=64, dtype="f32", rng_seed=1)
    batch = as_batch(wl.generate(spec))
    g = upload(batch)
    for bad in (0, -3, 5000):
        with pytest.raises(binding.SvError):
            binding.verify_batch(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"], g["temperature"],
                                 g["tau"], 1, lazy_max_rows=bad)
    torch.cuda.synchronize()
