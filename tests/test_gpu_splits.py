"""Outputs do not depend on how rows are split over waves.

sv_set_tuning forces the pass-1 split w1 (waves per potential proposal row) and the
pass-2 split w2 (waves per request's last row). A split changes only the order of the
floating-point sums, so tokens and accept lengths must be identical for every split on
every request the oracle does not flag, on the gated B=64, T=4, V=151936 bf16 batch, a
ragged micro batch and the unaligned scalar path. The p(D) bits are expected to move with
w1 on some rows: that shows the override reaches the kernels.
"""
import numpy as np
import pytest

from lossless_rejection_sampling_row_amd import workloads as wl
from tests.gpu_util import as_batch, run_gpu, run_oracle, say, upload

pytestmark = pytest.mark.gpu

W1 = (1, 2, 4, 16)
W2 = (1, 7, 48)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_rejection_sampling_row_amd import binding
    binding.load_library()
    binding.set_tuning()
    yield
    binding.set_tuning()


def _batches():
    yield "gated B=64 T=4 V=151936 bf16", as_batch(wl.config(3)), (0, 1)
    yield "ragged micro V=40000 bf16", as_batch(wl.generate(wl.Spec(
        B=24, T=(0, 6), V=40000, dtype="bf16", n_spikes=8, sigma_d=(0.3, 2.5), temperature=(0.4, 1.3),
        greedy_frac=0.15, tau=(0.0, 0.05, 0.3, 0.6), noprop_frac=0.1, rng_seed=4242, verify_seed=3))), (3, 4)
    yield "unaligned V=1001 f32", as_batch(wl.generate(wl.Spec(
        B=10, T=(1, 5), V=1001, dtype="f32", n_spikes=2, sigma_d=1.0, temperature=(0.5, 1.0),
        greedy_frac=0.2, tau=(0.0, 0.2), rng_seed=17, verify_seed=2))), (5,)


@pytest.mark.parametrize("which", [0, 1, 2])
def test_tokens_identical_across_splits(which):
    from lossless_rejection_sampling_row_amd import binding
    label, batch, seeds = list(_batches())[which]
    ro = np.asarray(batch["row_offsets"], dtype=np.int64)
    g = upload(batch)
    for s in seeds:
        ora = run_oracle(batch, seed=s)
        keep = ora.flags == 0
        binding.set_tuning()
        ref = run_gpu(batch, seed=s, gpu=g)
        pd_bits = {ref.p_D.tobytes()}
        try:
            for w1 in W1:
                for w2 in W2:
                    binding.set_tuning(w1=w1, w2=w2)
                    assert binding.get_tuning() == {"w1": w1, "w2": w2}
                    say(f"[splits] {label} seed={s} w1={w1} w2={w2}")
                    got = run_gpu(batch, seed=s, gpu=g)
                    pd_bits.add(got.p_D.tobytes())
                    for b in np.flatnonzero(keep):
                        lo, hi = int(ro[b]), int(ro[b + 1])
                        assert got.out_accept_len[b] == ref.out_accept_len[b], (label, s, w1, w2, b)
                        assert np.array_equal(got.out_tokens[lo:hi], ref.out_tokens[lo:hi]), (label, s, w1, w2, b)
                    # and both agree with the oracle
                    assert np.array_equal(got.out_accept_len[keep], ora.out_accept_len[keep])
        finally:
            binding.set_tuning()
        if which == 0:
            assert len(pd_bits) > 1, "p(D) bits identical under every split: the override did not reach the kernels"
