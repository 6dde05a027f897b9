"""The allocation-free verify (sv_verify_batch_static) against sv_verify_batch.

Both run the same kernels; the static call takes its workspace from the library's per-GPU
array instead of an argument. Three calls in a row on one stream, each with a different
workspace layout (the gated B=64, T=4, V=151936 bf16 batch, then a smaller ragged fp32
batch with unaligned rows, then the first again), must each give the tokens and accept
lengths of sv_verify_batch bit for bit, since the array keeps the previous call's contents.
"""
import numpy as np
import pytest

from lossless_rejection_sampling_row_amd import workloads as wl
from tests.gpu_util import as_batch, say, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_rejection_sampling_row_amd import binding
    binding.load_library()
    yield


def _both(batch, seed):
    import torch
    from lossless_rejection_sampling_row_amd import binding
    g = upload(batch)
    R = int(g["target"].shape[0])
    B = int(g["row_offsets"].numel()) - 1
    ref_t, ref_l = binding.verify_batch(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"],
                                        g["temperature"], g["tau"], seed)
    out_t = torch.full((R,), -7, dtype=torch.int32, device="cuda")
    out_l = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    binding.verify_batch_static(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"], g["temperature"],
                                g["tau"], seed, out_t, out_l)
    torch.cuda.synchronize()
    return ref_t.cpu().numpy(), ref_l.cpu().numpy(), out_t.cpu().numpy(), out_l.cpu().numpy()


def test_static_matches_workspace_call_across_layouts():
    big = as_batch(wl.config(3))
    small = as_batch(wl.generate(wl.Spec(B=7, T=(0, 5), V=1001, dtype="f32", n_spikes=2, sigma_d=1.0,
                                         temperature=(0.5, 1.0), greedy_frac=0.2, tau=(0.0, 0.2),
                                         rng_seed=31, verify_seed=3)))
    for label, batch, seed in (("gated B=64 T=4 V=151936 bf16", big, 5), ("ragged B=7 V=1001 fp32", small, 6),
                               ("gated B=64 T=4 V=151936 bf16 again", big, 7)):
        say(f"[static] {label} seed={seed}")
        rt, rl, st, sl = _both(batch, seed)
        assert np.array_equal(rl, sl), label
        assert np.array_equal(rt, st), label
        assert (sl >= 0).all()
