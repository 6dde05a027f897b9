"""The seeded input generator: deterministic, correctly rounded, right shapes."""
import numpy as np
import pytest

from lossless_rejection_sampling_row_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 30, 200000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0039062, 1e30, -1e-30], dtype=np.float32)])
    # halfway cases: low 16 bits exactly 0x8000
    halfway = (rng.integers(0, 2**16, 1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, halfway[np.isfinite(halfway)]])
    ours = wl.round_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_generator_is_deterministic_and_shaped():
    spec = wl.Spec(B=5, T=(1, 4), V=300, dtype="bf16", n_spikes=8, sigma_d=(0.5, 3.0),
                   temperature=(0.5, 1.2), greedy_frac=0.2, tau=0.5, gated_frac=0.4,
                   noprop_frac=0.2, rng_seed=42, verify_seed=9)
    a, b = wl.generate(spec), wl.generate(spec)
    for k in ("target", "draft", "draft_tokens", "row_offsets", "temperature", "tau"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    ro = a.row_offsets
    assert ro[0] == 0 and ro[-1] == a.R and np.all(np.diff(ro) >= 2)
    assert a.target.dtype == np.uint16 and a.target.shape == (a.R, 300)
    last = ro[1:] - 1
    assert np.all(a.draft_tokens[last] == -1)
    prop = np.setdiff1d(np.arange(a.R), last)
    assert np.all(a.draft_tokens[prop] < 300) and np.all(a.draft_tokens[prop] >= -1)
    assert (a.temperature == 0).sum() == 1 and (a.tau > 0).sum() == 2
    assert a.seed == 9


@pytest.mark.parametrize("cfg,shape", [(1, (1, 5, 32000, "f32"))])
def test_small_config_shape(cfg, shape):
    w = wl.config(cfg)
    assert (w.B, w.R, w.V, w.dtype) == shape


def test_spikes_are_eight_sigma():
    spec = wl.Spec(B=2, T=1, V=1000, n_spikes=8, sigma_t=3.0, sigma_d=0.0, dtype="f32", rng_seed=3)
    w = wl.generate(spec)
    # 8 tokens per row sit about 24 above the N(0, 3) bulk
    top = np.sort(w.target, axis=1)[:, -8:]
    rest = np.sort(w.target, axis=1)[:, :-8]
    assert np.all(top.min(axis=1) > rest.max(axis=1))
    assert np.all(np.abs(top.mean(axis=1) - 24.0) < 6.0)
