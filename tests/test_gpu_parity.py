"""GPU parity: the HIP verify path against the CPU oracle, element by element.

The bar:
* accept lengths and emitted token ids are bit-exact on every request the
  oracle does not flag;
* verdicts are bit-exact;
* accept uniforms are bit-exact;
* p(D), q(D), mu(D) agree to 1e-5 relative;
* the residual mass agrees to max(1e-5 * R, 2e-6).

Flagged requests have a decision within 1e-6 of a boundary, so fp32 may
decide them the other way. They are counted here; their rate over the
benchmark batches at scale is the subject of test_gpu_flag_rate.py.
"""
import numpy as np
import pytest

from lossless_rejection_sampling_row_amd import workloads as wl
from tests.gpu_util import (Parity, as_batch, check_properties, compare, run_gpu, run_oracle, say,
                            upload)
from tests.helpers import batch_from_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from lossless_rejection_sampling_row_amd import binding
    binding.load_library()
    yield


def _parity(batch, seeds=(None,), requests=None, label=""):
    """Both entry points against the oracle: the diagnostic call (with row records, a kernel
    of its own) and the plain call."""
    tot = Parity()
    g = upload(batch)
    for s in seeds:
        say(f"[parity] {label} seed={s if s is not None else batch['seed']}")
        gpu = run_gpu(batch, seed=s, gpu=g)
        fast = run_gpu(batch, seed=s, gpu=g, diag=False)
        ora = run_oracle(batch, seed=s, requests=requests)
        tot.add(compare(batch, gpu, ora, requests=requests))
        compare(batch, fast, ora, requests=requests, check_diag=False)
        if requests is not None:
            check_properties(batch, gpu)
            check_properties(batch, fast)
    say(f"[parity] {label}: {tot}")
    return tot


def test_config1_many_seeds():
    w = as_batch(wl.config(1))
    tot = _parity(w, seeds=range(200), label="ungated B=1 T=4 V=32000 fp32")
    assert tot.flagged_rows <= 1e-4 * tot.rows + 5


@pytest.mark.parametrize("V", [1, 2, 3, 5, 8, 64, 1000, 2049, 4097, 16384, 16385, 40000])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_micro_batches(V, dtype):
    spec = wl.Spec(B=24, T=(0, 6), V=V, dtype=dtype, sigma_t=2.5, n_spikes=min(8, V // 4),
                   sigma_d=(0.3, 2.5), temperature=(0.4, 1.3), greedy_frac=0.15, tau=(0.0, 0.05, 0.3, 0.6),
                   noprop_frac=0.1, rng_seed=7000 + V, verify_seed=V)
    batch = as_batch(wl.generate(spec))
    _parity(batch, seeds=range(12), label=f"micro V={V} {dtype}")


@pytest.mark.parametrize("V,dtype", [(300001, "bf16"), (300001, "f32"), (524288, "bf16")])
def test_long_rows(V, dtype):
    # Rows longer than any workload's: 300001 logits are not 16-byte aligned in either dtype
    # (the scalar path); 524288 aligned bf16 logits give pass 1 and pass 2 their largest
    # per-row wave counts.
    spec = wl.Spec(B=5, T=(1, 4), V=V, dtype=dtype, sigma_t=3.0, n_spikes=8, sigma_d=(0.5, 2.0),
                   temperature=(0.6, 1.2), greedy_frac=0.2, tau=(0.0, 0.3), rng_seed=7100 + V % 89,
                   verify_seed=V)
    batch = as_batch(wl.generate(spec))
    _parity(batch, seeds=range(3), label=f"long rows V={V} {dtype}")


@pytest.mark.parametrize("cfg,seeds", [(2, (0, 1, 2)), (3, (0, 1, 2, 3))])
def test_full_config(cfg, seeds):
    batch = as_batch(wl.config(cfg))
    _parity(batch, seeds=seeds, label=wl.CONFIG_NAMES[cfg])


@pytest.mark.parametrize("cfg", [4, 5])
def test_full_size_sampled(cfg):
    batch = as_batch(wl.config(cfg))
    B = len(batch["row_offsets"]) - 1
    reqs = sorted(np.random.default_rng(cfg).choice(B, size=48, replace=False).tolist())
    _parity(batch, seeds=(0,), requests=reqs, label=wl.CONFIG_NAMES[cfg])


def test_determinism_and_seed_dependence():
    batch = as_batch(wl.config(3))
    g = upload(batch)
    a = run_gpu(batch, seed=11, gpu=g)
    for _ in range(5):
        b = run_gpu(batch, seed=11, gpu=g)
        assert np.array_equal(a.out_tokens, b.out_tokens)
        assert np.array_equal(a.out_accept_len, b.out_accept_len)
        assert np.array_equal(a.p_D.view(np.int64), b.p_D.view(np.int64))
        assert np.array_equal(a.resid_mass.view(np.int64), b.resid_mass.view(np.int64))
    c = run_gpu(batch, seed=12, gpu=g)
    assert not np.array_equal(a.out_tokens, c.out_tokens)
    for _ in range(3):  # the plain call: same tokens, run after run
        f = run_gpu(batch, seed=11, gpu=g, diag=False)
        assert np.array_equal(a.out_tokens, f.out_tokens)
        assert np.array_equal(a.out_accept_len, f.out_accept_len)


def test_stats_counters():
    batch = as_batch(wl.config(5))
    gpu = run_gpu(batch, seed=3)
    ro = batch["row_offsets"]
    k = gpu.out_accept_len
    valid = k >= 0
    v = gpu.verdict
    final = ro[:-1][valid] + k[valid]
    assert gpu.stats[0] == valid.sum()
    assert gpu.stats[2] == k[valid].sum()
    assert gpu.stats[3] == (v[final] == 2).sum()
    assert gpu.stats[4] == (v[final] == 3).sum()
    assert gpu.stats[5] == (v[final] == 4).sum()
    assert gpu.stats[1] == k[valid].sum() + gpu.stats[3] + gpu.stats[4]
    assert gpu.stats[6] == ((batch["temperature"] == 0) & valid).sum()
    assert gpu.stats[7] == (~valid).sum()
    assert gpu.stats[8] == k[valid].sum() + gpu.stats[3]            # offered = accepted + rejected
    last = ro[1:][valid] - 1
    noprop = (v[final] == 4) & (final < last)
    assert gpu.stats[9] == noprop.sum() and gpu.stats[9] > 0
    assert gpu.stats[10] == 0
    # Drafted ids outside [0, V) other than -1 read as no proposal, and are counted as bad.
    V = batch["target"].shape[1]
    bad = dict(batch)
    bad["draft_tokens"] = np.array(batch["draft_tokens"], copy=True)
    holes = np.flatnonzero(bad["draft_tokens"] == -1)
    bad["draft_tokens"][holes[0::3]] = V + 3
    bad["draft_tokens"][holes[1::3]] = -9
    g2 = run_gpu(bad, seed=3)
    assert np.array_equal(g2.out_tokens, gpu.out_tokens) and np.array_equal(g2.out_accept_len, k)
    assert np.array_equal(g2.stats[:10], gpu.stats[:10])
    dfin = bad["draft_tokens"][final]
    assert g2.stats[10] == (noprop & (dfin != -1)).sum() and g2.stats[10] > 0


# ---------------------------------------------------------------- edge cases

def _rows(tl, dl, toks, ro, T, tau, seed=0):
    return batch_from_rows(np.asarray(tl, np.float32), np.asarray(dl, np.float32), toks, ro, T, tau, seed)


def _both(batch, label):
    say(f"[edge] {label}")
    gpu = run_gpu(batch)
    ora = run_oracle(batch)
    compare(batch, gpu, ora)
    compare(batch, run_gpu(batch, diag=False), ora, check_diag=False)
    return gpu, ora


def test_empty_batch():
    import torch
    from lossless_rejection_sampling_row_amd import binding
    say("[edge] empty batch")
    z = torch.zeros((0, 7), dtype=torch.float32, device="cuda")
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    toks, lens = binding.verify_batch(z, z, e, torch.zeros(1, dtype=torch.int32, device="cuda"),
                                      torch.zeros(0, device="cuda"), torch.zeros(0, device="cuda"), 0)
    torch.cuda.synchronize()
    assert toks.numel() == 0 and lens.numel() == 0


def test_single_row_requests_and_greedy():
    rng = np.random.default_rng(1)
    V = 50
    tl = rng.normal(0, 2, (6, V))
    dl = tl + rng.normal(0, 1, (6, V))
    # requests: [1 row], [2 rows], [3 rows]; temperatures 1, 0, 0.5
    batch = _rows(tl, dl, [-1, 3, -1, 7, 9, -1], [0, 1, 3, 6], [1.0, 0.0, 0.5], [0.0, 0.2, 0.0], seed=5)
    _both(batch, "single-row and greedy requests")


def test_all_null_and_tau_above_one():
    w = wl.generate(wl.Spec(B=16, T=4, V=3000, dtype="bf16", n_spikes=8, sigma_d=1.0, temperature=1.0,
                            tau=1.5, rng_seed=77, verify_seed=1))
    gpu, ora = _both(as_batch(w), "tau > 1: every row NULL")
    assert np.all(gpu.out_accept_len == 0)


def test_identical_draft_always_accepts():
    rng = np.random.default_rng(2)
    V, n, B = 777, 5, 8
    tl = rng.normal(0, 3, (B * n, V)).astype(np.float32)
    toks = np.array([rng.integers(0, V) if (r % n) != n - 1 else -1 for r in range(B * n)])
    # drafter tokens drawn from q = p
    from tests.helpers import target_law
    for r in range(B * n):
        if r % n != n - 1:
            toks[r] = rng.choice(V, p=target_law(tl[r], 1.0))
    batch = _rows(tl, tl, toks, np.arange(0, B * n + 1, n), np.ones(B), np.zeros(B), seed=3)
    gpu, _ = _both(batch, "draft == target")
    assert np.all(gpu.out_accept_len == n - 1)


def test_zero_target_mass_at_draft_token():
    V = 4
    tl = np.array([[0.0, 0.0, -np.inf, 0.0], [0.0, 0.0, 0.0, 0.0]] * 50)
    dl = np.array([[0.0, 0.0, -1e4, 0.0], [0.0, 0.0, 0.0, 0.0]] * 50)
    toks = np.tile([2, -1], 50)
    batch = _rows(tl, dl, toks, np.arange(0, 101, 2), np.ones(50), np.zeros(50), seed=9)
    gpu, _ = _both(batch, "p(D) = 0 with underflowed q(D)")
    assert np.all(gpu.out_accept_len == 0) and np.all(gpu.out_tokens[0::2] != 2)


def test_invalid_inputs_fail_closed():
    V = 9
    rng = np.random.default_rng(3)
    tl = rng.normal(0, 1, (12, V))
    dl = tl + rng.normal(0, 1, (12, V))
    toks = np.array([1, 2, 3, -1] * 3)
    ro = [0, 4, 8, 12]
    base = dict(T=[1.0, 1.0, 1.0], tau=[0.0, 0.0, 0.0])
    # request 0: NaN target on row 0; request 1: bad temperature; request 2 valid
    t2 = tl.copy()
    t2[0, 3] = np.nan
    batch = _rows(t2, dl, toks, ro, [1.0, -2.0, 0.8], base["tau"], seed=4)
    gpu, _ = _both(batch, "NaN row, bad temperature")
    assert gpu.out_accept_len[0] == -1 and gpu.out_accept_len[1] == -1 and gpu.out_accept_len[2] >= 0
    # +inf draft logit, tau NaN, all -inf target row
    d3 = dl.copy()
    d3[4, 0] = np.inf
    t3 = tl.copy()
    t3[8, :] = -np.inf
    batch = _rows(t3, d3, toks, ro, [1.0, 1.0, 1.0], [float("nan"), 0.0, 0.0], seed=4)
    gpu, _ = _both(batch, "+inf draft, NaN tau, all -inf row")
    assert np.all(gpu.out_accept_len == -1)
    # out-of-range draft tokens are "no proposal"
    batch = _rows(tl, dl, [V, 2, 3, -1, 1, -5, 3, -1, 1, 2, 3, -1], ro, [1.0, 0.0, 1.0], [0.0, 0.0, 0.0], seed=4)
    gpu, _ = _both(batch, "out-of-range draft tokens")
    assert gpu.out_accept_len[0] == 0
    # broken row offsets fail the whole batch
    for bad_ro in ([0, 4, 4, 12], [0, 5, 3, 12], [1, 4, 8, 12], [0, 4, 8, 11]):
        batch = _rows(tl, dl, toks, bad_ro, [1.0] * 3, [0.0] * 3, seed=4)
        say(f"[edge] broken row_offsets {bad_ro}")
        gpu = run_gpu(batch)
        assert np.all(gpu.out_accept_len == -1) and np.all(gpu.out_tokens == -1)


def test_unaligned_rows_take_the_scalar_path():
    for dtype, V in (("bf16", 1001), ("f32", 1001), ("bf16", 12), ("f32", 6)):
        spec = wl.Spec(B=10, T=(1, 5), V=V, dtype=dtype, n_spikes=2, sigma_d=1.0, temperature=(0.5, 1.0),
                       greedy_frac=0.2, tau=(0.0, 0.2), rng_seed=V, verify_seed=2)
        _parity(as_batch(wl.generate(spec)), seeds=range(4), label=f"unaligned V={V} {dtype}")


def test_ties_go_to_lower_index():
    # greedy rows with tied maxima: argmax must be the lowest index
    V = 300
    tl = np.zeros((4, V))
    tl[:, [17, 150, 299]] = 5.0
    dl = np.zeros((4, V))
    dl[:, [40, 41]] = 3.0
    batch = _rows(tl, dl, [40, -1, 17, -1], [0, 2, 4], [0.0, 0.0], [0.0, 0.5], seed=0)
    gpu, _ = _both(batch, "greedy ties")
    assert gpu.out_tokens[0] == 17 and gpu.out_tokens[2] == 17


def test_long_windows():
    # windows longer than a wavefront of rows
    spec = wl.Spec(B=3, T=(60, 80), V=500, dtype="f32", sigma_d=0.05, temperature=1.0, tau=0.0,
                   rng_seed=5, verify_seed=5)
    _parity(as_batch(wl.generate(spec)), seeds=range(3), label="long windows")


def test_chi_square_on_gpu(stat_samples):
    from tests.helpers import chi2_threshold, chi_square, emitted_tokens, repeated_window, target_law
    from tests.test_oracle_sampled import CHI_D, CHI_T
    T = 0.7
    p = target_law(CHI_T, T)
    for n_draft, tau in ((4, 0.0), (4, 0.3)):
        batch = repeated_window(CHI_T, CHI_D, stat_samples + 50, n_draft, T, tau, np.random.default_rng(41), seed=41)
        say(f"[stats] chi-square n_draft={n_draft} tau={tau}")
        gpu = run_gpu(batch, diag=False)
        toks = emitted_tokens(gpu.out_tokens, gpu.out_accept_len, batch["row_offsets"])[:stat_samples]
        assert toks.size == stat_samples
        assert chi_square(toks, p) < chi2_threshold(5, 1e-4)
