"""GPU parity of the sampler-match comparison rule (mlxcel PR #992, sections The premise
correction and The acceptance ceiling) against the oracle's rule="sampler_match".

The bar: accept lengths and emitted tokens bit-exact on every request the oracle
does not flag (F3: two race keys within a relative 1e-6), flagged rows below
1e-4 of all rows; fail-closed cases identical; the GPU's emitted stream passes
the page's chi-square recipe and accepts at sum_x p(x) q(x).

Synthetic drafts rarely equal a fresh target draw, so some batches feed the
oracle's own draw at a request's stop row back as its drafted token: that row
then accepts and the window goes deeper.
"""
import numpy as np
import pytest

from lossless_rejection_sampling_row_amd import workloads as wl
from oracle import verify as ov
from tests.gpu_util import as_batch, say, upload
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


def _gpu_run(batch, seed=None, g=None):
    import torch
    from lossless_rejection_sampling_row_amd import binding
    g = g if g is not None else upload(batch)
    toks, lens = binding.verify_sampler_match(g["target"], g["draft_tokens"], g["row_offsets"], g["temperature"],
                                              batch["seed"] if seed is None else seed)
    torch.cuda.synchronize()
    return toks.cpu().numpy(), lens.cpu().numpy()


def _oracle(batch, seed=None, requests=None):
    return ov.verify_batch(batch["target"], batch["draft"], batch["draft_tokens"], batch["row_offsets"],
                           batch["temperature"], batch["tau"], batch["seed"] if seed is None else seed,
                           batch["dtype"], requests=requests, rule="sampler_match")


def _deepen(batch, seed, frac=0.6, rounds=3, rng_seed=0):
    """Feed the oracle's stop-row draw back as the drafted token for a fraction of requests."""
    batch = dict(batch)
    batch["draft_tokens"] = np.array(batch["draft_tokens"], dtype=np.int32, copy=True)
    ro = np.asarray(batch["row_offsets"], dtype=np.int64)
    pick = np.random.default_rng(rng_seed).random(ro.size - 1) < frac
    for _ in range(rounds):
        ora = _oracle(batch, seed=seed, requests=np.flatnonzero(pick).tolist())
        for b in np.flatnonzero(pick):
            k = int(ora.out_accept_len[b])
            if 0 <= k < ro[b + 1] - ro[b] - 1:
                batch["draft_tokens"][ro[b] + k] = ora.out_tokens[ro[b] + k]
    return batch


def _compare(batch, toks, lens, ora, requests=None):
    ro = np.asarray(batch["row_offsets"], dtype=np.int64)
    todo = range(ro.size - 1) if requests is None else requests
    n_rows = n_flag = 0
    for b in todo:
        lo, hi = int(ro[b]), int(ro[b + 1])
        n_rows += hi - lo
        if ora.flags[b]:
            n_flag += hi - lo
            continue
        ctx = f"request {b} rows {lo}..{hi - 1}"
        assert lens[b] == ora.out_accept_len[b], f"{ctx}: accept_len gpu {lens[b]} oracle {ora.out_accept_len[b]}"
        assert np.array_equal(toks[lo:hi], ora.out_tokens[lo:hi]), \
            f"{ctx}: tokens gpu {toks[lo:hi]} oracle {ora.out_tokens[lo:hi]}"
    return n_rows, n_flag


def _parity(batch, seeds, label, requests=None, deepen=True):
    rows = flagged = accepted = 0
    for s in seeds:
        b = _deepen(batch, s) if deepen else batch
        say(f"[match] {label} seed={s}")
        toks, lens = _gpu_run(b, seed=s)
        ora = _oracle(b, seed=s, requests=requests)
        r, f = _compare(b, toks, lens, ora, requests)
        rows += r
        flagged += f
        accepted += int(lens[lens > 0].sum())
    say(f"[match] {label}: rows {rows} flagged rows {flagged} accepted tokens {accepted}")
    return rows, flagged, accepted


@pytest.mark.parametrize("V", [1, 2, 5, 64, 1000, 4097, 40000])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_micro_batches(V, dtype):
    spec = wl.Spec(B=24, T=(0, 6), V=V, dtype=dtype, sigma_t=2.5, n_spikes=min(8, V // 4),
                   sigma_d=(0.3, 2.5), temperature=(0.4, 1.3), greedy_frac=0.15, tau=(0.0, 0.3),
                   noprop_frac=0.1, rng_seed=9100 + V, verify_seed=V)
    rows, flagged, accepted = _parity(as_batch(wl.generate(spec)), range(6), f"micro V={V} {dtype}")
    assert flagged <= 1e-4 * rows
    if V > 1:
        assert accepted > 0


@pytest.mark.parametrize("cfg,seeds", [(2, (0, 1)), (3, (0, 1, 2))])
def test_full_config(cfg, seeds):
    rows, flagged, _ = _parity(as_batch(wl.config(cfg)), seeds, wl.CONFIG_NAMES[cfg])
    assert flagged <= 1e-4 * rows


@pytest.mark.parametrize("cfg", [4, 5])
def test_full_size_sampled(cfg):
    batch = as_batch(wl.config(cfg))
    B = len(batch["row_offsets"]) - 1
    reqs = sorted(np.random.default_rng(cfg).choice(B, size=32, replace=False).tolist())
    say(f"[match] {wl.CONFIG_NAMES[cfg]} sampled")
    toks, lens = _gpu_run(batch, seed=0)
    ora = _oracle(batch, seed=0, requests=reqs)
    _compare(batch, toks, lens, ora, reqs)
    ro = np.asarray(batch["row_offsets"], dtype=np.int64)
    dt = np.asarray(batch["draft_tokens"])
    V = np.asarray(batch["target"]).shape[1]
    for b in range(B):  # every request: a prefix of the drafts, then one draw
        lo, hi = int(ro[b]), int(ro[b + 1])
        k = int(lens[b])
        assert 0 <= k <= hi - lo - 1
        assert np.array_equal(toks[lo:lo + k], dt[lo:lo + k])
        assert 0 <= toks[lo + k] < V and np.all(toks[lo + k + 1:hi] == -1)


def test_greedy_is_argmax_against_argmax():
    rng = np.random.default_rng(12)
    V, n, B = 300, 4, 16
    tl = rng.normal(0, 1, (B * n, V)).astype(np.float32)
    tl[:, 77] = tl.max(axis=1) + (rng.random(B * n) < 0.3)  # ties between 77 and the old max
    am = np.argmax(tl, axis=1)
    toks = np.where(rng.random(B * n) < 0.7, am, (am + 1) % V)
    toks[n - 1::n] = -1
    batch = batch_from_rows(tl, tl, toks, np.arange(0, B * n + 1, n), np.zeros(B), np.zeros(B), seed=1)
    say("[match] greedy")
    g_toks, g_lens = _gpu_run(batch)
    ora = ov.verify_batch(batch["target"], batch["draft"], batch["draft_tokens"], batch["row_offsets"],
                          batch["temperature"], batch["tau"], 1, "f32", rule="argmax")
    assert np.array_equal(g_toks, ora.out_tokens) and np.array_equal(g_lens, ora.out_accept_len)
    assert (g_lens > 0).any() and (g_lens < n - 1).any()


def test_invalid_inputs_fail_closed():
    V = 9
    rng = np.random.default_rng(3)
    tl = rng.normal(0, 1, (12, V)).astype(np.float32)
    ro = [0, 4, 8, 12]
    t2 = tl.copy()
    t2[0, 3] = np.nan       # request 0: NaN on its first row
    t2[7, :] = -np.inf      # request 1: all -inf on its last row, reached when rows 4..6 accept
    t2[11, 2] = np.inf      # request 2: +inf on its last row
    # drafts equal to each row's greedy argmax, so greedy requests walk to their last row
    am = np.argmax(np.where(np.isfinite(t2), t2, -1e30), axis=1)
    toks = np.where(np.arange(12) % 4 == 3, -1, am)
    batch = batch_from_rows(t2, t2, toks, ro, [1.0, 0.0, 0.0], [0.0] * 3, seed=4)
    say("[match] NaN, all -inf and +inf rows")
    g_toks, g_lens = _gpu_run(batch)
    ora = _oracle(batch)
    assert np.array_equal(g_lens, ora.out_accept_len) and np.array_equal(g_toks, ora.out_tokens)
    assert np.all(g_lens == -1)
    # a bad row behind the stop is never read as a decision
    t3 = tl.copy()
    t3[3, 0] = np.nan
    d0 = (int(np.argmax(t3[0])) + 1) % V
    batch = batch_from_rows(t3, t3, [d0, 1, 1, -1] + [1, 2, 3, -1] * 2, ro, [0.0, 1.0, -2.0],
                            [0.0] * 3, seed=4)
    say("[match] stop before a bad row, bad temperature")
    g_toks, g_lens = _gpu_run(batch)
    ora = _oracle(batch)
    assert np.array_equal(g_lens, ora.out_accept_len) and np.array_equal(g_toks, ora.out_tokens)
    assert g_lens[0] == 0 and g_lens[2] == -1
    for bad_ro in ([0, 4, 4, 12], [0, 5, 3, 12], [1, 4, 8, 12], [0, 4, 8, 11]):
        batch = batch_from_rows(tl, tl, [1, 2, 3, -1] * 3, bad_ro, [1.0] * 3, [0.0] * 3, seed=4)
        say(f"[match] broken row_offsets {bad_ro}")
        g_toks, g_lens = _gpu_run(batch)
        assert np.all(g_lens == -1) and np.all(g_toks == -1)


def test_unaligned_rows_take_the_scalar_path():
    for dtype, V in (("bf16", 1001), ("f32", 1001), ("bf16", 12), ("f32", 6)):
        spec = wl.Spec(B=10, T=(1, 5), V=V, dtype=dtype, n_spikes=2, sigma_d=1.0, temperature=(0.5, 1.0),
                       greedy_frac=0.2, tau=(0.0, 0.2), rng_seed=V, verify_seed=2)
        _parity(as_batch(wl.generate(spec)), range(3), f"unaligned V={V} {dtype}")


def test_empty_batch():
    import torch
    from lossless_rejection_sampling_row_amd import binding
    say("[match] empty batch")
    z = torch.zeros((0, 7), dtype=torch.float32, device="cuda")
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    toks, lens = binding.verify_sampler_match(z, e, torch.zeros(1, dtype=torch.int32, device="cuda"),
                                              torch.zeros(0, device="cuda"), 0)
    torch.cuda.synchronize()
    assert toks.numel() == 0 and lens.numel() == 0


def test_chi_square_and_acceptance_on_gpu(stat_samples):
    from tests.helpers import chi2_threshold, chi_square, emitted_tokens, repeated_window, target_law
    from tests.test_oracle_sampled import CHI_D, CHI_T
    T = 0.7
    p = target_law(CHI_T, T)
    q = target_law(CHI_D, T)
    batch = repeated_window(CHI_T, CHI_D, stat_samples + 50, 4, T, 0.0, np.random.default_rng(43), seed=43)
    say("[match] chi-square")
    toks, lens = _gpu_run(batch)
    em = emitted_tokens(toks, lens, batch["row_offsets"])[:stat_samples]
    assert em.size == stat_samples
    assert chi_square(em, p) < chi2_threshold(5, 1e-4)
    # acceptance of the first row: sum_x p(x) q(x)
    n = lens.size
    spq = float((p * q).sum())
    acc = float((lens >= 1).mean())
    assert abs(acc - spq) < 4.5 * np.sqrt(spq * (1 - spq) / n), (acc, spq)
