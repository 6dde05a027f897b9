"""GPU parity of the per-row acceptance sums (sv_row_acceptance) against the oracle.

sum_x min(p, mu) and sum_x p q per proposal row (oracle.verify.row_sums). Both
sums add positive float32 terms per lane and merge in fp64, so the bar is 1e-5
relative (absolute 1e-9 for tiny sums). Rows with a token whose q lies within
1e-6 of the gate are skipped and counted, since a float32 gate decision there
may legitimately differ. NaN must match NaN exactly.

A statistical check ties the sums to the sampler: over many seeds, the
frequency with which the verify kernels accept a request's first draft matches
the first row's sum min(p, mu) (the acceptance the pages compare measured rates
against: mlxcel PR #992, section The acceptance ceiling).
"""
import numpy as np
import pytest

from lossless_rejection_sampling_row_amd import workloads as wl
from oracle import verify as ov
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


def _gpu_sums(batch, g=None):
    import torch
    from lossless_rejection_sampling_row_amd import binding
    g = g or upload(batch)
    smin, spq = binding.row_acceptance(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"],
                                       g["temperature"], g["tau"], tau_step=g.get("tau_step"),
                                       min_cum=g.get("min_cum"), target_filter=g.get("target_filter"),
                                       draft_filter=g.get("draft_filter"))
    torch.cuda.synchronize()
    return smin.cpu().numpy().astype(np.float64), spq.cpu().numpy().astype(np.float64)


def _oracle_sums(batch):
    return ov.row_sums(batch["target"], batch["draft"], batch["draft_tokens"], batch["row_offsets"],
                       batch["temperature"], batch["tau"], batch["dtype"], tau_step=batch.get("tau_step"),
                       min_cum=batch.get("min_cum"), target_filter=batch.get("target_filter"),
                       draft_filter=batch.get("draft_filter"))


def _compare(batch, label):
    gm, gp = _gpu_sums(batch)
    om, op, near = _oracle_sums(batch)
    assert np.array_equal(np.isnan(gm), np.isnan(om)), f"{label}: NaN pattern of sum min differs"
    assert np.array_equal(np.isnan(gp), np.isnan(op)), f"{label}: NaN pattern of sum pq differs"
    rows = np.isfinite(om) & ~near
    for name, a, b in (("sum min", gm, om), ("sum pq", gp, op)):
        err = np.abs(a[rows] - b[rows])
        tol = np.maximum(1e-5 * np.abs(b[rows]), 1e-9)
        worst = int(np.argmax(err / tol)) if rows.any() else 0
        assert np.all(err <= tol), f"{label}: {name} row {np.flatnonzero(rows)[worst]} gpu {a[rows][worst]} oracle {b[rows][worst]}"
    say(f"[sums] {label}: {int(rows.sum())} rows compared, {int(near.sum())} near the gate")
    return int(rows.sum())


@pytest.mark.parametrize("V,dtype", [(1, "f32"), (5, "bf16"), (64, "f32"), (2049, "bf16"), (16385, "f32"),
                                     (40000, "bf16")])
def test_micro_batches(V, dtype):
    spec = wl.Spec(B=24, T=(0, 6), V=V, dtype=dtype, sigma_t=2.5, n_spikes=min(8, V // 4), sigma_d=(0.3, 2.5),
                   temperature=(0.4, 1.3), greedy_frac=0.15, tau=(0.0, 0.05, 0.3, 0.6), noprop_frac=0.1,
                   rng_seed=8100 + V, verify_seed=V)
    assert _compare(as_batch(wl.generate(spec)), f"micro V={V} {dtype}") > 0 or V == 1


def test_with_schedules_and_floors():
    spec = wl.Spec(B=32, T=(1, 8), V=4096, dtype="bf16", sigma_t=2.5, n_spikes=8, sigma_d=(0.3, 2.0),
                   temperature=(0.5, 1.2), greedy_frac=0.1, tau=(0.0, 0.1, 0.3), noprop_frac=0.05,
                   rng_seed=8300, verify_seed=1)
    batch = as_batch(wl.generate(spec))
    rng = np.random.default_rng(3)
    ro = np.asarray(batch["row_offsets"])
    batch["tau_step"] = rng.choice([0.0, 0.05, 0.2, 0.4], size=int(ro[-1])).astype(np.float32)
    batch["min_cum"] = rng.choice([0.0, 1e-3, 0.05, 0.3], size=len(batch["tau"])).astype(np.float32)
    _compare(batch, "schedules and floors")


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_config(cfg):
    _compare(as_batch(wl.config(cfg)), wl.CONFIG_NAMES[cfg])


def test_invalid_rows_and_broken_offsets_give_nan():
    spec = wl.Spec(B=6, T=(3, 3), V=512, dtype="f32", sigma_t=2.0, rng_seed=91, verify_seed=2)
    batch = as_batch(wl.generate(spec))
    ro = np.asarray(batch["row_offsets"])
    t = np.array(batch["target"], copy=True)
    t[ro[1] + 1, 7] = np.nan            # request 1: its second row is invalid, so rows 1 and 2 get NaN
    batch["target"] = t
    tau = np.array(batch["tau"], copy=True)
    tau[2] = np.nan                      # request 2 fails closed
    batch["tau"] = tau
    gm, _ = _gpu_sums(batch)
    om, _, _ = _oracle_sums(batch)
    assert np.isfinite(gm[ro[1]]) and np.all(np.isnan(gm[ro[1] + 1:ro[2]]))
    assert np.all(np.isnan(gm[ro[2]:ro[3]]))
    assert np.array_equal(np.isnan(gm), np.isnan(om))
    batch["row_offsets"] = np.array(ro, copy=True)
    batch["row_offsets"][2] = batch["row_offsets"][1]   # not strictly increasing
    gm, gp = _gpu_sums(batch)
    assert np.all(np.isnan(gm)) and np.all(np.isnan(gp))


@pytest.mark.parametrize("tau", [0.0, 0.01])
def test_first_row_acceptance_frequency_matches_sum_min(tau):
    import torch
    from lossless_rejection_sampling_row_amd import binding
    # 64 requests share one window, so one call gives 64 draws of the first row's verdict.
    # V = 300 with these spreads puts q's largest entries around 0.01-0.05, so tau = 0.01
    # gates part of the mass away and the acceptance sits strictly between 0 and 1.
    spec = wl.Spec(B=1, T=(2, 2), V=300, dtype="bf16", sigma_t=2.0, sigma_d=0.6, temperature=1.0, tau=tau,
                   rng_seed=17, verify_seed=0)
    one = as_batch(wl.generate(spec))
    B = 64
    batch = dict(one)
    batch["target"] = np.tile(one["target"], (B, 1))
    batch["draft"] = np.tile(one["draft"], (B, 1))
    batch["draft_tokens"] = np.tile(one["draft_tokens"], B)
    n = len(one["draft_tokens"])
    # sum min(p, mu) is the acceptance when D ~ q, so every request draws its own D from q
    q0 = ov.distribution(ov.decode_logits(np.asarray(one["draft"])[:1], one["dtype"])[0],
                         float(one["temperature"][0]))
    batch["row_offsets"] = np.arange(B + 1, dtype=np.int32) * n
    batch["temperature"] = np.full(B, one["temperature"][0], dtype=np.float32)
    batch["tau"] = np.full(B, one["tau"][0], dtype=np.float32)
    g = upload(batch)
    sm, _ = _gpu_sums(batch, g)
    a = sm[0]
    assert np.allclose(sm[::n], a)
    rng = np.random.default_rng(23)
    hits = tot = 0
    for seed in range(60):
        dt = np.tile(one["draft_tokens"], B).astype(np.int32)
        dt[::n] = rng.choice(q0.size, size=B, p=q0 / q0.sum())
        g["draft_tokens"].copy_(torch.from_numpy(dt))
        _, lens = binding.verify_batch(g["target"], g["draft"], g["draft_tokens"], g["row_offsets"],
                                       g["temperature"], g["tau"], 1000 + seed)
        torch.cuda.synchronize()
        ln = lens.cpu().numpy()
        hits += int((ln >= 1).sum())
        tot += B
    freq = hits / tot
    sd = np.sqrt(a * (1 - a) / tot)
    say(f"[sums] first-row acceptance {freq:.4f} vs sum min {a:.4f} (sd {sd:.4f}, {tot} draws)")
    assert 0.05 < a < 0.95, "the check needs an acceptance away from 0 and 1"
    assert abs(freq - a) < 5 * sd + 1e-3


# ---------------------------------------------------------------- under the filter chain

@pytest.mark.parametrize("V,dtype", [(64, "bf16"), (4097, "f32"), (4099, "bf16"), (20000, "bf16")])
def test_filtered_micro_batches(V, dtype):
    spec = wl.Spec(B=24, T=(1, 6), V=V, dtype=dtype, sigma_t=3.0, n_spikes=min(8, V // 4), sigma_d=(0.5, 2.0),
                   temperature=(0.5, 1.2), greedy_frac=0.1, tau=(0.0, 0.1, 0.3), noprop_frac=0.05,
                   rng_seed=700 + V, verify_seed=1)
    batch = as_batch(wl.generate(spec))
    rng = np.random.default_rng(V)
    B = len(batch["tau"])
    for side in ("target_filter", "draft_filter"):
        batch[side] = (rng.choice([0, 1, 5, 50, V], size=B).astype(np.int32),
                       rng.choice([1.0, 0.5, 0.9, 0.99], size=B).astype(np.float32),
                       rng.choice([0.0, 0.02, 0.2], size=B).astype(np.float32))
    _compare(batch, f"filtered V={V} {dtype}")


def test_filtered_gated_batch_full_size():
    batch = as_batch(wl.config(3))
    batch["target_filter"], batch["draft_filter"] = wl.sampler_filters(len(batch["tau"]), rng_seed=9)
    _compare(batch, "filtered config 3")


def test_invalid_filter_values_give_nan():
    batch = as_batch(wl.generate(wl.Spec(B=6, T=3, V=512, dtype="f32", temperature=1.0, rng_seed=5, verify_seed=1)))
    k = np.zeros(6, np.int32)
    k[2] = -1
    batch["target_filter"] = (k, None, None)
    gm, _ = _gpu_sums(batch)
    ro = batch["row_offsets"]
    assert np.isnan(gm[ro[2]:ro[3]]).all()
    assert np.isfinite(gm[ro[0]:ro[1] - 1]).all()
    _compare(batch, "invalid filter")
