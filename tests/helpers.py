"""Small builders shared by the tests: batches from explicit logits, drafter draws, chi-square."""
import numpy as np
from scipy import stats


def batch_from_rows(target_rows, draft_rows, draft_tokens, row_offsets, temperature, tau, seed=0):
    """A verify batch in the C-ABI layout from explicit fp32 logits (exact values)."""
    return dict(
        target=np.ascontiguousarray(target_rows, dtype=np.float32),
        draft=np.ascontiguousarray(draft_rows, dtype=np.float32),
        draft_tokens=np.ascontiguousarray(draft_tokens, dtype=np.int32),
        row_offsets=np.ascontiguousarray(row_offsets, dtype=np.int32),
        temperature=np.ascontiguousarray(temperature, dtype=np.float32),
        tau=np.ascontiguousarray(tau, dtype=np.float32),
        seed=int(seed),
        dtype="f32",
    )


def repeated_window(t_logits, d_logits, n_requests, n_draft, T, tau, rng, seed=0):
    """n_requests identical windows: every row has the same target and draft logits.

    The drafter draws each row's token from q = softmax(d_logits / T) with the
    test's own numpy RNG (argmax at T == 0).
    """
    V = len(t_logits)
    n_rows = n_draft + 1
    R = n_requests * n_rows
    target = np.tile(np.asarray(t_logits, dtype=np.float32), (R, 1))
    draft = np.tile(np.asarray(d_logits, dtype=np.float32), (R, 1))
    d64 = np.asarray(d_logits, dtype=np.float32).astype(np.float64)
    if T == 0:
        toks = np.full(R, int(np.argmax(d64)), dtype=np.int64)
    else:
        q = target_law(d_logits, T)
        toks = rng.choice(V, size=R, p=q)
    toks[n_rows - 1::n_rows] = -1
    ro = np.arange(0, R + 1, n_rows)
    return batch_from_rows(target, draft, toks, ro, np.full(n_requests, T), np.full(n_requests, tau), seed)


def emitted_tokens(out_tokens, out_accept_len, row_offsets):
    toks = []
    for b, k in enumerate(out_accept_len):
        if k < 0:
            continue
        lo = row_offsets[b]
        toks.extend(int(t) for t in out_tokens[lo:lo + k + 1])
    return np.asarray(toks, dtype=np.int64)


def chi_square(tokens, p):
    counts = np.bincount(tokens, minlength=len(p)).astype(np.float64)
    expected = len(tokens) * np.asarray(p, dtype=np.float64)
    keep = expected > 0
    assert counts[~keep].sum() == 0, "token outside the support of p"
    return float(((counts[keep] - expected[keep]) ** 2 / expected[keep]).sum())


def chi2_threshold(dof, alpha):
    return float(stats.chi2.ppf(1.0 - alpha, dof))


def target_law(logits, T):
    """softmax(logits / T) in float64 via scipy (a library routine, not the oracle's code)."""
    from scipy.special import softmax
    return softmax(np.asarray(logits, dtype=np.float32).astype(np.float64) / T)
