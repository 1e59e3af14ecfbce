"""The oracle's accept-count law, pinned to the expected-tokens closed form.

Explainer page, section "一轮能赚多少：接受率的算术": with per-token acceptance
beta and draft length gamma a round produces (1 - beta^(gamma+1)) / (1 - beta)
tokens on average; the page prints three values of it.  Reading: the count
includes the resampled or bonus token (a + 1 for a accepted drafts), which is
what makes the printed acceptance lengths above K possible.

With identical p and q at every position the acceptance at each position is an
independent Bernoulli(alpha), alpha = sum_v min(p, q), so the number of
accepted drafts a is a geometric law truncated at K:
P(a = j) = alpha^j (1 - alpha) for j < K and P(a = K) = alpha^K.
"""
import json
import os

import numpy as np
import pytest

import oracle
from stats_helpers import chi2_pvalue, draw_categorical, expected_tokens_per_round, softmax_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_closed_form_reproduces_printed_table():
    with open(os.path.join(GOLDEN, "expected_tokens_table.json")) as f:
        tab = json.load(f)
    for row in tab["rows"]:
        v = expected_tokens_per_round(row["beta"], row["gamma"])
        assert round(v, 2) == row["printed"], (row, v)


def _mixture_rows(V, alpha_target, seed):
    """fp32 logits of p and of q = (1 - lam) p + lam r with lam chosen so that
    sum min(p, q) = 1 - lam * TV(p, r) hits alpha_target."""
    rng = np.random.default_rng(seed)
    pl = (1.5 * rng.standard_normal(V)).astype(np.float32)
    p = softmax_rows(pl)
    r = softmax_rows(rng.standard_normal(V))
    tv = 0.5 * np.abs(p - r).sum()
    lam = (1.0 - alpha_target) / tv
    assert 0 < lam < 1
    q = (1 - lam) * p + lam * r
    ql = np.log(q).astype(np.float32)
    return pl, ql


@pytest.mark.parametrize("alpha_target,K", [(0.5, 4), (0.8, 4), (0.9, 8), (0.8, 8)])
def test_accept_count_law(alpha_target, K):
    V, N = 64, 1_000_000
    pl, ql = _mixture_rows(V, alpha_target, seed=int(alpha_target * 100) + K)
    # alpha of the rows actually stored (fp32 logits), by the library softmax
    p = softmax_rows(pl)
    q = softmax_rows(ql)
    alpha = float(np.minimum(p, q).sum())
    tl = np.repeat(pl[None, None, :], K + 1, axis=1)
    dl = np.repeat(ql[None, None, :], K + 1, axis=1)
    x = draw_categorical(np.repeat(q[None], K, axis=0), N, np.random.default_rng(K))
    res = oracle.verify(tl, dl, x, np.ones(N, np.float32), seed=K * 31 + 1, debug=False, trace=False)
    a = res.accepted
    law = np.array([alpha ** j * (1 - alpha) for j in range(K)] + [alpha ** K])
    counts = np.bincount(a, minlength=K + 1)
    assert chi2_pvalue(counts, law) >= 1e-4
    mean_tokens = float((a + 1).mean())
    want = expected_tokens_per_round(alpha, K)
    var = float((law * (np.arange(K + 1) + 1.0) ** 2).sum() - want ** 2)
    z = (mean_tokens - want) / np.sqrt(var / N)
    assert abs(z) < 4, (mean_tokens, want, z)
