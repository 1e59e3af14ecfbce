"""Pins of the oracle's ragged per-request draft counts K_b <= K.

Positions k >= K_b of request b do not exist (their tokens and rows are never
read); the request stops at its first rejection among positions 0..K_b-1 or
takes the bonus from row K_b (explainer page, section "核心思想", with the
draft length chosen per request).  Pinned against the same oracle run on the
request alone with K = K_b (the uniforms depend only on request, position and
step, so the two runs must agree token for token), by the K_b = 0 law (one
token from p_0), and by the data checks.
"""
import numpy as np

import oracle
import workloads
from stats_helpers import chi2_pvalue, softmax_rows


def _inputs(seed, B=10, K=6, V=300):
    inp = workloads.mixture_inputs("ragged", B, K, V, __import__("torch").float32, seed, "cpu",
                                   temps=(0.0, 0.7, 1.0), lam_lo=0.1, lam_hi=0.6)
    return (workloads.logits_numpy(inp.target), workloads.logits_numpy(inp.draft),
            inp.draft_tokens.numpy(), inp.temperature.numpy())


def test_full_counts_equal_no_table():
    tl, dl, x, T = _inputs(1)
    for step in range(3):
        a = oracle.verify(tl, dl, x, T, seed=4, step=step)
        b = oracle.verify(tl, dl, x, T, seed=4, step=step, num_drafts=np.full(len(T), x.shape[1]))
        for f in ("accepted", "tokens", "debug_probs"):
            np.testing.assert_array_equal(getattr(a, f), getattr(b, f))


def test_each_request_equals_its_own_shorter_run():
    tl, dl, x, T = _inputs(2)
    B, K = x.shape
    rng = np.random.default_rng(2)
    kb = rng.integers(1, K + 1, B)
    x2 = x.copy()
    for b in range(B):
        x2[b, kb[b]:] = -5  # tokens past K_b are never read
    for step in range(4):
        r = oracle.verify(tl, dl, x2, T, seed=8, step=step, num_drafts=kb)
        assert r.n_bad == 0
        for b in range(B):
            k = int(kb[b])
            s = oracle.verify(tl[b:b + 1, :k + 1], dl[b:b + 1, :k], x[b:b + 1, :k], T[b:b + 1], seed=8, step=step,
                              request_base=b)
            assert r.accepted[b] == s.accepted[0]
            np.testing.assert_array_equal(r.tokens[b, :k + 1], s.tokens[0])
            assert (r.tokens[b, k + 1:] == -1).all()
            np.testing.assert_array_equal(r.debug_probs[b, :k], s.debug_probs[0])
            assert (r.debug_probs[b, k:] == 0).all()


def test_no_drafts_samples_row_zero():
    """K_b = 0: no accept test, one token drawn from p_0 (chi-square over
    many requests sharing the rows)."""
    rng = np.random.default_rng(3)
    V, K, N = 32, 2, 60_000
    tl = (1.3 * rng.standard_normal((1, K + 1, V))).astype(np.float32)
    dl = tl + rng.standard_normal((1, K + 1, V)).astype(np.float32)
    x = np.zeros((N, K), np.int32)
    r = oracle.verify(tl, dl, x, np.ones(N, np.float32), seed=1, num_drafts=np.zeros(N, np.int32), debug=False)
    assert (r.accepted == 0).all() and (r.tokens[:, 1:] == -1).all()
    pv = chi2_pvalue(np.bincount(r.tokens[:, 0], minlength=V), softmax_rows(tl[0, 0]))
    assert pv >= 1e-4
    # greedy: the argmax of row 0
    r = oracle.verify(tl, dl, x[:3], np.zeros(3, np.float32), num_drafts=[0, 0, 0], debug=False)
    assert (r.tokens[:, 0] == np.argmax(tl[0, 0])).all()


def test_invalid_counts():
    tl, dl, x, T = _inputs(5, B=4)
    r = oracle.verify(tl, dl, x, T, num_drafts=[-1, 7, 3, 6])
    assert r.n_bad == 2 and (r.accepted[:2] == -1).all() and (r.tokens[:2] == -1).all()
    assert (r.accepted[2:] >= 0).all()
