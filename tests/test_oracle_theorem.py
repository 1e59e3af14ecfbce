"""The oracle's output law, pinned to the distribution-preservation theorem.

Explainer page, section "修正拒绝采样": accepting x ~ q with probability
min(1, p(x)/q(x)) and otherwise resampling from normalize(max(0, p - q)) emits a
token distributed exactly as p, for any q.  With all rows fixed and shared by
every request, the token emitted at position k by the requests that reach k
(all earlier drafts accepted) must follow p_k, and the bonus token after K
acceptances must follow p_K.  The number of acceptances at k among the
requests reaching it is Binomial(n_k, sum_v min(p_k, q_k)).

Two planted mistakes (in the oracle, on the CPU) show the test has power:
mutation 1 resamples from p instead of the residual, mutation 2 accepts with
probability p(x) ignoring q.
"""
import numpy as np
import pytest

import oracle
from stats_helpers import binom_z, chi2_pvalue, draw_categorical, softmax_rows

N_REQ = 1_000_000
K = 3


def _rows(V, seed):
    rng = np.random.default_rng(seed)
    tl = (1.5 * rng.standard_normal((K + 1, V))).astype(np.float32)
    dl = (tl + rng.standard_normal((K + 1, V))).astype(np.float32)
    return tl, dl


def _run(V, seed, mutation=0, T=1.0):
    tl, dl = _rows(V, seed)
    p = softmax_rows(tl, T)
    q = softmax_rows(dl, T)
    rng = np.random.default_rng(seed + 1000)
    x = draw_categorical(q[:K], N_REQ, rng)
    r = oracle.verify(tl[None], dl[None], x, np.full(N_REQ, T, np.float32), seed=seed + 7,
                      debug=False, trace=False, mutation=mutation)
    assert r.n_bad == 0
    return p, q, x, r


def _pvalues(p, q, x, r, V):
    pv, zs = [], []
    a = r.accepted
    for k in range(K + 1):
        reach = a >= k
        tok = r.tokens[reach, k]
        counts = np.bincount(tok, minlength=V)
        pv.append(chi2_pvalue(counts, p[k]))
        if k < K:
            acc_k = int((a[reach] > k).sum())
            alpha = float(np.minimum(p[k], q[k]).sum())
            zs.append(binom_z(acc_k, int(reach.sum()), alpha))
    return pv, zs


@pytest.mark.parametrize("V", [16, 64])
def test_output_follows_target_distribution(V):
    p, q, x, r = _run(V, seed=V)
    pv, zs = _pvalues(p, q, x, r, V)
    assert min(pv) >= 1e-4, pv
    assert max(abs(z) for z in zs) < 5, zs
    # every position is exercised by a large number of requests
    assert (r.accepted == K).sum() > 1000


def test_output_follows_target_at_lower_temperature():
    V = 32
    p, q, x, r = _run(V, seed=5, T=0.6)
    pv, zs = _pvalues(p, q, x, r, V)
    assert min(pv) >= 1e-4, pv
    assert max(abs(z) for z in zs) < 5, zs


@pytest.mark.parametrize("mutation", [1, 2])
def test_planted_mistakes_are_detected(mutation):
    V = 64
    p, q, x, r = _run(V, seed=V, mutation=mutation)
    pv, zs = _pvalues(p, q, x, r, V)
    assert min(pv) < 1e-4 or max(abs(z) for z in zs) >= 5, (pv, zs)
