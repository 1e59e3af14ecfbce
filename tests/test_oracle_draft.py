"""Pins of the oracle's draft-token sampling at the new-token indices.

The draft token of position k of request b is drawn from
q = softmax(logits[row_index[b, k]] / T_b) (the drafter's distribution that
the next verification checks, explainer page, section "修正拒绝采样"; the rows
are the new-token indices of the expanded batch, "P-EAGLE" page, section
"Triton Kernel").  Pinned by the output law (chi-square against a library
softmax, with a planted mistake the test must catch), by the wiring of its
uniform to the published Philox generator (pinned by its known-answer
vectors elsewhere), and by the special cases.
"""
import numpy as np
import pytest

import oracle
from stats_helpers import chi2_pvalue, softmax_rows


def _rows(seed, N=3, V=64, scale=1.5):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((N, V))).astype(np.float32)


@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
def test_output_law(T):
    """200000 requests draw K = 3 positions from rows 0, 1, 2: each position's
    tokens follow softmax(row / T)."""
    lg = _rows(1)
    B = 200_000
    ri = np.tile(np.arange(3, dtype=np.int32), (B, 1))
    r = oracle.draft_sample(lg, ri, np.full(B, T, np.float32), seed=5, step=2)
    assert r.n_bad == 0
    for k in range(3):
        p = softmax_rows(lg[k], T)
        pv = chi2_pvalue(np.bincount(r.tokens[:, k], minlength=64), p)
        assert pv >= 1e-4, (T, k, pv)


def test_planted_mistake_is_caught():
    """Ignoring the temperature (mutation 1) must fail the same test."""
    lg = _rows(1)
    B = 200_000
    ri = np.tile(np.arange(3, dtype=np.int32), (B, 1))
    r = oracle.draft_sample(lg, ri, np.full(B, 0.6, np.float32), seed=5, step=2, mutation=1)
    pvs = [chi2_pvalue(np.bincount(r.tokens[:, k], minlength=64), softmax_rows(lg[k], 0.6)) for k in range(3)]
    assert min(pvs) < 1e-6


def test_uniform_stream():
    """The uniform of (request b + base, position k, step) is word 0 of
    Philox4x32-10 at counter {b + base, k, step, 1}: a stream apart from the
    verification's (counter word 3 = 0)."""
    lg = _rows(2, N=5, V=16)
    ri = np.array([[0, 4, 2], [1, 1, 3]], np.int32)
    seed, step, base = 0x1234_5678_9ABC_DEF0, 7, 40
    r = oracle.draft_sample(lg, ri, [1.0, 0.8], seed=seed, step=step, request_base=base)
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for b in range(2):
        for k in range(3):
            w = oracle.philox4x32_10([b + base, k, step, 1], key)
            assert r.trace[b, k] == oracle.uniform(w[0])
            assert r.trace[b, k] == oracle.draft_uniform(seed, step, b + base, k)
            v = oracle.philox4x32_10([b + base, k, step, 0], key)
            assert r.trace[b, k] not in (oracle.uniform(v[0]), oracle.uniform(v[1]))
            # and the token is the inverse CDF of that uniform over the row's softmax
            p = oracle.softmax(lg[ri[b, k]], [1.0, 0.8][b])
            assert r.tokens[b, k] == oracle.invcdf(p, p.sum(), r.trace[b, k])


def test_special_cases():
    lg = np.array([[0.5, 2.0, 2.0, -1.0],             # tied maximum
                   [-np.inf, -np.inf, 3.0, -np.inf],  # one finite logit
                   [1.0, 1.0, 1.0, 1.0],
                   [-np.inf] * 4], np.float32)       # no finite maximum
    # greedy: lowest index of the maximum
    r = oracle.draft_sample(lg, [[0, 1, 2]], [0.0])
    assert r.tokens.tolist() == [[1, 2, 0]] and r.n_bad == 0
    # a single finite logit is drawn with certainty at any temperature
    r = oracle.draft_sample(lg, np.ones((500, 1), np.int32), np.full(500, 0.3, np.float32), seed=1)
    assert (r.tokens == 2).all()
    # invalid rows and temperatures give -1, position by position / request by request
    r = oracle.draft_sample(lg, [[0, -1, 4], [3, 2, 2], [0, 1, 2], [0, 1, 2], [0, 1, 2]],
                            [1.0, 1.0, -1.0, np.nan, np.inf])
    assert r.tokens[0, 1] == -1 and r.tokens[0, 2] == -1 and r.tokens[0, 0] >= 0
    assert r.tokens[1, 0] == -1 and (r.tokens[1, 1:] >= 0).all()
    assert (r.tokens[2:] == -1).all()
    assert r.n_bad == 3 + 9
    # V = 1
    r = oracle.draft_sample(np.zeros((2, 1), np.float32), [[0, 1]], [0.7])
    assert r.tokens.tolist() == [[0, 0]]
    # bf16 bit patterns give the same draws as the same values in fp32
    vals = _rows(3, N=4, V=32).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    exact = (bits.astype(np.uint32) << 16).view(np.float32)
    ri = np.array([[0, 1, 2, 3], [3, 2, 1, 0]], np.int32)
    a = oracle.draft_sample(bits, ri, [1.0, 0.5], seed=9)
    b = oracle.draft_sample(exact, ri, [1.0, 0.5], seed=9)
    np.testing.assert_array_equal(a.tokens, b.tokens)


def test_greedy_limit():
    """A temperature near 0 concentrates the draw on the argmax."""
    lg = _rows(4, N=2, V=50)
    B = 2000
    ri = np.tile(np.array([0, 1], np.int32), (B, 1))
    r = oracle.draft_sample(lg, ri, np.full(B, 1e-3, np.float32), seed=3)
    assert (r.tokens[:, 0] == np.argmax(lg[0])).all() and (r.tokens[:, 1] == np.argmax(lg[1])).all()
