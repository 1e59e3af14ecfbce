"""Exhaustive check of the oracle's decisions over every 24-bit uniform code.

V = 4, K = 2.  Each decision draws one uniform u = c * 2^-24, c in [0, 2^24).
For the accept test at a draft x the oracle must accept for exactly
ceil(t * 2^24) codes, t = min(1, p(x)/q(x)); its inverse CDF must return each
token y for r(y)/R * 2^24 codes, up to one code at each boundary.  Summing the
exact code counts over the draft token x ~ q then gives the law of the emitted
token, which must equal p at every row (the theorem of the explainer page,
section "修正拒绝采样") up to the 2^-24 quantisation of u.
"""
import math

import numpy as np
import pytest

import oracle
from stats_helpers import softmax_rows

CODES = (np.arange(2 ** 24, dtype=np.uint64) << np.uint64(8)).astype(np.uint32)
Q = 2.0 ** 24


def _case(seed):
    rng = np.random.default_rng(seed)
    tl = (1.5 * rng.standard_normal((3, 4))).astype(np.float32)
    dl = (tl + rng.standard_normal((3, 4))).astype(np.float32)
    return tl, dl


def _row_law(p, q):
    """Exact (code-counted) law of the token emitted at a row whose draft is
    x ~ q, given the row is reached."""
    V = len(p)
    w, W, fb = oracle.residual(p, q)
    assert not fb
    np.testing.assert_array_equal(w, np.maximum(p - q, 0.0))
    hits = np.bincount(oracle.invcdf_many(w, W, CODES), minlength=V).astype(np.float64)
    for y in range(V):
        assert abs(hits[y] - w[y] / W * Q) <= 1.0 + 1e-9, (y, hits[y], w[y] / W * Q)
    law = np.zeros(V)
    for x in range(V):
        n_acc = int(oracle.accept_many(p[x], q[x], CODES).sum())
        t = min(1.0, p[x] / q[x])
        assert abs(n_acc - math.ceil(t * Q)) <= 1, (x, n_acc, t * Q)
        pa = n_acc / Q
        law[x] += q[x] * pa
        law += q[x] * (1 - pa) * hits / Q
    return law


@pytest.mark.parametrize("seed", [0, 1])
def test_exhaustive_codes_reproduce_target_law(seed):
    tl, dl = _case(seed)
    p = softmax_rows(tl)
    q = softmax_rows(dl)
    # oracle softmax against the library softmax for these rows
    for k in range(3):
        np.testing.assert_allclose(oracle.softmax(tl[k], 1.0), p[k], rtol=1e-14, atol=0)
    for k in range(2):
        law = _row_law(p[k], q[k])
        assert np.max(np.abs(law - p[k])) <= 2.0 / Q, (k, law, p[k])
    # bonus row: inverse CDF straight over p
    hits = np.bincount(oracle.invcdf_many(p[2], p[2].sum(), CODES), minlength=4)
    assert np.max(np.abs(hits / Q - p[2])) <= 2.0 / Q


def test_verify_composes_the_primitives():
    """oracle.verify with explicit uniforms follows the decision primitives in
    order: accept tests at rows 0..K-1 until the first rejection, the residual
    draw at the rejecting row, the draw from p at row K otherwise."""
    tl, dl = _case(3)
    p = softmax_rows(tl)
    q = softmax_rows(dl)
    rng = np.random.default_rng(9)
    N = 4096
    x = rng.integers(0, 4, (N, 2)).astype(np.int32)
    u = (rng.integers(0, 2 ** 24, (N, 3, 2)) / Q).astype(np.float64)
    res = oracle.verify(tl[None], dl[None], x, np.ones(N, np.float32), uniforms=u)
    for i in range(N):
        want = []
        a = 2
        for k in range(2):
            if oracle.accept(p[k][x[i, k]], q[k][x[i, k]], u[i, k, 0]):
                want.append(int(x[i, k]))
                continue
            w = np.maximum(p[k] - q[k], 0.0)
            want.append(oracle.invcdf(w, w.sum(), u[i, k, 1]))
            a = k
            break
        else:
            want.append(oracle.invcdf(p[2], p[2].sum(), u[i, 2, 1]))
        assert res.accepted[i] == a
        assert list(res.tokens[i, :a + 1]) == want
        assert all(res.tokens[i, a + 1:] == -1)
