"""The GPU-versus-oracle comparator itself, on the CPU: a result equal to
the oracle's is exact; a result that differs at a decision whose uniform is
far from its threshold fails; one that differs at a decision within the
window of its threshold is counted as near-threshold.  The "GPU" results here
are the oracle's own outputs, edited."""
import numpy as np

import oracle
import parity


def _case(seed=0, B=6, K=3, V=40):
    rng = np.random.default_rng(seed)
    tl = (1.5 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    dl = (tl + rng.standard_normal((B, K + 1, V))).astype(np.float32)
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    T = np.ones(B, np.float32)
    return tl, dl, x, T


def test_exact_and_far_mismatch():
    tl, dl, x, T = _case()
    r = oracle.verify(tl, dl, x, T, seed=2)
    rep = parity.compare(tl, dl, x, T, r.accepted, r.tokens, r.debug_probs, seed=2)
    assert rep.ok() and rep.exact == len(T)
    # a different token at the sampling row, far from every CDF boundary in between
    tok = r.tokens.copy()
    b = 0
    a = int(r.accepted[b])
    w, W = oracle.sampling_weights(tl, dl, x, T, b, a)
    F = np.cumsum(w) / W
    u = r.trace[b, a, 2]
    cand = [v for v in range(len(w)) if w[v] > 0 and v != tok[b, a]
            and np.min(np.abs(u - F[min(v, tok[b, a]):max(v, tok[b, a])])) > 1e-3]
    tok[b, a] = cand[0]
    rep = parity.compare(tl, dl, x, T, r.accepted, tok, None, seed=2)
    assert not rep.ok() and "sample@%d" % a in rep.failures[0]


def test_near_threshold_sampling_is_counted():
    """Uniforms overridden so that the sampling draw sits 1e-9 above a CDF
    boundary: the neighbouring token is accepted as near-threshold."""
    tl, dl, x, T = _case(3, B=1)
    r0 = oracle.verify(tl, dl, x, T, seed=1)
    a = int(r0.accepted[0])
    w, W = oracle.sampling_weights(tl, dl, x, T, 0, a)
    F = np.cumsum(w) / W
    v = next(i for i in range(1, len(w)) if w[i] > 0 and w[i - 1] > 0)  # positive weight on both sides
    # keep the accept decisions, move the sampling uniform next to F[v-1]
    u = np.zeros((1, x.shape[1] + 1, 2))
    u[0, :, 0] = r0.trace[0, :, 0]
    u[0, :, 1] = r0.trace[0, :, 2]
    u[0, a, 1] = F[v - 1] + 1e-9
    r = oracle.verify(tl, dl, x, T, uniforms=u)
    assert int(r.tokens[0, a]) == v
    # the comparator draws its uniforms from Philox, so its margin is checked through the overridden u
    margin = parity._sampling_margin(tl, dl, x, T, 0, a, u[0, a, 1], v - 1, v)
    assert margin < parity.WINDOW
    far = parity._sampling_margin(tl, dl, x, T, 0, a, u[0, a, 1] + 0.01, v - 1, v)
    assert far > parity.WINDOW
