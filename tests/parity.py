"""GPU-versus-oracle comparison for the verification outputs.

Bar (per request, same inputs, same seed / step / request index):
  * accepted counts and emitted tokens bit-exact, EXCEPT when the first
    decision on which the two sides differ is near its threshold: an accept
    test whose uniform u lies within WINDOW of the oracle's threshold
    min(1, p(x)/q(x)), or a sampling draw whose u' lies within WINDOW of the
    oracle's normalised CDF at some boundary between the two emitted tokens.
    Such requests are counted, not failed; everything after that decision may
    legitimately differ.  Greedy (T = 0) and invalid requests have no tolerance.
  * debug probabilities p_k(x_k), q_k(x_k) within PROB_TOL max-abs (fp32).
"""
import numpy as np

import oracle

WINDOW = 1e-6
PROB_TOL = 1e-6


class Report:
    def __init__(self):
        self.requests = 0
        self.exact = 0
        self.near = []       # (b, kind, margin)
        self.failures = []   # human-readable
        self.max_prob_err = 0.0

    def ok(self):
        return not self.failures

    def summary(self):
        return ("%d requests: %d bit-exact, %d near-threshold, %d failures, max |dp| %.3g"
                % (self.requests, self.exact, len(self.near), len(self.failures), self.max_prob_err))


def _sampling_margin(tl, dl, x, T, b_local, j, u, y_g, y_o, num_drafts=None):
    w, W = oracle.sampling_weights(tl, dl, x, T, b_local, j, num_drafts=num_drafts)
    F = np.cumsum(w) / W
    lo, hi = min(y_g, y_o), max(y_g, y_o)
    if lo < 0:
        return np.inf
    return float(np.min(np.abs(u - F[lo:hi]))) if hi > lo else np.inf


def compare(tl, dl, x, T, acc_g, tok_g, dbg_g=None, seed=0, step=0, request_base=0, report=None,
            check_debug=True, num_drafts=None):
    """Compare GPU outputs for a batch with the oracle run on the same host
    inputs (tl, dl: oracle-format logits [B, K+1, V]; x [B, K]; T [B]).
    request_base is the global index of row 0 of this batch."""
    rep = report if report is not None else Report()
    res = oracle.verify(tl, dl, x, T, seed=seed, step=step, request_base=request_base,
                        debug=dbg_g is not None and check_debug, trace=True, num_drafts=num_drafts)
    B, K1 = res.tokens.shape
    K = K1 - 1
    acc_g = np.asarray(acc_g)
    tok_g = np.asarray(tok_g)
    for b in range(B):
        rep.requests += 1
        ao, ag = int(res.accepted[b]), int(acc_g[b])
        to, tg = res.tokens[b], tok_g[b]
        if ao == ag and np.array_equal(to, tg):
            rep.exact += 1
            continue
        gb = request_base + b
        if ao < 0 or ag < 0 or float(T[b]) == 0.0:
            rep.failures.append("request %d (T=%g): gpu a=%d %s vs oracle a=%d %s"
                                % (gb, T[b], ag, list(tg), ao, list(to)))
            continue
        if ao != ag:
            k = min(ao, ag)
            u, thr = res.trace[b, k, 0], res.trace[b, k, 1]
            margin = abs(u - thr)
            kind = "accept@%d" % k
        else:
            k = ao
            u = res.trace[b, k, 2]
            margin = _sampling_margin(tl[b:b + 1] if tl.shape[0] > 1 else tl,
                                      dl[b:b + 1] if dl.shape[0] > 1 else dl,
                                      x[b:b + 1], T[b:b + 1], 0, k, u, int(tg[k]), int(to[k]),
                                      None if num_drafts is None else np.asarray(num_drafts)[b:b + 1])
            kind = "sample@%d" % k
        if margin < WINDOW:
            rep.near.append((gb, kind, margin))
        else:
            rep.failures.append("request %d (T=%g) %s margin %.3g: gpu a=%d %s vs oracle a=%d %s"
                                % (gb, T[b], kind, margin, ag, list(tg), ao, list(to)))
    if dbg_g is not None and check_debug:
        d = np.abs(np.asarray(dbg_g, np.float64) - res.debug_probs.astype(np.float64))
        rep.max_prob_err = max(rep.max_prob_err, float(d.max()) if d.size else 0.0)
        if d.size and d.max() > PROB_TOL:
            rep.failures.append("debug probabilities differ by %.3g" % d.max())
    return rep
