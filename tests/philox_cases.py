"""Inputs whose verification and draft-sampling outputs are closed forms of
the Philox uniforms, shared by the device-versus-oracle stream test (GPU) and
its CPU check against the oracle's own outputs.

* Draft sampling over V equal logits: the inverse CDF of equal weights is
  floor(u * V).
* Verification with shared all-zero target rows (p uniform) and a draft row
  table: positions before j = K_b - 1 read draft row 0 (equal to the target:
  p(x)/q(x) = 1, accepted whatever u), position j reads a row uniform over
  its first m tokens (p(x)/q(x) = m / V for x inside); a request accepts all
  K_b drafts iff u_j < m / V and then emits the bonus floor(u'_{K_b} V), else
  it emits the residual's token m + floor(u'_j (V - m)) (the residual is
  uniform over the tokens the draft row leaves out); K_b = 0 emits
  floor(u'_0 V).
"""
import numpy as np

import oracle

M32 = 0xFFFFFFFF


def draft_expected(seed, step, request_base, B, K, V):
    b, k = np.meshgrid(np.arange(B, dtype=np.int64), np.arange(K, dtype=np.int64), indexing="ij")
    u = oracle.draft_uniforms(seed, step, (b + request_base) & M32, k)
    return np.floor(u * V).astype(np.int64)


class VerifyCase:
    """Host arrays of one verification case: target [1, K+1, V] zeros, draft
    row table rows [nrows, V], tokens x [B, K], row index [B, K], draft counts
    kb [B]; m[r] = tokens in the support of draft row r (row 0: all V)."""

    def __init__(self, rng, B, K, V, nrows=48):
        self.B, self.K, self.V = B, K, V
        self.target = np.zeros((1, K + 1, V), np.float32)
        self.m = np.concatenate([[V], rng.integers(1, V, nrows - 1)])
        self.drows = np.zeros((nrows, V), np.float32)
        for r in range(1, nrows):
            self.drows[r, self.m[r]:] = -np.inf
        kb = rng.integers(0, K + 1, B).astype(np.int32)
        kb[:min(B, 4)] = [0, 1, K, K - 1][:min(B, 4)]
        self.kb = kb
        self.rsel = rng.integers(1, nrows, B)
        x = rng.integers(0, V, (B, K)).astype(np.int32)
        ridx = np.zeros((B, K), np.int32)
        j = np.arange(B), np.maximum(kb - 1, 0)
        ridx[j] = np.where(kb > 0, self.rsel, 0)
        x[j] = np.where(kb > 0, rng.integers(0, V, B) % self.m[self.rsel], x[j])
        self.x, self.ridx = x, ridx

    def expected(self, seed, step, request_base):
        """(accepted counts [B], emitted token [B]) from the oracle's uniforms."""
        B, V, kb = self.B, self.V, self.kb
        g = (np.arange(B, dtype=np.int64) + request_base) & M32
        jj = np.maximum(kb - 1, 0)
        ua, us_j = oracle.verify_uniforms(seed, step, g, jj)   # accept test and residual draw at j
        _, us_k = oracle.verify_uniforms(seed, step, g, kb)     # bonus draw at K_b
        mb = self.m[self.rsel].astype(np.float64)
        thr = (1.0 / V) / (1.0 / mb)                            # p_j(x) / q_j(x), as both sides divide
        accept = (kb > 0) & (ua < thr)
        bonus = (kb == 0) | accept
        want_a = np.where(bonus, kb, kb - 1)
        want_y = np.where(bonus, np.floor(us_k * V), mb + np.floor(us_j * (V - mb))).astype(np.int64)
        return want_a, want_y, accept
