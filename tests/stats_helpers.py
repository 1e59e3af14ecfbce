"""Statistics helpers for the distribution tests (no verification arithmetic)."""
import numpy as np
from scipy import stats
from scipy.special import softmax as scipy_softmax


def softmax_rows(logits, T=1.0):
    """Library softmax (scipy) in float64 of float32 logits, row-wise."""
    return scipy_softmax(np.asarray(logits, np.float64) / T, axis=-1)


def chi2_pvalue(counts, probs, min_expected=5.0):
    """Pearson chi-square goodness of fit of integer ``counts`` against
    ``probs``; bins with expectation below ``min_expected`` are merged (in
    ascending expectation) until every merged bin reaches it."""
    counts = np.asarray(counts, np.float64)
    probs = np.asarray(probs, np.float64)
    n = counts.sum()
    exp = probs * n
    order = np.argsort(exp)
    obs_m, exp_m = [], []
    acc_o = acc_e = 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += exp[i]
        if acc_e >= min_expected:
            obs_m.append(acc_o)
            exp_m.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0 or acc_o > 0:
        if exp_m:
            obs_m[-1] += acc_o
            exp_m[-1] += acc_e
        else:
            obs_m.append(acc_o)
            exp_m.append(acc_e)
    obs_m = np.array(obs_m)
    exp_m = np.array(exp_m)
    if len(obs_m) < 2:
        return 1.0
    chi2 = float(((obs_m - exp_m) ** 2 / exp_m).sum())
    return float(stats.chi2.sf(chi2, len(obs_m) - 1))


def binom_z(successes, trials, p):
    if trials == 0:
        return 0.0
    sd = np.sqrt(trials * p * (1 - p))
    if sd == 0:
        return 0.0 if successes == trials * p else np.inf
    return float((successes - trials * p) / sd)


def expected_tokens_per_round(beta, gamma):
    """Closed form (1 - beta^(gamma+1)) / (1 - beta) of the explainer page,
    section on the arithmetic of the acceptance rate."""
    if beta == 1.0:
        return gamma + 1.0
    return (1.0 - beta ** (gamma + 1)) / (1.0 - beta)


def draw_categorical(probs_rows, n, rng):
    """n independent draws from each row of probs_rows -> [n, rows] int32, by
    inverse CDF on numpy uniforms."""
    probs_rows = np.atleast_2d(np.asarray(probs_rows, np.float64))
    out = np.empty((n, probs_rows.shape[0]), np.int32)
    for r, p in enumerate(probs_rows):
        c = np.cumsum(p)
        c /= c[-1]
        u = rng.random(n)
        out[:, r] = np.minimum(np.searchsorted(c, u, side="right"), len(p) - 1)
    return out
