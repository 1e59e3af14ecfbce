"""The early-exit phase planner (host code of the C ABI, no GPU): its plan
must be a least-cost cut of positions 0..K found by enumerating every cut,
under the expected-rows model the header states, and degenerate inputs must
give the one-pass plan."""
import itertools

import numpy as np
import pytest


@pytest.fixture(scope="module")
def sv():
    import rejection_sampling_verify_03_amd as m
    return m


def phases_of(mask, K):
    starts = [0] + [k for k in range(1, K + 1) if (mask >> k) & 1]
    ends = starts[1:] + [K + 1]
    return list(zip(starts, ends))


def expected_cost(mask, K, survival, f, cost):
    """Rows a request reads under this cut, in expectation: a phase [s, e) is
    read iff the request reaches s; it holds the target rows s..e-1 (row K
    only in the last phase) and f draft rows per position below K."""
    total = 0.0
    for s, e in phases_of(mask, K):
        total += survival[s] * ((e - s) + f * (min(e, K) - s))
    return total + cost * (len(phases_of(mask, K)) - 1)


def brute_best(K, survival, f, cost):
    best = None
    for bits in itertools.product([0, 1], repeat=K):
        mask = sum(1 << (k + 1) for k, v in enumerate(bits) if v)
        c = expected_cost(mask, K, survival, f, cost)
        if best is None or c < best - 1e-12:
            best = c
    return best


@pytest.mark.parametrize("K", [1, 2, 5, 8, 10])
def test_plan_is_optimal(sv, K):
    rng = np.random.default_rng(K)
    for trial in range(12):
        beta = rng.uniform(0.2, 0.98)
        if trial % 3 == 0:  # geometric acceptance
            surv = [beta ** k for k in range(K + 1)]
        else:  # any non-increasing survival curve starting at 1
            surv = [1.0] + sorted(rng.uniform(0, 1, K).tolist(), reverse=True)
        f = rng.uniform(0, 1)
        cost = rng.choice([0.0, 0.3, 1.0, 3.0])
        mask = sv.spec_verify_plan_phases(K, surv, f, cost)
        assert mask & 1 == 0 and mask >> (K + 1) == 0
        got = expected_cost(mask, K, surv, f, cost)
        assert got <= brute_best(K, surv, f, cost) + 1e-9, (K, surv, f, cost, bin(mask))


def test_plan_special_cases(sv):
    K = 8
    # every request accepts everything: nothing to skip, one pass
    assert sv.spec_verify_plan_phases(K, [1.0] * (K + 1), 1.0, 0.5) == 0
    # free phase boundaries: every position its own phase when survival drops at each step
    surv = [0.9 ** k for k in range(K + 1)]
    assert sv.spec_verify_plan_phases(K, surv, 1.0, 0.0) == sum(1 << k for k in range(1, K + 1))
    # boundaries dearer than all rows: one pass
    assert sv.spec_verify_plan_phases(K, surv, 1.0, 1e6) == 0
    # every request rejects position 0: a phase boundary right after it
    assert sv.spec_verify_plan_phases(K, [1.0] + [0.0] * K, 1.0, 0.5) == 1 << 1
    # out-of-range arguments give the one-pass plan
    for args in [(0, [1.0], 1.0, 0.1), (64, [1.0] * 65, 1.0, 0.1), (K, [1.0] * 8 + [1.5], 1.0, 0.1),
                 (K, surv, -0.1, 0.1), (K, surv, 1.0, -1.0), (K, surv, 1.0, float("nan")),
                 (K, surv, float("inf"), 0.1)]:
        assert sv.spec_verify_plan_phases(*args) == 0, args
    assert sv.lib.spec_verify_plan_phases(K, None, 1.0, 0.1) == 0


def test_survival_from_accepted(sv):
    s = sv.survival_from_accepted([0, 2, 2, 4, -1], 4)
    assert s == [1.0, 0.75, 0.75, 0.25, 0.25]
