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


def test_phase_cost_by_batch_shape(sv):
    """The boundary price follows the batch shape: 12 us plus up to 7.7 us
    when one row of every request is less than one dispatch round of the
    row pass (1280 workgroups), in units of one row of every request at
    6.8 TB/s; invalid shapes price at -1 (the one-pass plan)."""
    def us(B, V, es=2):
        return sv.spec_verify_phase_cost(B, 8, V, sv.SPEC_BF16 if es == 2 else sv.SPEC_F32) * B * V * es / 6.8e6
    assert abs(us(256, 151936) - 12.0) < 1e-9      # 256 x 5 chunks = 1280 workgroups: a full round
    assert abs(us(1024, 201088) - 12.0) < 1e-9
    assert abs(us(64, 201088) - (12.0 + 7.7 * (1 - 64 * 7 / 1280))) < 1e-9
    assert abs(us(1, 1000, 4) - (12.0 + 7.7 * (1 - 1 / 1280))) < 1e-9
    assert us(128, 151936) > us(256, 151936)
    for args in [(0, 8, 1000, 1), (4, 0, 1000, 1), (4, 64, 1000, 1), (4, 8, 0, 1), (4, 8, 1000, 7)]:
        assert sv.spec_verify_phase_cost(*args) == -1.0, args
    assert sv.spec_verify_plan_phases(8, [0.9 ** k for k in range(9)], 1.0,
                                      sv.spec_verify_phase_cost(0, 8, 1000, 1)) == 0


def test_planned_cut_flips_across_shapes(sv):
    """With the acceptance curves the three workloads show, the shape-priced
    planner reads one pass at B=64 (V=201088, K=5: short kernels, a boundary
    costs more than the rows it saves), one boundary at the headline batch
    (B=256, V=151936, K=8, 178 of 256 requests sampled) and many at B=1024
    (V=201088, K=8, acceptance 0.8, where a boundary costs a fifth of a
    row-unit)."""
    c2 = [1.0, 0.708, 0.505, 0.375, 0.266, 0.188]
    head = [1.0, 0.8145, 0.7026, 0.6206, 0.5498, 0.501, 0.4668, 0.4395, 0.3989]
    c5 = [0.8 ** k for k in range(9)]
    assert sv.plan_phases(64, 5, 201088, c2, 1.0) == 0
    m = sv.plan_phases(256, 8, 151936, head, 178 / 256)
    assert m != 0 and bin(m).count("1") == 1, bin(m)
    m = sv.plan_phases(1024, 8, 201088, c5, 1.0)
    assert bin(m).count("1") >= 4, bin(m)
    # the constant 12 us price of before would have cut the B=64 batch
    row_us = 64 * 201088 * 2 / 6.8e3 / 1e3
    assert sv.spec_verify_plan_phases(5, c2, 1.0, 12.0 / row_us) != 0
