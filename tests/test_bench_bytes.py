"""The byte counts the benchmark divides by, checked against a row-by-row
enumeration of what each request reads (CPU only)."""
import numpy as np
import pytest

import bench


def rows_read(a, sampled, K, starts):
    """Rows (kind, position) a request stopping at `a` reads when the row pass
    runs in phases beginning at `starts`: every row of each phase that begins
    at or before its stop, the draft rows only when it samples."""
    rows = set()
    bounds = list(starts) + [K + 1]
    for s, e in zip(bounds[:-1], bounds[1:]):
        if s > a:
            break
        for k in range(s, e):
            rows.add(("t", k))
            if sampled and k < K:
                rows.add(("d", k))
    return rows


@pytest.mark.parametrize("K", [1, 3, 8])
def test_phased_and_sequential_bytes(K):
    rng = np.random.default_rng(K)
    B, V, es = 40, 1000, 2
    acc = rng.integers(0, K + 1, B)
    temps = rng.choice([0.0, 0.6, 1.0], B)
    for trial in range(20):
        mask = 0 if trial == 0 else int(rng.integers(0, 1 << (K + 1))) & ~1
        starts = [0] + [k for k in range(1, K + 1) if (mask >> k) & 1]
        want = sum(len(rows_read(int(a), t > 0, K, starts)) for a, t in zip(acc, temps)) * V * es
        assert bench.phased_logit_bytes(acc, temps, mask, K, V, es) == want, (K, mask)
    # one pass reads every target row and the sampled requests' draft rows
    assert bench.phased_logit_bytes(acc, temps, 0, K, V, es) == bench.one_pass_logit_bytes(B, K, V, es, temps)
    # the method's minimum: target rows 0..a, draft rows 0..min(a, K - 1) of sampled requests
    want = sum((a + 1) + (min(a + 1, K) if t > 0 else 0) for a, t in zip(acc, temps)) * V * es
    assert bench.sequential_logit_bytes(acc, temps, K, V, es) == want
    # a phase per position reads exactly the minimum
    every = sum(1 << k for k in range(1, K + 1))
    assert bench.phased_logit_bytes(acc, temps, every, K, V, es) == want


def test_algorithmic_bytes_of_the_headline_shape():
    """B = 256, K = 8, V = 151936 bf16 with 178 sampled requests: 9 target
    rows per request and 8 draft rows per sampled one, 303,872 bytes a row."""
    temps = np.array([1.0] * 178 + [0.0] * 78)
    logits = (256 * 9 + 178 * 8) * 151936 * 2
    assert logits == 1132834816  # the one-pass row kernel's algorithmic bytes in the benchmark line
    assert bench.one_pass_logit_bytes(256, 8, 151936, 2, temps) == logits
    io = 256 * 8 * 4 + 256 * 4 * 2 + 256 * 9 * 4
    assert bench.algorithmic_verify_bytes(256, 8, 151936, 2, temps) == logits + io
