"""Special cases whose outcome the pages or textbook facts fix exactly."""
import numpy as np
import pytest

import oracle
import workloads
from stats_helpers import chi2_pvalue, draw_categorical, softmax_rows


def test_identical_distributions_accept_everything():
    """Explainer page, section "核心思想": two models with the same (uniform
    1..100) distribution defeat naive 'accept if equal' (1 in 100), while the
    modified rule accepts every draft when p == q."""
    B, K, V = 2000, 5, 100
    t = np.zeros((1, K + 1, V), np.float32)  # uniform over 100 tokens
    rng = np.random.default_rng(0)
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    r = oracle.verify(t, t, x, np.ones(B, np.float32), seed=1)
    assert (r.accepted == K).all()
    assert (r.tokens[:, :K] == x).all()
    # random identical rows at two temperatures
    tl = (2 * rng.standard_normal((1, K + 1, 300))).astype(np.float32)
    for T in (0.6, 1.0):
        x = draw_categorical(softmax_rows(tl[0, :K], T), B, rng)
        r = oracle.verify(tl, tl, x, np.full(B, T, np.float32), seed=2)
        assert (r.accepted == K).all()


def test_disjoint_supports_reject_at_once_and_resample_from_p():
    B, K, V = 200_000, 3, 20
    rng = np.random.default_rng(1)
    tl = np.full((1, K + 1, V), -np.inf, np.float32)
    dl = np.full((1, K + 1, V), -np.inf, np.float32)
    tl[0, :, :10] = rng.standard_normal((K + 1, 10))
    dl[0, :, 10:] = rng.standard_normal((K + 1, 10))
    x = draw_categorical(softmax_rows(dl[0, :K]), B, rng)
    r = oracle.verify(tl, dl, x, np.ones(B, np.float32), seed=3, debug=False, trace=False)
    assert (r.accepted == 0).all()
    assert (r.tokens[:, 0] < 10).all() and (r.tokens[:, 1:] == -1).all()
    counts = np.bincount(r.tokens[:, 0], minlength=V)
    assert chi2_pvalue(counts, softmax_rows(tl[0, 0])) >= 1e-4


def test_one_hot_target_is_deterministic():
    """p = delta_c: a draft equal to c is accepted (t = 1), any other is
    rejected and the residual max(0, delta_c - q) is concentrated on c."""
    B, K, V = 5000, 4, 50
    rng = np.random.default_rng(2)
    c = rng.integers(0, V, K + 1)
    tl = np.full((1, K + 1, V), -np.inf, np.float32)
    tl[0, np.arange(K + 1), c] = 0.0
    dl = rng.standard_normal((1, K + 1, V)).astype(np.float32)
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    x[: B // 2] = c[:K]  # half the requests draft exactly c
    r = oracle.verify(tl, dl, x, np.ones(B, np.float32), seed=4)
    match = x == c[:K]
    a_want = np.where(match.all(1), K, np.argmin(match, axis=1))
    np.testing.assert_array_equal(r.accepted, a_want)
    for i in range(B):
        a = a_want[i]
        assert list(r.tokens[i, :a + 1]) == list(c[:a + 1])


def test_greedy_ties_go_to_lowest_index():
    K, V = 2, 16
    t = np.zeros((1, K + 1, V), np.float32)
    t[0, 0, [3, 7]] = 5.0       # tie at row 0
    t[0, 1, [2, 9]] = 4.0       # tie at row 1
    t[0, 2, [11, 12]] = 1.0     # tie at the bonus row
    d = np.zeros_like(t)
    x = np.array([[7, 2], [3, 9], [3, 2]], np.int32)
    r = oracle.verify(t, d, x, np.zeros(3, np.float32))
    np.testing.assert_array_equal(r.accepted, [0, 1, 2])
    assert list(r.tokens[0]) == [3, -1, -1]
    assert list(r.tokens[1]) == [3, 2, -1]
    assert list(r.tokens[2]) == [3, 2, 11]
    # bf16 logits: equal bit patterns tie, the lowest index wins
    tb = workloads.bf16_bits(__import__("torch").tensor(t).bfloat16())
    r2 = oracle.verify(tb, workloads.bf16_bits(__import__("torch").tensor(d).bfloat16()), x,
                       np.zeros(3, np.float32))
    np.testing.assert_array_equal(r2.tokens, r.tokens)


def test_greedy_matches_argmax_definition():
    rng = np.random.default_rng(5)
    B, K, V = 64, 5, 333
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    g = np.argmax(t, axis=2)
    x = g[:, :K].copy()
    flip = rng.random((B, K)) < 0.3
    x[flip] = (x[flip] + 1) % V
    r = oracle.verify(t, t, x.astype(np.int32), np.zeros(B, np.float32))
    for b in range(B):
        bad = np.flatnonzero(flip[b])
        a = bad[0] if len(bad) else K
        assert r.accepted[b] == a
        assert list(r.tokens[b, :a]) == list(x[b, :a])
        assert r.tokens[b, a] == g[b, a]


def test_greedy_argmax_counts_nan_as_minus_inf():
    """The greedy token when a row holds NaN logits: numpy's first-occurrence
    argmax of the row with every NaN replaced by -inf, both dtypes."""
    nan, inf = np.nan, np.inf
    rows = [
        [nan, 1.0, 2.0, 2.0],     # NaN first: the finite maximum, its lowest index
        [nan, nan, nan, nan],     # every entry NaN: index 0
        [nan, -inf, nan, -inf],   # nothing above -inf: index 0
        [-inf, nan, -inf, -inf],  # ditto with -inf first
        [1.0, nan, 3.0, nan],     # NaN between finite values
        [nan, inf, nan, inf],     # +inf wins, lowest index
        [-5.0, nan, -5.0, nan],   # ties below NaNs
    ]
    t = np.array(rows, np.float32)
    want = np.argmax(np.where(np.isnan(t), -inf, t), axis=1)
    assert list(want) == [2, 0, 0, 0, 2, 1, 0]
    for b, row in enumerate(t):
        assert oracle.argmax(row) == want[b]
    # through verify: one greedy request per row, K = 0 (the bonus row only)
    # and K = 1 with a draft that differs from the argmax
    B, V = len(rows), 4
    tl = np.repeat(t[:, None, :], 2, axis=1)
    x = ((want + 1) % V).astype(np.int32)[:, None]
    for dt in ("f32", "bf16"):
        tt = tl if dt == "f32" else workloads.bf16_bits(__import__("torch").tensor(tl).bfloat16())
        r = oracle.verify(tt, tt, x, np.zeros(B, np.float32))
        assert (r.accepted == 0).all()
        np.testing.assert_array_equal(r.tokens[:, 0], want)
        r0 = oracle.verify(tt, tt, x, np.zeros(B, np.float32), num_drafts=np.zeros(B, np.int32))
        np.testing.assert_array_equal(r0.tokens[:, 0], want)
        # the draft sampler's greedy draw takes the same argmax
        rd = oracle.draft_sample(tt[:, 0], np.arange(B, dtype=np.int32)[:, None], np.zeros(B, np.float32))
        np.testing.assert_array_equal(rd.tokens[:, 0], want)


def test_single_token_vocabulary_and_single_draft():
    r = oracle.verify(np.zeros((3, 3, 1), np.float32), np.zeros((3, 3, 1), np.float32),
                      np.zeros((3, 2), np.int32), np.array([1.0, 0.0, 0.5], np.float32))
    assert (r.accepted == 2).all() and (r.tokens == 0).all()
    rng = np.random.default_rng(6)
    B = 100_000
    tl = rng.standard_normal((1, 2, 8)).astype(np.float32)
    dl = rng.standard_normal((1, 2, 8)).astype(np.float32)
    x = draw_categorical(softmax_rows(dl[0, :1]), B, rng)
    r = oracle.verify(tl, dl, x, np.ones(B, np.float32), debug=False, trace=False)
    assert set(np.unique(r.accepted)) <= {0, 1}
    assert chi2_pvalue(np.bincount(r.tokens[:, 0], minlength=8), softmax_rows(tl[0, 0])) >= 1e-4


def test_invalid_requests_are_flagged():
    rng = np.random.default_rng(7)
    B, K, V = 5, 3, 10
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    x = rng.integers(0, V, (B, K)).astype(np.int32)
    T = np.ones(B, np.float32)
    x[1, 2] = V          # token out of range
    x[2, 0] = -1         # negative token
    T[3] = -1.0          # negative temperature
    t[4, 0, :] = -np.inf  # a row every sampled request reads, with no finite maximum
    r = oracle.verify(t, t, x, T)
    assert r.n_bad == 4
    assert r.accepted[0] == K
    for b in range(1, 5):
        assert r.accepted[b] == -1 and (r.tokens[b] == -1).all() and (r.debug_probs[b] == 0).all()


def test_rows_after_the_stop_are_never_read():
    """The verification walks the positions in order and stops at the first
    rejection (explainer page, section "核心思想"), so a row past the stop
    has no say, while a row at the stop, or the bonus row, does.  Position 0
    rejects with certainty (the draft token lies outside the target's
    support), so the rows of positions 1..K may be anything; the residual is
    then p_0 itself.  When every draft is accepted (identical rows) the bonus
    row K_b is read."""
    rng = np.random.default_rng(11)
    B, K, V = 6, 3, 12
    t = np.full((B, K + 1, V), -np.inf, np.float32)
    d = np.full((B, K + 1, V), -np.inf, np.float32)
    t[:, 0, :6] = rng.standard_normal((B, 6))
    d[:, 0, 6:] = rng.standard_normal((B, 6))
    x = rng.integers(6, V, (B, K)).astype(np.int32)  # p_0(x_0) = 0: rejected
    T = np.full(B, 0.8, np.float32)
    t[1, 2, 3] = np.nan  # a NaN past the stop
    t[2, 0, :] = -np.inf  # no finite maximum at the stop: invalid
    d[3, 0, :] = -np.inf  # the draft row at the stop: invalid
    r = oracle.verify(t, d, x, T, seed=5)
    assert list(r.accepted) == [0, 0, -1, -1, 0, 0]
    for b in (0, 1, 4, 5):
        assert 0 <= r.tokens[b, 0] < 6 and (r.tokens[b, 1:] == -1).all()
        assert r.debug_probs[b, 0, 0] == 0.0 and r.debug_probs[b, 0, 1] > 0.0  # p_0(x_0) = 0 < q_0(x_0)
        assert (r.debug_probs[b, 1:] == 0).all()  # positions whose rows have no finite maximum
    assert (r.tokens[2] == -1).all() and (r.tokens[3] == -1).all()
    # identical rows accept everything; the bonus row K_b must be usable
    u = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    xs = rng.integers(0, V, (B, K)).astype(np.int32)
    nd = np.array([3, 3, 2, 2, 0, 0], np.int32)
    u[1, 3, :] = -np.inf  # request 1's bonus row (K_b = 3)
    u[3, 3, :] = -np.inf  # past request 3's bonus row (K_b = 2): never read
    u[5, 0, :] = -np.inf  # request 5's bonus row (K_b = 0)
    r = oracle.verify(u, u, xs, np.ones(B, np.float32), seed=6, num_drafts=nd)
    assert list(r.accepted) == [3, -1, 2, 2, 0, -1]


def test_request_base_reproduces_a_shard():
    """A subset of requests run with request_base = its first index gives
    exactly the rows of the full run (counter keyed on the request)."""
    inp = workloads.verify_tiny(seed=0)
    tl = workloads.logits_numpy(inp.target)
    dl = workloads.logits_numpy(inp.draft)
    x = inp.draft_tokens.numpy()
    T = inp.temperature.numpy()
    full = oracle.verify(tl, dl, x, T, seed=11, step=3)
    part = oracle.verify(tl[2:], dl[2:], x[2:], T[2:], seed=11, step=3, request_base=2)
    np.testing.assert_array_equal(full.tokens[2:], part.tokens)
    np.testing.assert_array_equal(full.accepted[2:], part.accepted)
    again = oracle.verify(tl, dl, x, T, seed=11, step=3)
    np.testing.assert_array_equal(full.tokens, again.tokens)
    other = oracle.verify(tl, dl, x, T, seed=11, step=4)
    assert (other.trace[:, 0, 0] != full.trace[:, 0, 0]).any()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_softmax_matches_library_and_debug_probs(dtype):
    import torch
    rng = np.random.default_rng(8)
    B, K, V = 6, 3, 257
    t32 = (3 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    d32 = (t32 + rng.standard_normal((B, K + 1, V))).astype(np.float32)
    t32[0, 0, :5] = -np.inf
    if dtype == "bf16":
        tt, dt = torch.tensor(t32).bfloat16(), torch.tensor(d32).bfloat16()
        tl, dl = workloads.bf16_bits(tt), workloads.bf16_bits(dt)
        tv, dv = tt.float().numpy(), dt.float().numpy()
    else:
        tl, dl, tv, dv = t32, d32, t32, d32
    T = np.array([1.0, 0.6, 1.3, 0.25, 2.0, 1.0], np.float32)
    x = rng.integers(5, V, (B, K)).astype(np.int32)
    r = oracle.verify(tl, dl, x, T)
    for b in range(B):
        for k in range(K):
            p = softmax_rows(tv[b, k], float(T[b]))
            q = softmax_rows(dv[b, k], float(T[b]))
            np.testing.assert_allclose(oracle.softmax(tl[b, k], float(T[b])), p, rtol=1e-13, atol=1e-300)
            assert r.debug_probs[b, k, 0] == np.float32(p[x[b, k]])
            assert r.debug_probs[b, k, 1] == np.float32(q[x[b, k]])


def _boundary_temperature(m, factor):
    """The temperature at which |m| * log2(e) / T = factor * 2^24, as fp32."""
    return np.float32(abs(m) * np.log2(np.e) / (factor * 2.0 ** 24))


def test_scaled_maximum_range_of_sampled_rows():
    """A sampled row counts only while its largest logit m has
    |m| * log2(e) / T within 2^24 (the fp32 reference of the kernels).
    Pinned on either side of the bound with a 0.1 % margin, where rounding
    cannot decide; a temperature between 0 and the smallest normal fp32 value
    is invalid; and far inside the bound, at a temperature tiny against the
    logit gaps, the draw is the argmax (the T -> 0 limit of softmax)."""
    rng = np.random.default_rng(17)
    V = 300
    for m in (10.0, -10.0, 2000.0):
        row = (m - 1.0 - rng.random(V)).astype(np.float32)
        row[123] = m
        t_in, t_out = _boundary_temperature(m, 0.999), _boundary_temperature(m, 1.001)
        assert oracle.scaled_max_in_range(row, t_in) and not oracle.scaled_max_in_range(row, t_out)
        assert oracle.scaled_max_in_range(row, 1.0)
        # through verify (K = 1; the target row is the row above, draft rows
        # equal, so the draft token 123 is accepted and the bonus row is read)
        tl = np.stack([row, row])[None].repeat(3, axis=0)
        x = np.full((3, 1), 123, np.int32)
        T = np.array([t_in, t_out, 1e-40], np.float32)
        r = oracle.verify(tl, tl, x, T, seed=1)
        assert r.accepted[0] == 1 and r.tokens[0].tolist() == [123, 123]
        assert r.accepted[1] == -1 and r.accepted[2] == -1 and (r.tokens[1:] == -1).all() and r.n_bad == 2
        # the draft sampler on the same row
        d = oracle.draft_sample(row[None], np.zeros((3, 1), np.int32), T, seed=2)
        assert d.tokens[:, 0].tolist() == [123, -1, -1]
    # a row with nothing finite stays out of range at any temperature
    assert not oracle.scaled_max_in_range(np.full(5, -np.inf, np.float32), 1.0)
    # bf16 rows: the bound on the bf16 value itself
    import torch
    rb = workloads.bf16_bits(torch.tensor([3.0, 96.0, -5.0]).bfloat16())
    assert oracle.scaled_max_in_range(rb, _boundary_temperature(96.0, 0.999))
    assert not oracle.scaled_max_in_range(rb, _boundary_temperature(96.0, 1.001))
