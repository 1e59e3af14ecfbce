"""GPU verification through the C ABI against the CPU oracle.

Element-by-element parity at sizes the oracle finishes in seconds (several
chunks per row, ragged tails, vector and scalar load paths, shared and padded
rows, every special case), then the full-size workloads in the launch
configuration the benchmark times, checked on sampled requests the oracle
computes one by one.  The bar is the one in ``parity.py``.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from parity import Report, compare
from stats_helpers import binom_z, chi2_pvalue, draw_categorical, softmax_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rejection_sampling_verify_03_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(inp):
    return (workloads.logits_numpy(inp.target), workloads.logits_numpy(inp.draft),
            inp.draft_tokens.cpu().numpy(), inp.temperature.cpu().numpy())


def run(sv, target, draft, x, T, seed=0, step=0, request_base=0, debug=True, ws=None):
    acc, tok, dbg = sv.verify(target, draft, x, T, seed=seed, step=step, request_base=request_base,
                              debug=debug, workspace=ws)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), tok.cpu().numpy(), None if dbg is None else dbg.cpu().numpy()


def to_dev(inp):
    inp.target = inp.target.cuda()
    inp.draft = inp.draft.cuda()
    inp.draft_tokens = inp.draft_tokens.cuda()
    inp.temperature = inp.temperature.cuda()
    return inp


def check(sv, inp, seeds=(0,), steps=(0,), debug=True):
    tl, dl, x, T = host(inp)
    rep = Report()
    for seed in seeds:
        for step in steps:
            acc, tok, dbg = run(sv, inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed, step,
                                debug=debug)
            compare(tl, dl, x, T, acc, tok, dbg, seed=seed, step=step, report=rep)
    say(inp.name, rep.summary())
    assert rep.ok(), rep.failures[:5]
    return rep


def test_tiny_fp32_many_steps(sv):
    say("case: tiny B4 K4 V1024 fp32, 64 steps")
    inp = to_dev(workloads.verify_tiny(seed=0))
    rep = check(sv, inp, seeds=(0, 1), steps=range(32))
    assert rep.exact >= rep.requests - 2


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 70001), (torch.float32, 33000),
                                     (torch.bfloat16, 2 * 32768 + 512),
                                     (torch.bfloat16, 64 * 4096 + 40007)])  # > 64 segments: the block scan path
def test_multi_chunk_mixed_temperatures(sv, dtype, V):
    say("case: B12 K5 V%d %s mixed T" % (V, dtype))
    inp = workloads.mixture_inputs("mixed B12 K5 V%d" % V, 12, 5, V, dtype, 3, "cuda",
                                   temps=(0.0, 0.6, 1.0), lam_lo=0.05, lam_hi=0.6)
    check(sv, inp, seeds=(0, 5), steps=(0, 1))


@pytest.mark.parametrize("dtype,V", [(torch.float32, 1023), (torch.bfloat16, 20003), (torch.bfloat16, 9)])
def test_scalar_load_path(sv, dtype, V):
    """Rows whose byte length is not a multiple of 16 take the scalar path."""
    say("case: scalar path V%d %s" % (V, dtype))
    inp = workloads.noisy_draft_inputs("scalar V%d" % V, 6, 4, V, dtype, 1, "cuda", "gauss",
                                       target_std=2.0, draft_noise=0.5)
    check(sv, inp, seeds=(0,), steps=range(4))


def test_padded_rows_and_views(sv):
    """Logits inside larger buffers: row stride > V (padded), and only the
    first K draft rows present."""
    say("case: padded rows")
    B, K, V = 8, 4, 5000
    base = workloads.mixture_inputs("pad", B, K, V, torch.bfloat16, 4, "cuda", temps=(0.6, 1.0),
                                    lam_lo=0.1, lam_hi=0.5)
    tpad = torch.full((B, K + 1, V + 64), -30.0, dtype=torch.bfloat16, device="cuda")
    tpad[:, :, :V] = base.target
    dpad = torch.full((B, K, V + 128), -30.0, dtype=torch.bfloat16, device="cuda")
    dpad[:, :, :V] = base.draft[:, :K]
    tl, dl, x, T = host(base)
    acc, tok, dbg = run(sv, tpad[:, :, :V], dpad[:, :, :V], base.draft_tokens, base.temperature, 9, 2)
    rep = compare(tl, dl, x, T, acc, tok, dbg, seed=9, step=2)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]


def test_shared_rows_broadcast(sv):
    """Request stride 0: every request reads the same rows."""
    say("case: shared rows")
    K, V, B = 3, 700, 512
    rng = np.random.default_rng(0)
    tl = (1.5 * rng.standard_normal((1, K + 1, V))).astype(np.float32)
    dl = (tl + rng.standard_normal((1, K + 1, V))).astype(np.float32)
    x = draw_categorical(softmax_rows(dl[0, :K]), B, rng)
    T = np.ones(B, np.float32)
    t = torch.from_numpy(tl).cuda().expand(B, K + 1, V)
    d = torch.from_numpy(dl).cuda().expand(B, K + 1, V)
    acc, tok, dbg = run(sv, t, d, torch.from_numpy(x).cuda(), torch.from_numpy(T).cuda(), 3)
    rep = compare(tl, dl, x, T, acc, tok, dbg, seed=3)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]


def test_special_cases(sv):
    say("case: special cases")
    rng = np.random.default_rng(1)
    # identical distributions => everything accepted
    B, K, V = 64, 5, 100
    t = torch.zeros(B, K + 1, V, device="cuda")
    x = torch.from_numpy(rng.integers(0, V, (B, K)).astype(np.int32)).cuda()
    acc, tok, _ = run(sv, t, t, x, torch.ones(B, device="cuda"))
    assert (acc == K).all() and (tok[:, :K] == x.cpu().numpy()).all()
    tl = (2 * rng.standard_normal((B, K + 1, 3000))).astype(np.float32)
    tt = torch.from_numpy(tl).cuda().bfloat16()
    acc, _, _ = run(sv, tt, tt, torch.from_numpy(rng.integers(0, 3000, (B, K)).astype(np.int32)).cuda(),
                    torch.full((B,), 0.6, device="cuda"))
    assert (acc == K).all()
    # disjoint supports => reject at once, resample inside p's support
    tl = np.full((B, K + 1, 40), -np.inf, np.float32)
    dl = np.full((B, K + 1, 40), -np.inf, np.float32)
    tl[:, :, :20] = rng.standard_normal((B, K + 1, 20))
    dl[:, :, 20:] = rng.standard_normal((B, K + 1, 20))
    x = rng.integers(20, 40, (B, K)).astype(np.int32)
    T = np.ones(B, np.float32)
    acc, tok, dbg = run(sv, torch.from_numpy(tl).cuda(), torch.from_numpy(dl).cuda(),
                        torch.from_numpy(x).cuda(), torch.from_numpy(T).cuda(), 5)
    assert (acc == 0).all() and (tok[:, 0] < 20).all()
    rep = compare(tl, dl, x, T, acc, tok, dbg, seed=5)
    assert rep.ok(), rep.failures[:5]
    # one-hot targets => deterministic output
    c = rng.integers(0, 50, (B, K + 1))
    tl = np.full((B, K + 1, 50), -np.inf, np.float32)
    for b in range(B):
        tl[b, np.arange(K + 1), c[b]] = 0.0
    dl = rng.standard_normal((B, K + 1, 50)).astype(np.float32)
    x = rng.integers(0, 50, (B, K)).astype(np.int32)
    x[: B // 2] = c[: B // 2, :K]
    acc, tok, dbg = run(sv, torch.from_numpy(tl).cuda(), torch.from_numpy(dl).cuda(),
                        torch.from_numpy(x).cuda(), torch.ones(B, device="cuda"), 6)
    for b in range(B):
        assert list(tok[b, :acc[b] + 1]) == list(c[b, :acc[b] + 1])
    # greedy with ties: lowest index
    t = torch.zeros(3, 3, 16, device="cuda")
    t[:, 0, 3] = t[:, 0, 7] = 5.0
    t[:, 1, 2] = t[:, 1, 9] = 4.0
    t[:, 2, 11] = t[:, 2, 12] = 1.0
    x = torch.tensor([[7, 2], [3, 9], [3, 2]], dtype=torch.int32, device="cuda")
    acc, tok, dbg = run(sv, t, t, x, torch.zeros(3, device="cuda"))
    assert list(acc) == [0, 1, 2]
    assert tok.tolist() == [[3, -1, -1], [3, 2, -1], [3, 2, 11]]
    assert (dbg == 0).all()
    # bf16 greedy ties across chunk boundaries (V spans 3 chunks)
    V = 3 * 32768
    t = torch.zeros(2, 2, V, device="cuda", dtype=torch.bfloat16)
    t[:, 0, [40000, 70000, 90000]] = 3.0
    t[:, 1, [5, 98000]] = 2.0
    acc, tok, _ = run(sv, t, t, torch.tensor([[40000], [70000]], dtype=torch.int32, device="cuda"),
                      torch.zeros(2, device="cuda"))
    assert list(acc) == [1, 0] and tok.tolist() == [[40000, 5], [40000, -1]]
    # all -inf greedy row => index 0, as the oracle's argmax
    t = torch.full((1, 2, 300), -float("inf"), device="cuda")
    acc, tok, _ = run(sv, t, t, torch.tensor([[0]], dtype=torch.int32, device="cuda"),
                      torch.zeros(1, device="cuda"))
    assert acc[0] == 1 and tok[0].tolist() == [0, 0]
    # V = 1 and K = 1
    acc, tok, _ = run(sv, torch.zeros(3, 3, 1, device="cuda"), torch.zeros(3, 3, 1, device="cuda"),
                      torch.zeros(3, 2, dtype=torch.int32, device="cuda"),
                      torch.tensor([1.0, 0.0, 0.5], device="cuda"))
    assert (acc == 2).all() and (tok == 0).all()
    inp = workloads.noisy_draft_inputs("K1", 16, 1, 999, torch.float32, 7, "cuda", "gauss")
    check(sv, inp, steps=range(3))
    # K = 63, the largest ballot
    inp = workloads.noisy_draft_inputs("K63", 3, 63, 256, torch.float32, 8, "cuda", "gauss",
                                       target_std=0.3, draft_noise=0.05)
    check(sv, inp, steps=range(2))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("offset", [0.0, 40.0])
@pytest.mark.parametrize("temps", [(0.1, 0.3), (0.01, 0.03), (5.0, 20.0, 100.0)])
def test_large_logits_low_temperature(sv, dtype, offset, temps):
    """Logits shifted by +40 at low temperatures (|logit| / T up to ~5000 at
    T = 0.01) and at high ones (nearly flat rows): a shift leaves p and q
    unchanged, so the exponent arithmetic must keep its accuracy whatever the
    logits' magnitude and the temperature.  Every request against the
    oracle, debug probabilities within the 1e-6 bar, over two chunks and a
    ragged tail per row."""
    say("case: logits + %g, T in %s, %s" % (offset, temps, dtype))
    inp = workloads.noisy_draft_inputs("shift %g %s" % (offset, dtype), 16, 5, 40000, dtype, 21, "cuda",
                                       "gauss", target_std=2.0, draft_noise=0.5, temps=temps,
                                       offset=offset)
    check(sv, inp, seeds=(0, 3), steps=(0, 1))
    # Zipf rows (a long tail far below the maximum) at the same temperatures
    inp = workloads.noisy_draft_inputs("zipf shift %g %s" % (offset, dtype), 8, 4, 70001, dtype, 22, "cuda",
                                       "zipf", draft_noise=0.7, temps=temps, offset=offset)
    check(sv, inp, seeds=(1,), steps=(0, 1))


def test_invalid_requests(sv):
    say("case: invalid request data")
    inp = workloads.noisy_draft_inputs("bad", 6, 3, 64, torch.float32, 2, "cuda", "gauss")
    x = inp.draft_tokens.clone()
    T = inp.temperature.clone()
    t = inp.target.clone()
    x[1, 2] = 64
    x[2, 0] = -5
    T[3] = -1.0
    T[4] = float("nan")
    t[5, 0, :] = -float("inf")  # a row every sampled request reads
    acc, tok, dbg = run(sv, t, inp.draft, x, T)
    assert acc[0] >= 0
    for b in range(1, 6):
        assert acc[b] == -1 and (tok[b] == -1).all() and (dbg[b] == 0).all(), b
    tl = workloads.logits_numpy(t)
    dl = workloads.logits_numpy(inp.draft)
    rep = compare(tl, dl, x.cpu().numpy(), T.cpu().numpy(), acc, tok, dbg)
    assert rep.ok(), rep.failures


def test_workspace_error_counts_invalid_requests(sv):
    say("case: workspace error word")
    inp = workloads.noisy_draft_inputs("bad", 6, 3, 64, torch.float32, 2, "cuda", "gauss")
    ws = sv.make_workspace(6, 3, 64)
    ws.fill_(0x5A)  # a stale count is cleared by the verification
    run(sv, inp.target, inp.draft, inp.draft_tokens, inp.temperature, ws=ws)
    assert sv.spec_workspace_error(ws) == 0
    x = inp.draft_tokens.clone()
    T = inp.temperature.clone()
    x[1, 2] = 64
    T[4] = -1.0
    acc, _, _ = run(sv, inp.target, inp.draft, x, T, ws=ws)
    assert sv.spec_workspace_error(ws) == 2 == int((acc == -1).sum())
    # phased rows: the count comes from the final decision all the same
    sv.verify(inp.target, inp.draft, x, T, workspace=ws, phase_starts=0b10)
    assert sv.spec_workspace_error(ws, torch.cuda.current_stream().cuda_stream) == 2


def test_determinism_and_workspace_reuse(sv):
    say("case: determinism / workspace reuse")
    big = workloads.mixture_inputs("reuse", 16, 6, 40000, torch.bfloat16, 11, "cuda", temps=(0.0, 1.0),
                                   lam_lo=0.1, lam_hi=0.5)
    small = workloads.verify_tiny(seed=3, device="cuda")
    ws = sv.make_workspace(16, 6, 40000)
    assert sv.spec_verify_workspace_bytes(4, 4, 1024) <= ws.numel()
    ws.fill_(0xA5)  # stale contents are never read
    r1 = run(sv, big.target, big.draft, big.draft_tokens, big.temperature, 1, 0, ws=ws)
    r1b = run(sv, big.target, big.draft, big.draft_tokens, big.temperature, 1, 0, ws=ws)
    r2 = run(sv, small.target, small.draft, small.draft_tokens, small.temperature, 1, 0, ws=ws)
    r3 = run(sv, big.target, big.draft, big.draft_tokens, big.temperature, 1, 0, ws=ws)
    r4 = run(sv, small.target, small.draft, small.draft_tokens, small.temperature, 1, 0)
    for a, b in zip(r1, r1b):
        assert np.array_equal(a, b)
    for a, b in zip(r1, r3):
        assert np.array_equal(a, b)
    for a, b in zip(r2, r4):
        assert np.array_equal(a, b)


def test_output_law_through_the_gpu(sv):
    """The distribution-preservation theorem on the GPU outputs: 10^6
    requests sharing rows (V = 64, K = 3); tokens at each reached position
    follow p_k, acceptance counts are binomial."""
    say("case: chi-square through the GPU, 1e6 requests")
    K, V, N = 3, 64, 1_000_000
    rng = np.random.default_rng(64)
    tl = (1.5 * rng.standard_normal((1, K + 1, V))).astype(np.float32)
    dl = (tl + rng.standard_normal((1, K + 1, V))).astype(np.float32)
    p, q = softmax_rows(tl[0]), softmax_rows(dl[0])
    x = draw_categorical(q[:K], N, rng)
    t = torch.from_numpy(tl).cuda().expand(N, K + 1, V)
    d = torch.from_numpy(dl).cuda().expand(N, K + 1, V)
    acc, tok, _ = run(sv, t, d, torch.from_numpy(x).cuda(), torch.ones(N, device="cuda"), seed=77,
                      debug=False)
    pv, zs = [], []
    for k in range(K + 1):
        reach = acc >= k
        pv.append(chi2_pvalue(np.bincount(tok[reach, k], minlength=V), p[k]))
        if k < K:
            zs.append(binom_z(int((acc[reach] > k).sum()), int(reach.sum()), float(np.minimum(p[k], q[k]).sum())))
    say("p-values", pv, "z", zs)
    assert min(pv) >= 1e-4 and max(abs(z) for z in zs) < 5


def test_gptoss_vocab_full_parity(sv):
    """B=64, K=5, V=201088 bf16 Zipf rows, draft = target + N(0, 0.7): every
    request against the oracle."""
    say("case: gpt-oss vocab B64 K5 V201088, full parity")
    inp = workloads.verify_gptoss(seed=0, device="cuda")
    rep = check(sv, inp, seeds=(0,), steps=(0, 1))
    assert rep.exact >= rep.requests - 4


def _sampled_parity(sv, inp, idx, seed, step, acc, tok, dbg, rep):
    for b in idx:
        tl = workloads.logits_numpy(inp.target[b:b + 1])
        dl = workloads.logits_numpy(inp.draft[b:b + 1])
        x = inp.draft_tokens[b:b + 1].cpu().numpy()
        T = inp.temperature[b:b + 1].cpu().numpy()
        compare(tl, dl, x, T, acc[b:b + 1], tok[b:b + 1], dbg[b:b + 1], seed=seed, step=step,
                request_base=b, report=rep)


@pytest.mark.parametrize("iseed", [1, 2])
def test_headline_every_request(sv, iseed):
    """The headline recipe (B=256, K=8, V=151936 bf16) on fresh inputs: every
    request of the batch against the oracle under two Philox streams, each
    run both in one pass and with the benchmarked early-exit cut
    {0..2 | 3..8} (bit-identical)."""
    say("case: headline B256 K8 V151936, every request, inputs seed %d" % iseed)
    inp = workloads.verify_headline(seed=iseed, device="cuda")
    tl, dl = workloads.logits_numpy(inp.target), workloads.logits_numpy(inp.draft)
    x, T = inp.draft_tokens.cpu().numpy(), inp.temperature.cpu().numpy()
    rep = Report()
    for seed, step in ((iseed, 0), (2 ** 40 + iseed, 77)):
        a1, t1, d1 = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=seed, step=step,
                               debug=True)
        a2, t2, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=seed, step=step,
                              debug=True, phase_starts=0b1000)
        torch.cuda.synchronize()
        assert torch.equal(a1, a2) and torch.equal(t1, t2), (seed, step)
        compare(tl, dl, x, T, a1.cpu().numpy(), t1.cpu().numpy(), d1.cpu().numpy(), seed=seed, step=step,
                report=rep)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]


def test_headline_full_size_sampled(sv):
    """B=256, K=8, V=151936 bf16, temperatures {0, 0.6, 1}, mixture drafts:
    the whole batch in one launch (as benchmarked), 40 requests checked
    against the oracle one by one, and run-to-run bit-identical."""
    say("case: headline B256 K8 V151936, sampled parity")
    inp = workloads.verify_headline(seed=0, device="cuda")
    acc, tok, dbg = run(sv, inp.target, inp.draft, inp.draft_tokens, inp.temperature, 0, 0)
    acc2, tok2, dbg2 = run(sv, inp.target, inp.draft, inp.draft_tokens, inp.temperature, 0, 0)
    assert np.array_equal(acc, acc2) and np.array_equal(tok, tok2) and np.array_equal(dbg, dbg2)
    rng = np.random.default_rng(0)
    idx = sorted(set([0, 1, 255] + list(rng.choice(256, 37, replace=False))))
    rep = Report()
    _sampled_parity(sv, inp, idx, 0, 0, acc, tok, dbg, rep)
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    T = inp.temperature.cpu().numpy()
    say("accepted mean by T:", {float(t): float(acc[T == t].mean()) for t in np.unique(T)})
    assert (acc >= 0).all() and (acc <= 8).all()


def masked_vocabulary(inp, kind, seed):
    """Vocabulary masks as a serving stack applies them (banned tokens,
    constrained decoding): logits set to -inf in place, then the draft tokens
    drawn again from the masked draft rows.  random30: the same random 30 %
    of each target and draft row; block: tokens 40000..109999 of every row,
    which covers whole 32K row-pass chunks and whole 4096-logit segments;
    disjoint_blocks: tokens 0..59999 of the target rows and 90000.. of the
    draft rows, so that many drafted tokens have p(x) = 0."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    ninf = float("-inf")
    if kind == "random30":
        m = torch.rand(inp.target.shape, generator=g, device="cuda") < 0.3
        inp.target[m] = ninf
        inp.draft[m] = ninf
    elif kind == "block":
        inp.target[:, :, 40000:110000] = ninf
        inp.draft[:, :, 40000:110000] = ninf
    else:
        inp.target[:, :, 0:60000] = ninf
        inp.draft[:, :, 90000:] = ninf
    inp.draft_tokens = workloads.redraw_tokens(inp, seed + 1)
    return inp


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("kind", ["random30", "block", "disjoint_blocks"])
def test_masked_vocabulary(sv, kind, dtype):
    """Rows with a part of the vocabulary at -inf at the headline vocabulary
    (V = 151936; mixed temperatures 0, 0.6, 1): every request against the
    oracle, and a planned cut and the dynamic exit equal to one pass."""
    say("case: masked vocabulary %s %s" % (kind, dtype))
    inp = workloads.noisy_draft_inputs("masked %s %s" % (kind, dtype), 24, 4, 151936, dtype, 31, "cuda", "zipf",
                                       draft_noise=0.7, temps=(0.0, 0.6, 1.0))
    inp = masked_vocabulary(inp, kind, 32)
    check(sv, inp, seeds=(0, 1), steps=(0, 1))
    a1, t1, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=0, step=0)
    for ps in (0b100, sv.SPEC_PHASES_DYNAMIC):
        a2, t2, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=0, step=0,
                              phase_starts=ps)
        torch.cuda.synchronize()
        assert torch.equal(a1, a2) and torch.equal(t1, t2), ps


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_greedy_rows_with_nan(sv, dtype):
    """Greedy rows holding NaN logits (V = 70001, three statistics chunks):
    a NaN counts as -inf in the argmax, so an all-NaN row or a row with
    nothing above -inf gives token 0, and a NaN ahead of the maximum does not
    hide it.  Every request against the oracle, one pass, the planned cut, the
    dynamic exit and the vocabulary split over 2, 3 and 4 shards."""
    import oracle
    say("case: greedy rows with NaN %s" % dtype)
    B, K, V = 12, 3, 70001
    g = torch.Generator().manual_seed(21)
    t = torch.randn(B, K + 1, V, generator=g)
    d = t + 0.5 * torch.randn(B, K + 1, V, generator=g)
    nan, inf = float("nan"), float("inf")
    t[0, 0] = nan                                    # an all-NaN row, accepted (draft 0)
    t[1, 1] = nan                                    # an all-NaN row, rejected: emits 0
    t[2, 0, 0] = nan                                 # NaN at index 0 ahead of the maximum
    t[3, K] = nan                                    # an all-NaN bonus row
    t[4, 0] = -inf
    t[4, 0, 40000:] = nan                            # -inf, then NaN over the last two chunks
    t[5, 1, :40000] = nan
    t[5, 1, 40000:] = -inf
    t[5, 1, 50000] = -3.0                            # the only number, behind a NaN chunk
    t[6, 2, :32768] = nan                            # a whole NaN chunk ahead of the maximum
    t[7, 0, 10] = nan
    t[7, 0, 65000] = inf                             # +inf behind a NaN
    t[8, 1, ::2] = nan                               # every other logit NaN
    T = torch.tensor([0.0] * 9 + [0.6, 1.0, 0.8])
    tt, dd = t.to(dtype), d.to(dtype)
    tl, dl = workloads.logits_numpy(tt), workloads.logits_numpy(dd)
    x = np.array([[oracle.argmax(tl[b, k]) for k in range(K)] for b in range(B)], np.int32)
    assert x[0, 0] == 0 and x[4, 0] == 0 and x[5, 1] == 50000 and x[7, 0] == 65000
    x[1, 1] = 5                                      # the all-NaN row's argmax is 0: rejected there
    x[6, 2] = (x[6, 2] + 1) % V
    x[9:] = np.random.default_rng(22).integers(0, V, (3, K)).astype(np.int32)
    Td = T.cuda()
    tg, dg, xg = tt.cuda(), dd.cuda(), torch.from_numpy(x).cuda()
    rep = Report()
    outs = []
    for ps in (0, 0b100, sv.SPEC_PHASES_DYNAMIC):
        a, tok, dbg = sv.verify(tg, dg, xg, Td, seed=4, step=0, debug=ps == 0, phase_starts=ps)
        torch.cuda.synchronize()
        a, tok = a.cpu().numpy(), tok.cpu().numpy()
        compare(tl, dl, x, T.numpy(), a, tok, None if dbg is None else dbg.cpu().numpy(), seed=4, step=0,
                report=rep)
        outs.append((a, tok))
    for G in (2, 3, 4):
        for ps in (0, 0b100):
            a, tok, _ = sv.verify_sharded(tg, dg, xg, Td, G, seed=4, step=0, phase_starts=ps)
            torch.cuda.synchronize()
            a, tok = a.cpu().numpy(), tok.cpu().numpy()
            compare(tl, dl, x, T.numpy(), a, tok, None, seed=4, step=0, report=rep)
            outs.append((a, tok))
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    a, tok = outs[0]
    assert list(a[:9]) == [K, 1, K, K, K, K, 2, K, K]
    assert tok[1, 1] == 0 and tok[3, K] == 0 and tok[0, 0] == 0 and tok[5, 1] == 50000 and tok[7, 0] == 65000
    assert (tok < V).all()
    for a2, t2 in outs[1:]:
        np.testing.assert_array_equal(a2, a)
        np.testing.assert_array_equal(t2, tok)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_temperature_tiny_against_the_logits(sv, dtype):
    """A sampled row counts only while its largest logit m keeps
    |m| * log2(e) / T within 2^24 (the exact fp32 integers the kernels hold
    a row's scaled maximum in): temperatures 0.1 % inside that bound for all
    of a request's rows, or 0.1 % outside it for its first target row (which
    every walk reads), 1e-5 and 1e-4 against logits near 20, subnormal
    temperatures (invalid), 3e38, and ordinary ones, at V = 70001.  Every
    request against the oracle in one pass, a planned cut, the dynamic exit
    and 2 and 3 shards, and the draft sampler on the first target rows."""
    import oracle
    say("case: temperatures tiny against the logits %s" % dtype)
    B, K, V = 14, 3, 70001
    g = torch.Generator().manual_seed(61)
    t = 3 * torch.randn(B, K + 1, V, generator=g) + 15
    d = t + 0.2 * torch.randn(B, K + 1, V, generator=g)
    t[6:8] -= 40                                     # negative maxima
    d[6:8] -= 40
    t[[1, 3], 0] += 5                                # the first target row holds the largest |maximum|
    t[7, 0] -= 5
    tt, dd = t.to(dtype), d.to(dtype)
    tl, dl = workloads.logits_numpy(tt), workloads.logits_numpy(dd)
    tv, dv = tt.float().numpy(), dd.float().numpy()  # values (bf16 oracle rows are bit patterns)
    rows_max = np.array([[abs(float(np.max(tv[b, k]))) for k in range(K + 1)] +
                         [abs(float(np.max(dv[b, k]))) for k in range(K)] for b in range(B)])
    mx, m0 = rows_max.max(axis=1), rows_max[:, 0]
    assert (m0[[1, 3, 7]] == mx[[1, 3, 7]]).all()
    f = np.log2(np.e) / 2.0 ** 24
    T = np.array([mx[0] * f / 0.999, m0[1] * f / 1.001, mx[2] * f / 0.999, m0[3] * f / 1.001,
                  1e-5, 1e-4, mx[6] * f / 0.999, m0[7] * f / 1.001, 1e-40, 3e38, 0.7, 1.0, 0.0, 2e-45],
                 np.float32)
    x = np.array([[oracle.argmax(dl[b, k]) for k in range(K)] for b in range(B)], np.int32)
    x[2, 1] = (x[2, 1] + 7) % V                      # a rejection inside the range
    Td = torch.from_numpy(T).cuda()
    tg, dg, xg = tt.cuda(), dd.cuda(), torch.from_numpy(x).cuda()
    ref = oracle.verify(tl, dl, x, T, seed=6, step=1)
    assert (ref.accepted[[0, 2, 4, 5, 6, 9, 10, 11, 12]] >= 0).all()
    assert (ref.accepted[[1, 3, 7, 8, 13]] == -1).all()
    rep = Report()
    outs = []
    ws = sv.make_workspace(B, K, V)
    for ps in (0, 0b100, sv.SPEC_PHASES_DYNAMIC):
        a, tok, dbg = sv.verify(tg, dg, xg, Td, seed=6, step=1, debug=ps == 0, phase_starts=ps, workspace=ws)
        torch.cuda.synchronize()
        a, tok = a.cpu().numpy(), tok.cpu().numpy()
        compare(tl, dl, x, T, a, tok, None if dbg is None else dbg.cpu().numpy(), seed=6, step=1, report=rep)
        # the out-of-range rows and subnormal temperatures are counted as data errors
        assert sv.spec_workspace_error(ws) == int((a == -1).sum()) == 5, ps
        outs.append((a, tok))
    for G in (2, 3):
        a, tok, _ = sv.verify_sharded(tg, dg, xg, Td, G, seed=6, step=1)
        torch.cuda.synchronize()
        a, tok = a.cpu().numpy(), tok.cpu().numpy()
        compare(tl, dl, x, T, a, tok, None, seed=6, step=1, report=rep)
        outs.append((a, tok))
    say(rep.summary())
    assert rep.ok(), rep.failures[:5]
    for a2, t2 in outs[1:]:
        np.testing.assert_array_equal(a2, outs[0][0])
        np.testing.assert_array_equal(t2, outs[0][1])
    # the draft sampler on the first target rows at the same temperatures
    lg = tt[:, 0].contiguous()
    ri = torch.arange(B, dtype=torch.int32).reshape(B, 1)
    tokd = sv.draft_sample(lg.cuda(), ri.cuda(), Td, seed=9).cpu().numpy()
    refd = oracle.draft_sample(workloads.logits_numpy(lg), ri.numpy(), T, seed=9)
    np.testing.assert_array_equal(tokd, refd.tokens)
    assert (tokd[[1, 3, 7, 8, 13], 0] == -1).all() and (tokd[[0, 2, 4, 5, 6, 9, 10, 11, 12], 0] >= 0).all()


def test_largest_vocabulary(sv):
    """V = SPEC_MAX_V (2^31 - 2^16, bf16: rows of 4.3 GB, byte offsets past
    2^31): rows that are -inf except at 24 indices spread over the whole row
    (past 2^30 and at its end among them), 16 requests sharing them, mixed
    temperatures.  A -inf logit carries no weight anywhere in the method, and
    the inverse CDF and the argmax keep vocabulary order, so the outputs must
    be the oracle's on the rows cut down to those 24 indices, mapped back.
    One pass, a planned cut and the dynamic exit, and the draft sampler on
    the same rows."""
    import oracle
    say("case: the largest vocabulary, V = %d" % sv.SPEC_MAX_V)
    B, K, V = 16, 1, sv.SPEC_MAX_V
    rng = np.random.default_rng(71)
    S = np.unique(np.concatenate([rng.integers(0, V, 16), [0, 5, 2**30 - 1, 2**30, 2**30 + 7, V - 4097, V - 2,
                                                            V - 1]]))
    n = len(S)
    vt = (2.0 * rng.standard_normal((K + 1, n))).astype(np.float32)
    vd = (vt[:K] + 0.7 * rng.standard_normal((K, n))).astype(np.float32)
    vt[0, rng.random(n) < 0.2] = -np.inf           # some of the indices hold no target weight either
    dev = torch.device("cuda")
    idx = torch.from_numpy(S).to(dev)
    t = torch.full((1, K + 1, V), float("-inf"), dtype=torch.bfloat16, device=dev)
    d = torch.full((1, K, V), float("-inf"), dtype=torch.bfloat16, device=dev)
    for k in range(K + 1):
        t[0, k, idx] = torch.from_numpy(vt[k]).to(dev).bfloat16()
    for k in range(K):
        d[0, k, idx] = torch.from_numpy(vd[k]).to(dev).bfloat16()
    # the cut-down rows as stored, shared by every request (leading dimension 1)
    tcl = workloads.logits_numpy(t[0][:, idx].unsqueeze(0))
    dcl = workloads.logits_numpy(d[0][:, idx].unsqueeze(0))
    xc = rng.integers(0, n, (B, K)).astype(np.int32)
    T = np.array([0.0, 0.0, 0.7, 1.0] * 4, np.float32)
    xc[0, 0] = xc[1, 0] = oracle.argmax(tcl[0, 0])  # greedy requests whose draft is the target argmax
    ref = oracle.verify(tcl, dcl, xc, T, seed=12, step=3, debug=False, trace=False)
    assert (ref.accepted >= 0).all() and ref.accepted[0] == 1
    want_tok = np.where(ref.tokens >= 0, S[np.maximum(ref.tokens, 0)], -1)
    tg, dg = t.expand(B, K + 1, V), d.expand(B, K, V)
    xg = torch.from_numpy(S[xc].astype(np.int32)).to(dev)
    Tg = torch.from_numpy(T).to(dev)
    for ps in (0, 0b10, sv.SPEC_PHASES_DYNAMIC):
        a, tok, _ = sv.verify(tg, dg, xg, Tg, seed=12, step=3, phase_starts=ps)
        torch.cuda.synchronize()
        a, tok = a.cpu().numpy(), tok.cpu().numpy()
        say("  phase_starts %#x: accepted %s" % (ps, a.tolist()))
        np.testing.assert_array_equal(a, ref.accepted)
        np.testing.assert_array_equal(tok, want_tok)
    # the draft sampler on the two target rows, as a [2, V] drafter buffer
    ri = torch.from_numpy(rng.integers(0, K + 1, (B, 3)).astype(np.int32)).to(dev)
    tokd = sv.draft_sample(t[0], ri, Tg, seed=5, step=1).cpu().numpy()
    refd = oracle.draft_sample(tcl[0], ri.cpu().numpy(), T, seed=5, step=1)
    np.testing.assert_array_equal(tokd, np.where(refd.tokens >= 0, S[np.maximum(refd.tokens, 0)], -1))
    del t, d, tg, dg
    torch.cuda.empty_cache()


def test_batch_past_the_3d_grid(sv):
    """B = 70000 requests (past the 65535 the row pass's 3-D grid holds in z,
    so its workgroups decode their request from the linear index), K = 3,
    V = 300 fp32, mixed temperatures: every request against the oracle in
    one pass, a planned cut, the dynamic exit and over 2 vocabulary shards."""
    say("case: B = 70000 (linear row-pass grid)")
    inp = workloads.noisy_draft_inputs("B70000", 70000, 3, 300, torch.float32, 73, "cuda", "gauss",
                                       target_std=1.5, draft_noise=0.6, temps=(0.0, 0.6, 1.0))
    tl, dl, x, T = host(inp)
    for ps in (0, 0b100, sv.SPEC_PHASES_DYNAMIC):
        acc, tok, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=9, step=2,
                                phase_starts=ps)
        torch.cuda.synchronize()
        rep = compare(tl, dl, x, T, acc.cpu().numpy(), tok.cpu().numpy(), None, seed=9, step=2)
        say("  phase_starts %#x:" % ps, rep.summary())
        assert rep.ok(), rep.failures[:5]
    # the vocabulary split over 2 shards (linear grids of their own)
    acc, tok, _ = sv.verify_sharded(inp.target, inp.draft, inp.draft_tokens, inp.temperature, 2, seed=9, step=2)
    torch.cuda.synchronize()
    rep = compare(tl, dl, x, T, acc.cpu().numpy(), tok.cpu().numpy(), None, seed=9, step=2)
    say("  2 shards:", rep.summary())
    assert rep.ok(), rep.failures[:5]


@pytest.mark.parametrize("V", [5000, 70001])
def test_largest_draft_count_every_mode(sv, V):
    """K = SPEC_MAX_K = 63 (one wave64 ballot) with drafts close to the target
    so that requests walk far, mixed temperatures: every request against the
    oracle in one pass, a four-phase cut and the dynamic exit (whose decider
    window covers 128 positions at V = 5000 and 42 at V = 70001)."""
    say("case: K = 63, V = %d, every mode" % V)
    inp = workloads.mixture_inputs("K63 V%d" % V, 24, sv.SPEC_MAX_K, V, torch.bfloat16, 75, "cuda",
                                   temps=(0.0, 0.6, 1.0), lam_lo=0.01, lam_hi=0.08)
    tl, dl, x, T = host(inp)
    for ps in (0, (1 << 8) | (1 << 20) | (1 << 40), sv.SPEC_PHASES_DYNAMIC):
        acc, tok, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=3, step=1,
                                phase_starts=ps)
        torch.cuda.synchronize()
        a = acc.cpu().numpy()
        rep = compare(tl, dl, x, T, a, tok.cpu().numpy(), None, seed=3, step=1)
        say("  phase_starts %#x: mean accepted %.1f," % (ps, a.mean()), rep.summary())
        assert rep.ok(), rep.failures[:5]
