"""Early-exit verification on the GPU (rows read in phases, only for requests
still alive, or in one pass whose workgroups decide as the rows come in)
through the C ABI.

For every case and phase plan, and for the dynamic exit (DYN), the accepted
counts and output tokens must be bit-identical to the one-pass launch on the
same inputs, the debug probabilities must equal the one-pass ones on every
position whose phase was read (dynamic: every position up to the stop) and
be 0 past it, and the outputs must meet the oracle bar of ``parity.py``.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from parity import Report, compare

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rejection_sampling_verify_03_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


DYN = 1  # phase_starts of the dynamic early exit (SPEC_PHASES_DYNAMIC)


def phase_end(a, mask, K):
    """End (exclusive) of the phase holding position a under the cut `mask`
    (the dynamic exit reports positions up to the stop)."""
    e = a + 1
    if mask == DYN:
        return e
    while e <= K and not (mask >> e) & 1:
        e += 1
    return e


def all_masks(K):
    return [m << 1 for m in range(1 << K)]


def one_vs_phased(sv, inp, mask, seed=0, step=0, x=None, T=None, target=None):
    x = inp.draft_tokens if x is None else x
    T = inp.temperature if T is None else T
    target = inp.target if target is None else target
    K = x.shape[1]
    a1, t1, d1 = sv.verify(target, inp.draft, x, T, seed=seed, step=step, debug=True)
    a2, t2, d2 = sv.verify(target, inp.draft, x, T, seed=seed, step=step, debug=True, phase_starts=mask)
    torch.cuda.synchronize()
    a1, t1, d1 = a1.cpu().numpy(), t1.cpu().numpy(), d1.cpu().numpy()
    a2, t2, d2 = a2.cpu().numpy(), t2.cpu().numpy(), d2.cpu().numpy()
    assert np.array_equal(a1, a2), ("accepted differ", bin(mask))
    assert np.array_equal(t1, t2), ("tokens differ", bin(mask))
    for b in range(len(a1)):
        if a1[b] < 0:
            assert (d2[b] == 0).all()
            continue
        e = min(phase_end(int(a1[b]), mask, K), K)
        assert np.array_equal(d1[b, :e], d2[b, :e]), (b, bin(mask))
        assert (d2[b, e:] == 0).all(), (b, bin(mask))
    return a2, t2


def oracle_check(inp, acc, tok, seed, step, idx=None):
    rep = Report()
    if idx is None:
        compare(workloads.logits_numpy(inp.target), workloads.logits_numpy(inp.draft),
                inp.draft_tokens.cpu().numpy(), inp.temperature.cpu().numpy(), acc, tok, None,
                seed=seed, step=step, report=rep)
    else:
        for b in idx:
            compare(workloads.logits_numpy(inp.target[b:b + 1]), workloads.logits_numpy(inp.draft[b:b + 1]),
                    inp.draft_tokens[b:b + 1].cpu().numpy(), inp.temperature[b:b + 1].cpu().numpy(),
                    acc[b:b + 1], tok[b:b + 1], None, seed=seed, step=step, request_base=int(b), report=rep)
    say("  ", rep.summary())
    assert rep.ok(), rep.failures[:5]


def test_every_plan_tiny(sv):
    """B=4, K=4, V=1024 fp32: all 16 cuts of the positions, 8 steps each."""
    say("case: early exit, every plan and the dynamic exit, B4 K4 V1024 fp32")
    inp = workloads.verify_tiny(seed=0, device="cuda")
    for mask in all_masks(inp.K) + [DYN]:
        for step in range(8):
            acc, tok = one_vs_phased(sv, inp, mask, seed=1, step=step)
            if mask in (0b11110, DYN) and step < 2:
                oracle_check(inp, acc, tok, 1, step)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 70001), (torch.float32, 33000)])
def test_plans_multi_chunk_mixed_temperatures(sv, dtype, V):
    say("case: early exit B12 K5 V%d %s mixed T" % (V, dtype))
    inp = workloads.mixture_inputs("mixed B12 K5 V%d" % V, 12, 5, V, dtype, 3, "cuda",
                                   temps=(0.0, 0.6, 1.0), lam_lo=0.05, lam_hi=0.6)
    for mask in [1 << 1, 1 << 3, 1 << 5, 0b111110, 0b101010, DYN]:
        for step in range(2):
            acc, tok = one_vs_phased(sv, inp, mask, seed=5, step=step)
            oracle_check(inp, acc, tok, 5, step)


def test_plans_scalar_path_and_K63(sv):
    say("case: early exit, scalar path and K=63")
    inp = workloads.noisy_draft_inputs("scalar V20003", 6, 4, 20003, torch.bfloat16, 1, "cuda", "gauss",
                                       target_std=2.0, draft_noise=0.5)
    for mask in [0b11110, 0b00100, DYN]:
        acc, tok = one_vs_phased(sv, inp, mask, step=3)
        oracle_check(inp, acc, tok, 0, 3)
    inp = workloads.noisy_draft_inputs("K63", 3, 63, 256, torch.float32, 8, "cuda", "gauss",
                                       target_std=0.3, draft_noise=0.05)
    rng = np.random.default_rng(63)
    some = rng.choice(np.arange(1, 64), 9, replace=False)
    masks = [(1 << 64) - 2, 1 << 1, 1 << 63, int(sum(1 << int(k) for k in some)), DYN]
    for mask in masks:
        for step in range(2):
            acc, tok = one_vs_phased(sv, inp, mask, step=step)
    oracle_check(inp, acc, tok, 0, 1)


def test_invalid_requests_phased(sv):
    """Invalid tokens anywhere and invalid temperatures are caught by the first
    decision; a row without a finite normaliser at a position every request
    reaches is caught in every mode."""
    say("case: early exit, invalid request data")
    inp = workloads.noisy_draft_inputs("bad", 6, 3, 64, torch.float32, 2, "cuda", "gauss")
    x = inp.draft_tokens.clone()
    T = inp.temperature.clone()
    t = inp.target.clone()
    x[1, 2] = 64
    x[2, 0] = -5
    T[3] = -1.0
    T[4] = float("nan")
    t[5, 0, :] = -float("inf")
    for mask in [0b0010, 0b1110, 0b1000, DYN]:
        acc, tok = one_vs_phased(sv, inp, mask, x=x, T=T, target=t)
        assert acc[0] >= 0
        for b in range(1, 6):
            assert acc[b] == -1 and (tok[b] == -1).all(), (b, bin(mask))


def test_rows_past_the_stop_do_not_count(sv):
    """Position 0 rejects with certainty (the draft token lies outside the
    target's support), so rows of later positions without a finite maximum,
    or with a NaN, leave the request valid in every mode; the same row at
    the stop, or the bonus row of a request that accepts everything, makes
    it invalid (explainer page, section "核心思想": the positions are taken
    in order and the first rejection ends the request).  Every mode equals
    the oracle."""
    say("case: rows past the stop, every mode")
    B, K, V = 8, 4, 3000
    g = torch.Generator().manual_seed(17)
    t = torch.full((B, K + 1, V), -float("inf"))
    d = torch.full((B, K + 1, V), -float("inf"))
    t[:, 0, :1500] = torch.randn(B, 1500, generator=g)
    d[:, 0, 1500:] = torch.randn(B, 1500, generator=g)
    t[:, 1:, :] = torch.randn(B, K, V, generator=g)
    d[:, 1:, :] = t[:, 1:, :]
    x = torch.randint(1500, V, (B, K), generator=g, dtype=torch.int32)
    T = torch.full((B,), 0.7)
    t[1, 2, 7] = float("nan")          # past the stop
    t[2, 3, :] = -float("inf")         # past the stop
    d[3, 1, :] = -float("inf")         # past the stop
    t[4, 0, :] = -float("inf")         # at the stop: invalid
    d[5, 0, :] = -float("inf")         # at the stop: invalid
    # requests 6 and 7 accept everything (identical rows everywhere)
    t[6:, 0, :] = torch.randn(2, V, generator=g)
    d[6:, 0, :] = t[6:, 0, :]
    x[6:] = torch.randint(0, V, (2, K), generator=g, dtype=torch.int32)
    t[7, K, :] = -float("inf")         # request 7's bonus row: invalid
    inp = type("Inp", (), {})()
    inp.target, inp.draft = t.cuda(), d.cuda()
    inp.draft_tokens, inp.temperature = x.cuda(), T.cuda()
    want = [0, 0, 0, 0, -1, -1, K, -1]
    for mask in [0, 0b0100, 0b11110, DYN]:
        a, tok, dbg = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=3, step=1,
                                debug=True, phase_starts=mask)
        torch.cuda.synchronize()
        a = a.cpu().numpy()
        assert list(a) == want, (bin(mask), list(a))
        rep = compare(workloads.logits_numpy(t), workloads.logits_numpy(d), x.numpy(), T.numpy(),
                      a, tok.cpu().numpy(), dbg.cpu().numpy() if mask == 0 else None, seed=3, step=1)
        assert rep.ok(), (bin(mask), rep.failures[:3])


def test_headline_planned(sv):
    """B=256, K=8, V=151936 bf16 as benchmarked: plans from the measured
    survival curve of one step at two boundary prices (the decision kernel
    alone, and the price the library gives this batch shape, which the
    benchmark plans with), each 3 steps bit-identical to one pass and 24
    requests against the oracle."""
    say("case: early exit, headline B256 K8 V151936 with measured plans")
    inp = workloads.verify_headline(seed=0, device="cuda")
    B, K, V = inp.B, inp.K, inp.V
    acc, _, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=0, step=100)
    surv = sv.survival_from_accepted(acc.cpu().numpy(), K)
    f = float((inp.temperature > 0).float().mean())
    masks = []
    for cost in (0.7, sv.spec_verify_phase_cost(B, K, V, sv.SPEC_BF16)):
        mask = sv.spec_verify_plan_phases(K, surv, f, cost)
        say("  survival", [round(s, 3) for s in surv], "cost", round(cost, 3), "plan", bin(mask))
        assert mask != 0
        if mask not in masks:
            masks.append(mask)
    masks.append(DYN)
    for i, mask in enumerate(masks):
        for step in range(3):
            acc, tok = one_vs_phased(sv, inp, mask, step=step)
        rng = np.random.default_rng(2 + i)
        oracle_check(inp, acc, tok, 0, 2, idx=sorted(rng.choice(inp.B, 24, replace=False)))


def test_gptoss_vocab_planned_full_parity(sv):
    """B=64, K=5, V=201088 bf16: every position its own phase, every request
    against the oracle."""
    say("case: early exit, gpt-oss vocab B64 K5 V201088, full parity")
    inp = workloads.verify_gptoss(seed=0, device="cuda")
    acc, tok = one_vs_phased(sv, inp, 0b111110, step=0)
    oracle_check(inp, acc, tok, 0, 0)
    acc, tok = one_vs_phased(sv, inp, DYN, step=1)
    oracle_check(inp, acc, tok, 0, 1)


def test_dynamic_exit_graph_replays_on_new_inputs(sv):
    """The dynamic exit captured in a HIP graph and replayed on new inputs
    written into the captured buffers between replays: each replay equals an
    eager one-pass launch on the same inputs.  (The records a launch writes
    carry a tag that the launch counter in the workspace changes at every
    launch, replays included; records of an earlier replay must not pass for
    this one's.)"""
    say("case: dynamic exit, graph replays on new inputs")
    dev = torch.device("cuda")
    B, K, V = 48, 6, 40000
    vin = workloads.mixture_inputs("dyn graph", B, K, V, torch.bfloat16, 31, dev, temps=(0.0, 0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.6)
    tgt, dft, x, T = vin.target.clone(), vin.draft.clone(), vin.draft_tokens.clone(), vin.temperature.clone()
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ws = sv.make_workspace(B, K, V, dev)
    a = sv.verify_args(tgt, dft, x, T, acc, tok, None, ws, seed=8, step=2, phase_starts=DYN)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        assert sv.spec_verify_launch(a, s.cuda_stream) == sv.SPEC_OK
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        assert sv.spec_verify_launch(a, torch.cuda.current_stream().cuda_stream) == sv.SPEC_OK
    for rep in range(5):
        nin = workloads.mixture_inputs("dyn graph %d" % rep, B, K, V, torch.bfloat16, 40 + rep, dev,
                                       temps=(0.0, 0.6, 1.0), lam_lo=0.05, lam_hi=0.6)
        tgt.copy_(nin.target)
        dft.copy_(nin.draft)
        x.copy_(nin.draft_tokens)
        T.copy_(nin.temperature)
        acc.fill_(-5)
        tok.fill_(-5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a1, t1, _ = sv.verify(nin.target, nin.draft, nin.draft_tokens, nin.temperature, seed=8, step=2)
        torch.cuda.synchronize()
        assert torch.equal(acc, a1) and torch.equal(tok, t1), rep
    say("  5 replays on new inputs equal to the eager one pass")


@pytest.mark.parametrize("B,K,V,dtype", [(1, 1, 9, torch.float32), (3, 2, 9, torch.bfloat16),
                                         (2, 1, 4_300_000, torch.bfloat16), (5, 3, 302151, torch.bfloat16)])
def test_dynamic_exit_edge_shapes(sv, B, K, V, dtype):
    """The dynamic exit at the edges of its grid: one request, one draft, a
    row of one chunk, rows of more chunks than a decider can load at once
    (V = 4.3M: 132 chunks a row, so no decision is taken and every row is
    read) and of ten; bit-identical to one pass, and against the oracle."""
    say("case: dynamic exit B%d K%d V%d %s" % (B, K, V, dtype))
    inp = workloads.mixture_inputs("dyn edge", B, K, V, dtype, 5 + K, "cuda", temps=(0.0, 0.7, 1.0),
                                   lam_lo=0.05, lam_hi=0.6)
    for step in range(3):
        acc, tok = one_vs_phased(sv, inp, DYN, seed=2, step=step)
        if V < 1_000_000 or step == 0:
            oracle_check(inp, acc, tok, 2, step)


def test_dynamic_exit_random_shapes(sv):
    """Twenty seeded random shapes (B, K, V, dtype, temperatures, ragged
    counts or not, seed and step): the dynamic exit bit-identical to one pass
    on every output, debug probabilities up to each stop included."""
    say("case: dynamic exit, random shapes")
    rng = np.random.default_rng(2026)
    for it in range(20):
        B = int(rng.integers(1, 300))
        K = int(rng.integers(1, 12))
        V = int(rng.choice([37, 1000, 4096, 33000, 70001, 151936]))
        dtype = torch.bfloat16 if rng.random() < 0.7 else torch.float32
        temps = (0.0, 0.6, 1.0) if rng.random() < 0.7 else (1.0,)
        inp = workloads.mixture_inputs("rand %d" % it, B, K, V, dtype, 100 + it, "cuda", temps=temps,
                                       lam_lo=0.05, lam_hi=0.7)
        kw = {}
        if rng.random() < 0.4:
            kb = torch.from_numpy(rng.integers(0, K + 1, B).astype(np.int32)).cuda()
            kw["num_drafts"] = kb
        seed, step = int(rng.integers(0, 2**63)), int(rng.integers(0, 2**32))
        a1, t1, d1 = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=seed, step=step,
                               debug=True, **kw)
        a2, t2, d2 = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=seed, step=step,
                               debug=True, phase_starts=DYN, **kw)
        torch.cuda.synchronize()
        assert torch.equal(a1, a2) and torch.equal(t1, t2), (it, B, K, V, dtype)
        a = a1.cpu().numpy()
        d1, d2 = d1.cpu().numpy(), d2.cpu().numpy()
        for b in range(B):
            if a[b] >= 0:
                n = min(int(a[b]) + 1, K)
                assert np.array_equal(d1[b, :n], d2[b, :n]) and (d2[b, n:] == 0).all(), (it, b)
        say("  %2d: B=%d K=%d V=%d %s ragged=%s accepted %s" % (it, B, K, V, str(dtype)[6:], "num_drafts" in kw,
                                                           np.bincount(a[a >= 0], minlength=K + 1)))


def test_dynamic_exit_first_launch_on_zeroed_workspace(sv):
    """The first launch on a workspace of zero bytes (a fresh allocation, or
    the library's own no-alloc array at load) starts from launch counter 0:
    the record words it has not written yet must not pass for this launch's,
    so the outputs equal one pass."""
    say("case: dynamic exit, first launch on a zeroed workspace")
    dev = torch.device("cuda")
    B, K, V = 192, 8, 151936
    inp = workloads.mixture_inputs("dyn zero ws", B, K, V, torch.bfloat16, 77, dev, temps=(0.0, 0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.5)
    a1, t1, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=4, step=9)
    for trial in range(3):
        ws = torch.zeros(sv.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
        a2, t2, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=4, step=9,
                              workspace=ws, phase_starts=DYN)
        torch.cuda.synchronize()
        assert (a2 >= 0).all(), (trial, int((a2 < 0).sum()))
        assert torch.equal(a1, a2) and torch.equal(t1, t2), trial
    say("  3 fresh zeroed workspaces: equal to one pass")


def test_dynamic_exit_records_from_2_31_launches_ago_do_not_pass(sv):
    """Records left in the workspace by a launch 2^31 launches back (where
    32-bit tags of the low bits of the counter read the same) must not pass
    for this launch's, whole or caught half-written: a dynamic launch at
    counter 5 leaves records of other inputs, the counter is moved to
    5 + 2^31, and the next dynamic launch on new inputs equals one pass."""
    say("case: dynamic exit, records of a launch 2^31 back")
    dev = torch.device("cuda")
    B, K, V = 192, 8, 151936
    old = workloads.mixture_inputs("dyn stale", B, K, V, torch.bfloat16, 78, dev, temps=(0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.5)
    new = workloads.mixture_inputs("dyn fresh", B, K, V, torch.bfloat16, 79, dev, temps=(0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.5)
    a1, t1, _ = sv.verify(new.target, new.draft, new.draft_tokens, new.temperature, seed=4, step=9)
    for trial in range(3):
        ws = torch.zeros(sv.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
        counter = ws[8:16].view(torch.int64)
        counter.fill_(5)
        sv.verify(old.target, old.draft, old.draft_tokens, old.temperature, seed=1, step=3, workspace=ws,
                  phase_starts=DYN)
        torch.cuda.synchronize()
        counter.fill_(5 + 2 ** 31)
        a2, t2, _ = sv.verify(new.target, new.draft, new.draft_tokens, new.temperature, seed=4, step=9,
                              workspace=ws, phase_starts=DYN)
        torch.cuda.synchronize()
        assert (a2 >= 0).all(), (trial, int((a2 < 0).sum()))
        assert torch.equal(a1, a2) and torch.equal(t1, t2), trial
    say("  3 workspaces with records of a launch 2^31 back: equal to one pass")


def test_dynamic_exit_on_a_workspace_cut_from_another(sv):
    """Two workspaces cut from one allocation 1536 bytes apart (as an
    allocator hands out a freed block again after small output tensors took
    its start), their launch counters holding the same leftover value: the
    tagged records a dynamic exit on other inputs leaves in the first lie in
    the second's record area, 24 records off, carrying the tag the second's
    launch would expect if the tag were the counter alone.  The dynamic exit
    on the second must equal one pass (the tag also depends on the
    workspace's address)."""
    say("case: dynamic exit on a workspace cut from another one's memory")
    dev = torch.device("cuda")
    B, K, V = 24, 6, 50000
    inp = workloads.mixture_inputs("dyn carved ws", B, K, V, torch.bfloat16, 81, dev, temps=(0.0, 0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.6)
    old = workloads.mixture_inputs("dyn carved ws, other", B, K, V, torch.bfloat16, 82, dev,
                                   temps=(0.0, 0.6, 1.0), lam_lo=0.05, lam_hi=0.6)
    a1, t1, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=5, step=0)
    n = sv.spec_verify_workspace_bytes(B, K, V)
    for trial, counter0 in enumerate((7, 0x40297C9488840000, 2 ** 31 - 1)):
        big = torch.zeros(n + 2 * 1536, dtype=torch.uint8, device=dev)
        ws_a, ws_b = big[1536:1536 + n], big[3072:3072 + n]
        ws_a[8:16].view(torch.int64).fill_(counter0)
        sv.verify(old.target, old.draft, old.draft_tokens, old.temperature, seed=2, step=1, workspace=ws_a,
                  phase_starts=DYN)
        torch.cuda.synchronize()
        ws_b[8:16].view(torch.int64).fill_(counter0)  # the same counter as the first launch ran at
        a2, t2, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=5, step=0,
                              workspace=ws_b, phase_starts=DYN)
        torch.cuda.synchronize()
        assert (a2 >= 0).all(), (trial, int((a2 < 0).sum()))
        assert torch.equal(a1, a2) and torch.equal(t1, t2), trial
    say("  3 counters: equal to one pass")


def test_concurrent_calls_on_two_streams(sv):
    """Two halves of one batch verified at the same time on two streams, each
    call with its own workspace (request_base keeping the halves' uniforms
    those of the whole batch): one pass, a planned cut and the dynamic exit,
    and the two halves under different modes at once.  The outputs equal the
    whole batch verified in one call."""
    say("case: concurrent verifications on two streams")
    dev = torch.device("cuda")
    B, K, V = 128, 8, 151936
    inp = workloads.mixture_inputs("two streams", B, K, V, torch.bfloat16, 91, dev, temps=(0.0, 0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.6)
    a1, t1, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=3, step=4)
    torch.cuda.synchronize()
    h = B // 2
    halves = [slice(0, h), slice(h, B)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    wss = [sv.make_workspace(h, K, V, dev) for _ in range(2)]
    for modes in ((0, 0), (0b1000, 0b1000), (DYN, DYN), (DYN, 0b1000), (0, DYN)):
        outs = []
        for i, sl in enumerate(halves):
            acc = torch.full((h,), -5, dtype=torch.int32, device=dev)
            tok = torch.full((h, K + 1), -5, dtype=torch.int32, device=dev)
            outs.append((acc, tok))
            a = sv.verify_args(inp.target[sl], inp.draft[sl], inp.draft_tokens[sl], inp.temperature[sl], acc, tok,
                               None, wss[i], seed=3, step=4, phase_starts=modes[i], request_base=sl.start)
            streams[i].wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(streams[i]):
                assert sv.spec_verify_launch(a, streams[i].cuda_stream) == sv.SPEC_OK
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        a2 = torch.cat([o[0] for o in outs])
        t2 = torch.cat([o[1] for o in outs])
        assert torch.equal(a1, a2) and torch.equal(t1, t2), modes
        say("  modes %s: equal to the whole batch in one call" % (modes,))
