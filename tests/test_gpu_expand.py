"""GPU P-EAGLE expansion through the C ABI against the CPU oracle: every output
bit-exact (token ids, positions, masks, new-token indices, hidden map, start
indices, KV-cache slot mapping and the gathered hidden rows)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rejection_sampling_verify_03_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(e):
    for k in ("in_token_ids", "in_positions", "in_start", "accepted", "bonus", "target_hidden", "mask_hidden"):
        setattr(e, k, getattr(e, k).cuda())
    return e


def run_both(sv, e, with_hidden=True, accepted=None, in_start=None, hidden=None, block_table=None,
             block_size=0):
    acc = e.accepted if accepted is None else accepted
    st = e.in_start if in_start is None else in_start
    th = (e.target_hidden if hidden is None else hidden) if with_hidden else None
    out = sv.expand(e.in_token_ids, e.in_positions, st, acc, e.bonus, e.K, e.mask_id, th,
                    e.mask_hidden if with_hidden else None, block_table=block_table, block_size=block_size)
    torch.cuda.synchronize()
    ref = oracle.expand(e.in_token_ids.cpu().numpy(), e.in_positions.cpu().numpy(), st.cpu().numpy(),
                        acc.cpu().numpy(), e.bonus.cpu().numpy(), e.K, e.mask_id,
                        workloads.bf16_bits(th) if with_hidden else None,
                        workloads.bf16_bits(e.mask_hidden) if with_hidden else None,
                        block_table=None if block_table is None else block_table.cpu().numpy(),
                        block_size=block_size)
    return out, ref


def table_for(e, block_size, seed, unmapped_fraction=0.0, max_blocks=None):
    """A block table covering every position of the batch (or max_blocks)."""
    if max_blocks is None:
        top = int(e.in_positions.max()) + e.K + 2
        max_blocks = top // block_size + 1
    return workloads.block_tables(e.B, max_blocks, seed=seed, device="cuda",
                                  unmapped_fraction=unmapped_fraction)


def assert_same(out, ref, with_hidden=True, valid_rows=None):
    nti = out.new_token_indices.cpu().numpy()
    np.testing.assert_array_equal(nti, ref.new_token_indices)
    ok_req = (ref.new_token_indices[:, 0] >= 0)
    if (ref.out_start != -7).all():
        np.testing.assert_array_equal(out.out_start.cpu().numpy(), ref.out_start)
    # slots of valid requests (invalid ones are not written by either side)
    mask = ref.out_token_ids != -7
    for name in ("out_token_ids", "out_positions", "rejected_mask", "masked_mask"):
        np.testing.assert_array_equal(getattr(out, name).cpu().numpy()[mask], getattr(ref, name)[mask], name)
    hm_mask = ref.hidden_map != -7
    np.testing.assert_array_equal(out.hidden_map.cpu().numpy()[hm_mask], ref.hidden_map[hm_mask])
    if ref.slot_mapping is not None:
        np.testing.assert_array_equal(out.slot_mapping.cpu().numpy()[mask], ref.slot_mapping[mask], "slots")
    if with_hidden:
        got = workloads.bf16_bits(out.out_hidden)
        np.testing.assert_array_equal(got[mask], ref.out_hidden[mask])
    return ok_req


def test_full_size_expand(sv):
    """B=512, K=8, H=2880 (the GPT-OSS-20B hidden width), ragged accepted
    counts, positions from offsets in [0, 16384)."""
    say("case: expand B512 K8 H2880")
    for seed in (0, 1):
        e = workloads.expand_inputs(B=512, K=8, seed=seed, device="cuda")
        out, ref = run_both(sv, e)
        assert ref.n_bad == 0
        assert_same(out, ref)
    # with the KV-cache slot mapping through a paged block table of 16 slots per block
    out, ref = run_both(sv, e, block_table=table_for(e, 16, seed=7), block_size=16)
    assert_same(out, ref)
    sm = out.slot_mapping.cpu().numpy()
    assert ((sm == -1) == out.rejected_mask.cpu().numpy().astype(bool)).all()


def test_slot_mapping_edges(sv):
    """Unmapped blocks, positions past the table, one slot per block, and a
    block table inside a wider buffer."""
    say("case: expand slot mapping edges")
    e = workloads.expand_inputs(B=100, K=5, H=16, seed=11, device="cuda", max_offset=200)
    for bs, frac, mb in [(16, 0.3, None), (1, 0.0, None), (4, 0.0, 30), (7, 0.2, 12)]:
        bt = table_for(e, bs, seed=bs, unmapped_fraction=frac, max_blocks=mb)
        out, ref = run_both(sv, e, block_table=bt, block_size=bs)
        assert_same(out, ref)
    wide = torch.full((e.B, 64), 5, dtype=torch.int32, device="cuda")
    bt = table_for(e, 16, seed=3)
    wide[:, :bt.shape[1]] = bt
    out, ref = run_both(sv, e, block_table=wide[:, :bt.shape[1]], block_size=16)
    assert_same(out, ref)
    # no logical block at all: every slot -1
    out, ref = run_both(sv, e, block_table=wide[:, :0], block_size=16)
    assert_same(out, ref)
    assert (out.slot_mapping.cpu().numpy()[ref.out_token_ids != -7] == -1).all()


@pytest.mark.parametrize("K,H", [(1, 64), (2, 2880), (5, 100), (8, 7), (63, 16)])
def test_shapes_and_scalar_path(sv, K, H):
    """K = 1 (no MASK slots), H not a multiple of 8 (2-byte copy path)."""
    say("case: expand K%d H%d" % (K, H))
    e = workloads.expand_inputs(B=37, K=K, H=H, seed=K + H, device="cuda")
    out, ref = run_both(sv, e)
    assert_same(out, ref)


def test_ragged_requests_and_strided_hidden(sv):
    say("case: expand ragged")
    rng = np.random.default_rng(5)
    n = rng.integers(1, 40, 300)
    e = workloads.expand_inputs(B=300, K=6, H=256, seed=5, device="cuda", n_per_request=n)
    out, ref = run_both(sv, e)
    assert_same(out, ref)
    # hidden rows inside a wider buffer (row stride > H)
    wide = torch.zeros(e.N_in, 320, dtype=torch.bfloat16, device="cuda")
    wide[:, :256] = e.target_hidden
    out2, ref2 = run_both(sv, e, hidden=wide[:, :256])
    assert_same(out2, ref2)


def test_metadata_only(sv):
    say("case: expand without hidden rows")
    e = workloads.expand_inputs(B=64, K=4, H=8, seed=3, device="cuda")
    out, ref = run_both(sv, e, with_hidden=False)
    assert out.out_hidden is None
    assert_same(out, ref, with_hidden=False)


def test_invalid_requests(sv):
    say("case: expand invalid data")
    e = workloads.expand_inputs(B=6, K=3, H=16, seed=9, device="cuda")
    acc = e.accepted.clone()
    acc[2] = 4   # n = 4: a must be <= 3
    acc[4] = -1
    out, ref = run_both(sv, e, accepted=acc)
    assert ref.n_bad == 2
    assert_same(out, ref)
    # an empty request (n_b = 0)
    st = torch.tensor([0, 4, 4, 8, 12, 16, 24], dtype=torch.int32, device="cuda")
    out, ref = run_both(sv, e, in_start=st, accepted=torch.tensor([1, 0, 2, 3, 0, 7], dtype=torch.int32,
                                                                  device="cuda"))
    assert ref.n_bad == 1
    assert_same(out, ref)
    # start indices not covering the input: every request invalid
    st = e.in_start.clone()
    st[-1] -= 1
    out, ref = run_both(sv, e, in_start=st)
    assert ref.n_bad == 6
    assert (out.new_token_indices.cpu().numpy() == -1).all()


def test_chained_after_verify(sv):
    """The bonus read straight from a verification's output tokens."""
    say("case: verify -> expand chained")
    vin = workloads.verify_tiny(seed=2, device="cuda")
    acc, tok, _ = sv.verify(vin.target, vin.draft, vin.draft_tokens, vin.temperature, seed=4)
    B, K = vin.B, vin.K
    e = workloads.expand_inputs(B=B, K=K, H=64, seed=2, device="cuda", accepted=acc.cpu())
    out = sv.expand(e.in_token_ids, e.in_positions, e.in_start, acc, None, K, e.mask_id, e.target_hidden,
                    e.mask_hidden, verify_tokens=tok)
    torch.cuda.synchronize()
    a = acc.cpu().numpy()
    bonus = tok.cpu().numpy()[np.arange(B), a]
    ref = oracle.expand(e.in_token_ids.cpu().numpy(), e.in_positions.cpu().numpy(), e.in_start.cpu().numpy(),
                        a, bonus, K, e.mask_id, workloads.bf16_bits(e.target_hidden),
                        workloads.bf16_bits(e.mask_hidden))
    assert_same(out, ref)


@pytest.mark.parametrize("phase_starts", [0b100100, 1])
def test_chained_step_graph_capture(sv, phase_starts):
    """verify (early-exit phases, or the dynamic exit) -> expand (bonus from the verify tokens, KV
    slot mapping) chained on one stream with no host round trip, captured
    into a HIP graph and replayed: every replay, with eager work and a reset
    of the outputs between replays, must reproduce the eager outputs."""
    say("case: chained verify -> expand, graph capture")
    dev = torch.device("cuda")
    vin = workloads.mixture_inputs("chain B64 K8 V32768", 64, 8, 32768, torch.bfloat16, 12, dev,
                                   temps=(0.0, 0.6, 1.0), lam_lo=0.05, lam_hi=0.6)
    B, K, V = vin.B, vin.K, vin.V
    e = workloads.expand_inputs(B=B, K=K, H=256, seed=12, device="cuda")
    bt = table_for(e, 16, seed=12)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ws = sv.make_workspace(B, K, V, dev)
    out = sv.expand_outputs(B, K, e.N_in, e.H, dev, with_slots=True)
    va = sv.verify_args(vin.target, vin.draft, vin.draft_tokens, vin.temperature, acc, tok, None, ws,
                        seed=21, step=3, phase_starts=phase_starts)
    xa = sv.expand_args(e.in_token_ids, e.in_positions, e.in_start, acc, None, K, e.mask_id, e.target_hidden,
                        e.mask_hidden, out, verify_tokens=tok, block_table=bt, block_size=16)

    def step(stream):
        assert sv.spec_verify_launch(va, stream.cuda_stream) == sv.SPEC_OK
        assert sv.spec_expand_launch(xa, stream.cuda_stream) == sv.SPEC_OK

    names = ("out_token_ids", "out_positions", "rejected_mask", "masked_mask", "new_token_indices",
             "hidden_map", "out_start", "out_hidden", "slot_mapping")

    def snapshot():
        return [acc.clone(), tok.clone()] + [getattr(out, n).clone() for n in names]

    def reset():
        acc.fill_(-5)
        tok.fill_(-5)
        for n in names:
            getattr(out, n).zero_()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = snapshot()
    # the chained outputs against the oracle: the bonus is the verify's token at a
    a = acc.cpu().numpy()
    bonus = tok.cpu().numpy()[np.arange(B), a]
    ref = oracle.expand(e.in_token_ids.cpu().numpy(), e.in_positions.cpu().numpy(), e.in_start.cpu().numpy(),
                        a, bonus, K, e.mask_id, workloads.bf16_bits(e.target_hidden),
                        workloads.bf16_bits(e.mask_hidden), block_table=bt.cpu().numpy(), block_size=16)
    assert_same(out, ref)

    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step(torch.cuda.current_stream())
    for rep in range(4):
        x = torch.randn(1 << 20, device=dev)
        float(x.sum())  # eager work and a synchronisation between replays
        reset()
        g.replay()
        torch.cuda.synchronize()
        for i, (u, v) in enumerate(zip(snapshot(), eager)):
            assert torch.equal(u, v), (rep, i)
    say("  %d replays identical to the eager step" % 4)


def test_hidden_gather_apart_on_a_second_stream(sv):
    """The hidden rows gathered alone (spec_expand_hidden_launch) on a second
    stream while the verification runs, then the metadata on the first:
    the same bits as the fused expansion after the verification."""
    say("case: expand hidden rows on a second stream")
    dev = torch.device("cuda")
    vin = workloads.mixture_inputs("overlap B64 K8 V32768", 64, 8, 32768, torch.bfloat16, 15, dev,
                                   temps=(0.0, 1.0), lam_lo=0.05, lam_hi=0.6)
    B, K = vin.B, vin.K
    e = workloads.expand_inputs(B=B, K=K, H=2880, seed=15, device="cuda")
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ws = sv.make_workspace(B, K, vin.V, dev)
    ev = torch.cuda.Event()
    ev.record()  # create the event
    va = sv.verify_args(vin.target, vin.draft, vin.draft_tokens, vin.temperature, acc, tok, None, ws, seed=5,
                        phase_event=ev.cuda_event, phase_starts=0b100100)
    fused = sv.expand_outputs(B, K, e.N_in, e.H, dev)
    split = sv.expand_outputs(B, K, e.N_in, e.H, dev)
    for o in (fused, split):
        o.out_hidden.fill_(7)
    xf = sv.expand_args(e.in_token_ids, e.in_positions, e.in_start, acc, None, K, e.mask_id, e.target_hidden,
                        e.mask_hidden, fused, verify_tokens=tok)
    xs = sv.expand_args(e.in_token_ids, e.in_positions, e.in_start, acc, None, K, e.mask_id, e.target_hidden,
                        e.mask_hidden, split, verify_tokens=tok)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    assert sv.spec_verify_launch(va, main.cuda_stream) == sv.SPEC_OK
    side.wait_event(ev)  # after the row statistics: overlaps the sampling stage
    assert sv.spec_expand_hidden_launch(xs, side.cuda_stream) == sv.SPEC_OK
    meta = sv.expand_args(e.in_token_ids, e.in_positions, e.in_start, acc, None, K, e.mask_id, e.target_hidden,
                          e.mask_hidden, sv.ExpandOutputs(**{**split.__dict__, "out_hidden": None}),
                          verify_tokens=tok)
    assert sv.spec_expand_launch(meta, main.cuda_stream) == sv.SPEC_OK
    main.wait_stream(side)
    assert sv.spec_expand_launch(xf, main.cuda_stream) == sv.SPEC_OK
    torch.cuda.synchronize()
    for name in ("out_token_ids", "out_positions", "rejected_mask", "masked_mask", "new_token_indices",
                 "hidden_map", "out_start", "out_hidden"):
        assert torch.equal(getattr(fused, name), getattr(split, name)), name


EXPAND_NAMES = ("out_token_ids", "out_positions", "rejected_mask", "masked_mask", "new_token_indices",
                "hidden_map", "out_start", "out_hidden", "slot_mapping")


def _chained_case(sv, name, B, K, V, H, seed, temps, phase_starts, spoil=None, num_drafts=None, strided=False,
                  dtype=torch.bfloat16):
    """spec_verify_expand_launch against spec_verify_launch followed by
    spec_expand_launch on the same inputs: every output bit for bit."""
    dev = torch.device("cuda")
    vin = workloads.mixture_inputs(name, B, K, V, dtype, seed, dev, temps=temps, lam_lo=0.05, lam_hi=0.6)
    x = vin.draft_tokens.clone()
    if spoil is not None:
        spoil(x)
    e = workloads.expand_inputs(B=B, K=K, H=H, seed=seed, device="cuda")
    hidden = e.target_hidden
    if strided:  # a row stride wider than H
        wide = torch.zeros(e.N_in, H + 8, dtype=torch.bfloat16, device=dev)
        wide[:, :H] = hidden
        hidden = wide[:, :H]
    bt = table_for(e, 16, seed=seed, unmapped_fraction=0.1)
    res = []
    for fused in (False, True):
        acc = torch.full((B,), -7, dtype=torch.int32, device=dev)
        tok = torch.full((B, K + 1), -7, dtype=torch.int32, device=dev)
        ws = sv.make_workspace(B, K, V, dev)
        out = sv.expand_outputs(B, K, e.N_in, H, dev, with_slots=True)
        for n in EXPAND_NAMES:
            getattr(out, n).fill_(3)
        va = sv.verify_args(vin.target, vin.draft, x, vin.temperature, acc, tok, None, ws, seed=seed, step=2,
                            phase_starts=phase_starts, num_drafts=num_drafts)
        xa = sv.expand_args(e.in_token_ids, e.in_positions, e.in_start, acc, None, K, e.mask_id, hidden,
                            e.mask_hidden, out, verify_tokens=tok, block_table=bt, block_size=16)
        st = torch.cuda.current_stream().cuda_stream
        if fused:
            assert sv.spec_verify_expand_launch(va, xa, st) == sv.SPEC_OK
        else:
            assert sv.spec_verify_launch(va, st) == sv.SPEC_OK
            assert sv.spec_expand_launch(xa, st) == sv.SPEC_OK
        torch.cuda.synchronize()
        res.append([acc, tok] + [getattr(out, n) for n in EXPAND_NAMES])
    for i, (u, v) in enumerate(zip(*res)):
        assert torch.equal(u, v), (name, i)
    return res[1]


def test_verify_expand_chained_call(sv):
    say("case: spec_verify_expand_launch == verify then expand")
    # one pass and early-exit phases, greedy and sampled requests, the KV
    # slot mapping with unmapped blocks, headline-sized rows
    _chained_case(sv, "chain one pass", 48, 8, 151936, 2880, 31, (0.0, 0.6, 1.0), 0)
    _chained_case(sv, "chain phased", 48, 8, 151936, 2880, 32, (0.0, 0.6, 1.0), 0b100100)
    # the benchmarked step: B=256, K=8, V=151936, H=2880, phases {0..2 | 3..8}
    _chained_case(sv, "chain headline", 256, 8, 151936, 2880, 38, (0.0, 0.6, 1.0), 0b1000)
    # all sampled (every bonus id comes from the draw), all greedy
    _chained_case(sv, "chain sampled", 16, 5, 32768, 256, 33, (1.0,), 0b1000)
    _chained_case(sv, "chain greedy", 16, 5, 32768, 256, 34, (0.0,), 0)
    # invalid draft tokens: accepted -1, the expansion marks the request invalid
    def spoil(x):
        x[1, 0] = -3
        x[4, 2] = 1 << 20
    acc = _chained_case(sv, "chain invalid", 8, 4, 4096, 64, 35, (0.0, 1.0), 0, spoil=spoil)[0]
    assert acc[1].item() == -1 and acc[4].item() == -1
    # ragged draft counts, a strided hidden tensor (scalar copy path), an odd H
    nd = torch.tensor([4, 0, 2, 4, 1, 3, 4, 2], dtype=torch.int32, device="cuda")
    _chained_case(sv, "chain ragged", 8, 4, 4096, 64, 36, (0.0, 1.0), 0b100, num_drafts=nd, strided=True)
    _chained_case(sv, "chain odd H", 8, 4, 4096, 61, 37, (1.0,), 0)
    # fp32 logits (the 4-byte segment-sum kernel with the expansion appended)
    _chained_case(sv, "chain fp32", 12, 5, 10000, 128, 39, (0.0, 0.7, 1.0), 0b100, dtype=torch.float32)
    # K = 63 (windows of n_b + 62 slots) with an irregular cut
    _chained_case(sv, "chain K63", 6, 63, 4096, 64, 40, (0.0, 1.0), (1 << 10) | (1 << 40))


def test_verify_expand_chained_call_graph_capture(sv):
    say("case: spec_verify_expand_launch captured in a graph")
    dev = torch.device("cuda")
    B, K, V, H = 32, 8, 32768, 256
    vin = workloads.mixture_inputs("chain graph", B, K, V, torch.bfloat16, 41, dev, temps=(0.0, 0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.6)
    e = workloads.expand_inputs(B=B, K=K, H=H, seed=41, device="cuda")
    bt = table_for(e, 16, seed=41)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ws = sv.make_workspace(B, K, V, dev)
    out = sv.expand_outputs(B, K, e.N_in, H, dev, with_slots=True)
    va = sv.verify_args(vin.target, vin.draft, vin.draft_tokens, vin.temperature, acc, tok, None, ws, seed=9,
                        step=1, phase_starts=0b100100)
    xa = sv.expand_args(e.in_token_ids, e.in_positions, e.in_start, acc, None, K, e.mask_id, e.target_hidden,
                        e.mask_hidden, out, verify_tokens=tok, block_table=bt, block_size=16)

    def snapshot():
        return [acc.clone(), tok.clone()] + [getattr(out, n).clone() for n in EXPAND_NAMES]

    def reset():
        acc.fill_(-5)
        tok.fill_(-5)
        for n in EXPAND_NAMES:
            getattr(out, n).zero_()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        assert sv.spec_verify_expand_launch(va, xa, s.cuda_stream) == sv.SPEC_OK
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = snapshot()
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        assert sv.spec_verify_expand_launch(va, xa, torch.cuda.current_stream().cuda_stream) == sv.SPEC_OK
    for rep in range(3):
        x = torch.randn(1 << 20, device=dev)
        float(x.sum())
        reset()
        g.replay()
        torch.cuda.synchronize()
        for i, (u, v) in enumerate(zip(snapshot(), eager)):
            assert torch.equal(u, v), (rep, i)


@pytest.mark.parametrize("iseed", [0, 5])
def test_benchmarked_call_against_oracle(sv, iseed):
    """The benchmarked step at its own shape: one spec_verify_expand_launch
    over the headline batch (B=256, K=8, V=151936 bf16, T in {0, 0.6, 1},
    mixture drafts) and its expansion (H=2880, the bonus read from the
    verification's tokens, KV slot mapping through a 16-slot block table),
    rows read in the early-exit phases {0..2 | 3..8}; checked against
    oracle.verify followed by oracle.expand on the oracle's own outputs:
    every request, every expansion array and every hidden row."""
    from parity import Report, compare
    dev = torch.device("cuda")
    inp = workloads.verify_headline(seed=iseed, device=dev)
    e = workloads.step_expand_inputs(inp, seed=iseed)
    B, K, V, H = inp.B, inp.K, inp.V, e.H
    tl, dl = workloads.logits_numpy(inp.target), workloads.logits_numpy(inp.draft)
    x, T = inp.draft_tokens.cpu().numpy(), inp.temperature.cpu().numpy()
    hid, mhid = workloads.bf16_bits(e.target_hidden), workloads.bf16_bits(e.mask_hidden)
    host = {n: getattr(e, n).cpu().numpy() for n in ("in_token_ids", "in_positions", "in_start", "block_table")}
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ws = sv.make_workspace(B, K, V, dev)
    out = sv.expand_outputs(B, K, e.N_in, H, dev, with_slots=True)
    for seed, step in ((iseed, 0), ((1 << 40) + iseed, 77)):
        say("case: benchmarked call B256 K8 V151936 H2880, inputs %d, seed %d step %d" % (iseed, seed, step))
        for n in EXPAND_NAMES:
            getattr(out, n).fill_(3)
        va = sv.verify_args(inp.target, inp.draft, inp.draft_tokens, inp.temperature, acc, tok, None, ws,
                            seed=seed, step=step, phase_starts=0b1000)
        xa = sv.expand_args(e.in_token_ids, e.in_positions, e.in_start, acc, None, K, e.mask_id, e.target_hidden,
                            e.mask_hidden, out, verify_tokens=tok, block_table=e.block_table,
                            block_size=e.block_size)
        assert sv.spec_verify_expand_launch(va, xa, torch.cuda.current_stream().cuda_stream) == sv.SPEC_OK
        torch.cuda.synchronize()
        a_g, t_g = acc.cpu().numpy(), tok.cpu().numpy()
        rep = compare(tl, dl, x, T, a_g, t_g, None, seed=seed, step=step, report=Report())
        say("  verification:", rep.summary())
        assert rep.ok(), rep.failures[:5]
        res = oracle.verify(tl, dl, x, T, seed=seed, step=step, debug=False, trace=False)
        a_o = res.accepted
        ref = oracle.expand(host["in_token_ids"], host["in_positions"], host["in_start"], a_o,
                            res.tokens[np.arange(B), a_o], K, e.mask_id, hid, mhid,
                            block_table=host["block_table"], block_size=e.block_size)
        # requests whose verification differs only at a counted near-threshold
        # decision legitimately expand differently: leave their windows out
        same = (a_g == a_o) & (t_g == res.tokens).all(axis=1)
        win = 2 * K  # every window holds n_b + K - 1 = 2K slots
        slot_ok = np.repeat(same, win)
        in_ok = np.repeat(same, K + 1)
        for n in EXPAND_NAMES:
            g = getattr(out, n)
            g = workloads.bf16_bits(g) if n == "out_hidden" else g.cpu().numpy()
            r = getattr(ref, n)
            if n == "new_token_indices":
                g, r = g[same], r[same]
            elif n == "hidden_map":
                g, r = g[in_ok], r[in_ok]
            elif n != "out_start":
                g, r = g[slot_ok], r[slot_ok]
            assert np.array_equal(g, r), (n, iseed, seed, step)
        say("  expansion: every array bit-exact on %d of %d windows" % (int(same.sum()), B))
        assert same.sum() >= B - len(rep.near)
