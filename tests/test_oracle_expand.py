"""Pins of the oracle's P-EAGLE drafter-batch expansion and hidden fill.

"P-EAGLE: parallel speculative decoding in vLLM" page: section "Triton Kernel"
lists what one pass produces (shifted copy of ids and positions, the bonus
token, MASK-filled parallel-drafting slots, rejected-token mask, masked-token
mask, new-token indices, hidden-state mapping); section "Hidden State 管理"
says how the hidden rows are filled (target rows to their mapped slots, then
the MASK slots take a shared placeholder row); section "并行草稿生成的挑战"
says positions advance per request and start indices are recomputed.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _run(inp, with_hidden=True, block_table=None, block_size=0):
    return oracle.expand(
        inp.in_token_ids.numpy(), inp.in_positions.numpy(), inp.in_start.numpy(),
        inp.accepted.numpy(), inp.bonus.numpy(), inp.K, inp.mask_id,
        workloads.bf16_bits(inp.target_hidden) if with_hidden else None,
        workloads.bf16_bits(inp.mask_hidden) if with_hidden else None,
        block_table=None if block_table is None else block_table.numpy(), block_size=block_size)


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "expand_worked_example.json")) as f:
        ex = json.load(f)
    r = oracle.expand(ex["in_token_ids"], ex["in_positions"], ex["in_start"], ex["accepted"],
                      ex["bonus"], ex["K"], ex["mask_id"], block_table=ex["block_table"],
                      block_size=ex["block_size"])
    e = ex["expected"]
    assert r.n_bad == 0
    for key in ("out_start", "out_token_ids", "out_positions", "rejected_mask", "masked_mask",
                "hidden_map", "slot_mapping"):
        assert list(getattr(r, key)) == e[key], key
    assert r.new_token_indices.tolist() == e["new_token_indices"]
    # without a block table nothing else changes
    r2 = oracle.expand(ex["in_token_ids"], ex["in_positions"], ex["in_start"], ex["accepted"],
                       ex["bonus"], ex["K"], ex["mask_id"])
    assert r2.slot_mapping is None and list(r2.out_token_ids) == e["out_token_ids"]


def test_hand_worked_slot_edge_cases():
    """Positions past the block table or in a block marked -1 get no slot."""
    with open(os.path.join(GOLDEN, "expand_worked_example.json")) as f:
        cases = json.load(f)["slot_edge_cases"]
    for c in cases:
        r = oracle.expand(c["in_token_ids"], c["in_positions"], c["in_start"], c["accepted"], c["bonus"],
                          c["K"], c["mask_id"], block_table=c["block_table"], block_size=c["block_size"])
        assert list(r.slot_mapping) == c["expected_slot_mapping"], c["why"]


@pytest.mark.parametrize("block_size", [1, 16])
def test_slot_mapping_invariants(block_size):
    """Rejected slots and only they get -1 when every position has a block;
    every other slot lies in the block the table gives for its position, at
    the position's offset, and no two slots of the batch share a cache slot
    unless they share a request and a position."""
    inp = workloads.expand_inputs(B=64, K=6, H=8, seed=5, max_offset=300)
    max_blocks = (300 + 2 * 6 + 2) // block_size + 1
    bt = workloads.block_tables(64, max_blocks, seed=6)
    r = _run(inp, with_hidden=False, block_table=bt, block_size=block_size)
    sm = r.slot_mapping
    rej = r.rejected_mask.astype(bool)
    assert ((sm == -1) == rej).all()
    btn = bt.numpy()
    owner = np.repeat(np.arange(64), np.diff(r.out_start))
    pos = r.out_positions
    v = ~rej
    np.testing.assert_array_equal(sm[v] // block_size, btn[owner[v], pos[v] // block_size])
    np.testing.assert_array_equal(sm[v] % block_size, pos[v] % block_size)
    keys = set()
    for s_, b_, p_ in zip(sm[v], owner[v], pos[v]):
        keys.add((int(s_), int(b_), int(p_)))
    assert len({k[0] for k in keys}) == len({(k[1], k[2]) for k in keys})
    # blocks marked -1 leave their positions without a slot, and nothing else changes
    bt2 = workloads.block_tables(64, max_blocks, seed=6, unmapped_fraction=0.3)
    r2 = _run(inp, with_hidden=False, block_table=bt2, block_size=block_size)
    blk = pos // block_size
    hole = bt2.numpy()[owner, blk] != btn[owner, blk]
    np.testing.assert_array_equal(r2.slot_mapping[hole], -1)
    np.testing.assert_array_equal(r2.slot_mapping[~hole], sm[~hole])


def check_invariants(inp, r):
    """Facts fixed by the page, independent of the slot order inside a window."""
    B, K = inp.B, inp.K
    st = inp.in_start.numpy().astype(np.int64)
    n = np.diff(st)
    acc = inp.accepted.numpy()
    N_out = inp.N_in + B * (K - 1)
    # start indices: exclusive scan of the expanded request sizes n_b + K - 1
    want_start = np.concatenate([[0], np.cumsum(n + K - 1)])
    np.testing.assert_array_equal(r.out_start, want_start)
    masked = r.masked_mask.astype(bool)
    rejected = r.rejected_mask.astype(bool)
    assert set(np.unique(r.masked_mask)) <= {0, 1} and set(np.unique(r.rejected_mask)) <= {0, 1}
    assert not (masked & rejected).any()
    # the mapping is injective, and its image with the masked slots partitions the output
    hm = r.hidden_map
    assert len(np.unique(hm)) == inp.N_in
    cover = np.zeros(N_out, np.int64)
    np.add.at(cover, hm, 1)
    cover[masked] += 1
    assert (cover == 1).all()
    ids = inp.in_token_ids.numpy()
    pos = inp.in_positions.numpy()
    bonus = inp.bonus.numpy()
    for b in range(B):
        o0, o1 = r.out_start[b], r.out_start[b + 1]
        sl = slice(o0, o1)
        valid = ~masked[sl] & ~rejected[sl]
        # per request: a+1 valid (accepted drafts + bonus), n-1-a rejected, K-1 MASK
        assert valid.sum() == acc[b] + 1
        assert rejected[sl].sum() == n[b] - 1 - acc[b]
        assert masked[sl].sum() == K - 1
        assert (r.out_token_ids[sl][masked[sl]] == inp.mask_id).all()
        # every input row of the request maps into its own window
        assert ((hm[st[b]:st[b + 1]] >= o0) & (hm[st[b]:st[b + 1]] < o1)).all()
        # drafter inputs: the slot holding input hidden row j carries position pos_j + 1
        np.testing.assert_array_equal(r.out_positions[hm[st[b]:st[b + 1]]], pos[st[b]:st[b + 1]] + 1)
        # valid + MASK slots have strictly increasing, consecutive positions
        keep = valid | masked[sl]
        vp = r.out_positions[sl][keep]
        assert (np.diff(vp) == 1).all()
        assert vp[0] == pos[st[b]] + 1
        # the valid tokens are the accepted drafts followed by the bonus
        vt = r.out_token_ids[sl][valid]
        assert list(vt[:-1]) == list(ids[st[b] + 1:st[b] + 1 + acc[b]])
        assert vt[-1] == bonus[b]
        # new-token indices: the bonus slot then the K-1 MASK slots
        nti = r.new_token_indices[b]
        assert r.out_token_ids[nti[0]] == bonus[b] and valid[nti[0] - o0]
        assert masked[nti[1:]].all() and (np.diff(nti) > 0).all()


@pytest.mark.parametrize("seed", [0, 1])
def test_invariants_at_full_size(seed):
    inp = workloads.expand_inputs(B=512, K=8, H=64, seed=seed)
    r = _run(inp, with_hidden=False)
    assert r.n_bad == 0
    check_invariants(inp, r)


def test_invariants_ragged_requests():
    rng = np.random.default_rng(3)
    n = rng.integers(1, 12, 97)
    inp = workloads.expand_inputs(B=97, K=5, H=16, seed=3, n_per_request=n)
    r = _run(inp, with_hidden=False)
    assert r.n_bad == 0
    check_invariants(inp, r)


@pytest.mark.parametrize("K", [1, 2, 8])
def test_hidden_fill_follows_the_page(K):
    """The hidden-state fill as the P-EAGLE page's section "Hidden State 管理"
    describes it, written out row by row on the CPU: every input row i goes to
    output row hidden_map[i], then every output row flagged as a MASK slot
    takes the shared placeholder row instead.  The oracle's hidden rows equal
    that bit for bit, and every output row is written (none keeps the NaN it
    started with)."""
    inp = workloads.expand_inputs(B=37, K=K, H=48, seed=K)
    r = _run(inp)
    src = workloads.bf16_bits(inp.target_hidden)
    placeholder = workloads.bf16_bits(inp.mask_hidden)
    nan_bits = np.uint16(0x7FC0)  # a bf16 NaN: marks rows nobody wrote
    want = np.full((inp.N_out, inp.H), nan_bits, np.uint16)
    for i in range(inp.N_in):
        want[int(r.hidden_map[i])] = src[i]
    for row in range(inp.N_out):
        if r.masked_mask[row]:
            want[row] = placeholder
    np.testing.assert_array_equal(r.out_hidden, want)
    assert not (want == nan_bits).all(axis=1).any()


def test_invalid_requests_write_nothing():
    inp = workloads.expand_inputs(B=4, K=3, H=8, seed=9)
    acc = inp.accepted.clone()
    acc[2] = 4  # n = 4 => a must be <= 3
    r = oracle.expand(inp.in_token_ids.numpy(), inp.in_positions.numpy(), inp.in_start.numpy(),
                      acc.numpy(), inp.bonus.numpy(), 3, inp.mask_id)
    assert r.n_bad == 1
    o0, o1 = r.out_start[2], r.out_start[3]
    assert (r.out_token_ids[o0:o1] == -7).all()
    assert (r.new_token_indices[2] == -1).all()
    assert (r.new_token_indices[[0, 1, 3]] >= 0).all()
    # an empty request (n_b = 0) is invalid, its neighbours are not
    st = np.array([0, 4, 4, 8, 12], np.int32)
    r = oracle.expand(inp.in_token_ids.numpy()[:12], inp.in_positions.numpy()[:12], st,
                      [1, 0, 2, 3], inp.bonus.numpy(), 3, inp.mask_id)
    assert r.n_bad == 1 and (r.new_token_indices[1] == -1).all()
    assert (r.new_token_indices[[0, 2, 3]] >= 0).all()
    # start indices that do not cover the input rows invalidate every request
    st = inp.in_start.numpy().copy()
    st[-1] -= 1  # in_start[B] != N_in
    r = oracle.expand(inp.in_token_ids.numpy(), inp.in_positions.numpy(), st, inp.accepted.numpy(),
                      inp.bonus.numpy(), 3, inp.mask_id)
    assert r.n_bad == 4 and (r.new_token_indices == -1).all() and (r.out_start == -7).all()
