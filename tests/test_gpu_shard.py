"""Vocab-sharded verification on one GPU (every stage of every shard through
the C ABI, the exchanges through shared arrays) against the CPU oracle (bar
of ``parity.py``) and against the unsharded launch: every shard must take
the same decisions, and the results may differ from the unsharded ones only
where a decision sits within rounding of its threshold."""
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


def check(sv, inp, G, seed, step, bounds=None, idx=None):
    acc, tok, per = sv.verify_sharded(inp.target, inp.draft, inp.draft_tokens, inp.temperature, G, seed=seed,
                                      step=step, bounds=bounds)
    torch.cuda.synchronize()
    per = per.cpu().numpy()
    assert (per == per[0]).all(), "shards disagree on the accepted counts"
    acc, tok = acc.cpu().numpy(), tok.cpu().numpy()
    rep = Report()
    rows = range(inp.B) if idx is None else idx
    for b in rows:
        compare(workloads.logits_numpy(inp.target[b:b + 1]), workloads.logits_numpy(inp.draft[b:b + 1]),
                inp.draft_tokens[b:b + 1].cpu().numpy(), inp.temperature[b:b + 1].cpu().numpy(), acc[b:b + 1],
                tok[b:b + 1], None, seed=seed, step=step, request_base=int(b), report=rep)
    say("  G=%d: %s" % (G, rep.summary()))
    assert rep.ok(), rep.failures[:5]
    a1, t1, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=seed, step=step)
    same = (a1.cpu().numpy() == acc) & (t1.cpu().numpy() == tok).all(axis=1)
    return int(same.sum())


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8])
def test_sharded_parity(sv, G):
    say("case: vocab-sharded verify G=%d, B12 K5 V70001 bf16 mixed T" % G)
    inp = workloads.mixture_inputs("shard", 12, 5, 70001, torch.bfloat16, 9, "cuda", temps=(0.0, 0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.6)
    for step in range(3):
        same = check(sv, inp, G, 2, step)
        say("    %d of 12 requests identical to the unsharded launch" % same)


def test_uneven_slices_and_fp32(sv):
    say("case: vocab-sharded verify, uneven slices, fp32")
    inp = workloads.mixture_inputs("shard fp32", 8, 4, 33000, torch.float32, 4, "cuda", temps=(0.0, 1.0),
                                   lam_lo=0.1, lam_hi=0.5)
    for bounds in ([0, 1, 33000], [0, 4096, 4100, 20000, 33000], [0, 32999, 33000]):
        check(sv, inp, len(bounds) - 1, 5, 0, bounds=bounds)


def test_invalid_requests(sv):
    say("case: vocab-sharded verify, invalid data")
    inp = workloads.noisy_draft_inputs("bad", 5, 3, 300, torch.float32, 2, "cuda", "gauss")
    x = inp.draft_tokens.clone()
    T = inp.temperature.clone()
    x[1, 2] = 300
    T[2] = float("nan")
    T[3] = -1.0
    acc, tok, per = sv.verify_sharded(inp.target, inp.draft, x, T, 3)
    acc, tok = acc.cpu().numpy(), tok.cpu().numpy()
    assert acc[0] >= 0 and acc[4] >= 0
    for b in (1, 2, 3):
        assert acc[b] == -1 and (tok[b] == -1).all()


def test_headline_sharded_tp4(sv):
    """B=256, K=8, V=151936 bf16 over 4 shards (a TP = 4 target): 24 requests
    against the oracle, and the share identical to the unsharded launch."""
    say("case: vocab-sharded verify, headline over 4 shards")
    inp = workloads.verify_headline(seed=2, device="cuda")
    rng = np.random.default_rng(4)
    idx = sorted(rng.choice(inp.B, 24, replace=False))
    check(sv, inp, 4, 0, 0, idx=idx)
    acc, tok, _ = sv.verify_sharded(inp.target, inp.draft, inp.draft_tokens, inp.temperature, 4)
    a1, t1, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature)
    same = ((a1 == acc) & (t1 == tok).all(dim=1)).float().mean().item()
    say("  %.4f of requests identical to the unsharded launch" % same)
    assert same > 0.98
