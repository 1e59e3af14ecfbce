"""Ragged per-request draft counts K_b <= K on the GPU through the C ABI,
against the CPU oracle (bar of ``parity.py``), in one pass and in early-exit
phases.  Tokens past K_b are set to garbage: they must never be read."""
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


def ragged(inp, seed, lo=0):
    rng = np.random.default_rng(seed)
    kb = rng.integers(lo, inp.K + 1, inp.B).astype(np.int32)
    x = inp.draft_tokens.clone()
    for b in range(inp.B):
        x[b, kb[b]:] = -5
    return torch.from_numpy(kb).cuda(), x


def check(sv, inp, kb, x, seed, step, mask, idx=None):
    acc, tok, dbg = sv.verify(inp.target, inp.draft, x, inp.temperature, seed=seed, step=step, debug=True,
                              phase_starts=mask, num_drafts=kb)
    torch.cuda.synchronize()
    acc, tok, dbg = acc.cpu().numpy(), tok.cpu().numpy(), dbg.cpu().numpy()
    kbh = kb.cpu().numpy()
    assert (acc >= 0).all() and (acc <= kbh).all()
    rep = Report()
    rows = range(inp.B) if idx is None else idx
    for b in rows:
        compare(workloads.logits_numpy(inp.target[b:b + 1]), workloads.logits_numpy(inp.draft[b:b + 1]),
                x[b:b + 1].cpu().numpy(), inp.temperature[b:b + 1].cpu().numpy(), acc[b:b + 1], tok[b:b + 1],
                dbg[b:b + 1] if mask == 0 else None, seed=seed, step=step, request_base=int(b), report=rep,
                num_drafts=kbh[b:b + 1])
    say("  mask %s: %s" % (bin(mask), rep.summary()))
    assert rep.ok(), rep.failures[:5]
    return acc, tok


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 70001), (torch.float32, 20003)])
def test_ragged_parity(sv, dtype, V):
    say("case: ragged K B16 K6 V%d %s" % (V, dtype))
    inp = workloads.mixture_inputs("ragged B16 K6 V%d" % V, 16, 6, V, dtype, 7, "cuda",
                                   temps=(0.0, 0.6, 1.0), lam_lo=0.05, lam_hi=0.5)
    kb, x = ragged(inp, 7)
    for mask in (0, 0b0010100, 0b1111110, sv.SPEC_PHASES_DYNAMIC):
        for step in range(2):
            check(sv, inp, kb, x, 4, step, mask)


def test_full_counts_equal_no_table(sv):
    say("case: ragged K with every K_b = K")
    inp = workloads.mixture_inputs("full", 12, 5, 33000, torch.bfloat16, 2, "cuda", temps=(0.0, 1.0),
                                   lam_lo=0.1, lam_hi=0.5)
    full = torch.full((12,), 5, dtype=torch.int32, device="cuda")
    for mask in (0, 0b100100, sv.SPEC_PHASES_DYNAMIC):
        a = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=1, debug=True,
                      phase_starts=mask)
        b = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=1, debug=True,
                      phase_starts=mask, num_drafts=full)
        for u, v in zip(a, b):
            assert torch.equal(u, v)


def test_invalid_counts(sv):
    say("case: ragged K invalid counts")
    inp = workloads.mixture_inputs("bad", 6, 4, 5000, torch.float32, 3, "cuda", temps=(0.0, 1.0),
                                   lam_lo=0.1, lam_hi=0.5)
    kb = torch.tensor([-1, 5, 0, 4, 2, 1], dtype=torch.int32, device="cuda")
    for mask in (0, 0b00110, sv.SPEC_PHASES_DYNAMIC):
        acc, tok, _ = sv.verify(inp.target, inp.draft, inp.draft_tokens, inp.temperature, seed=2,
                                phase_starts=mask, num_drafts=kb)
        acc, tok = acc.cpu().numpy(), tok.cpu().numpy()
        assert acc[0] == -1 and acc[1] == -1 and (tok[:2] == -1).all()
        assert acc[2] == 0 and (tok[2, 1:] == -1).all() and tok[2, 0] >= 0
        assert (acc[2:] >= 0).all()


def test_headline_ragged_planned(sv):
    """B=256, K=8, V=151936 bf16 with K_b uniform in 0..8, in one pass, with
    an early-exit plan and with the dynamic exit; 24 requests against the
    oracle."""
    say("case: ragged K headline B256 K8 V151936")
    inp = workloads.verify_headline(seed=1, device="cuda")
    kb, x = ragged(inp, 11)
    rng = np.random.default_rng(3)
    idx = sorted(rng.choice(inp.B, 24, replace=False))
    a1, t1 = check(sv, inp, kb, x, 0, 0, 0, idx)
    a2, t2 = check(sv, inp, kb, x, 0, 0, 0b100100, idx)
    assert np.array_equal(a1, a2) and np.array_equal(t1, t2)
    a3, t3 = check(sv, inp, kb, x, 0, 0, sv.SPEC_PHASES_DYNAMIC, idx)
    assert np.array_equal(a1, a3) and np.array_equal(t1, t3)
