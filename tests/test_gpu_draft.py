"""GPU draft-token sampling at the new-token indices through the C ABI
against the CPU oracle.

Bar: every draft token bit-exact, except a sampled one whose uniform lies
within WINDOW of the oracle's normalised CDF at a boundary between the two
tokens (counted, not failed); greedy positions and invalid inputs exact.
Then the output law through the GPU (chi-square) and the chained P-EAGLE
loop at full size: expansion -> sampling at its new-token indices.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import WINDOW
from stats_helpers import chi2_pvalue, softmax_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rejection_sampling_verify_03_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def compare_draft(logits, row_index, T, tok_g, seed=0, step=0, request_base=0):
    """Returns (exact, near, failures) of GPU tokens against the oracle on the
    same host inputs (logits: numpy, uint16 bf16 bits or float32)."""
    ref = oracle.draft_sample(logits, row_index, T, seed=seed, step=step, request_base=request_base)
    tok_g = np.asarray(tok_g)
    exact, near, fails = 0, [], []
    B, K = row_index.shape
    for b in range(B):
        for k in range(K):
            g, o = int(tok_g[b, k]), int(ref.tokens[b, k])
            if g == o:
                exact += 1
                continue
            if o < 0 or g < 0 or float(T[b]) == 0.0:
                fails.append((b, k, g, o))
                continue
            p = oracle.softmax(logits[row_index[b, k]], float(T[b]))
            F = np.cumsum(p) / p.sum()
            lo, hi = min(g, o), max(g, o)
            margin = float(np.min(np.abs(ref.trace[b, k] - F[lo:hi])))
            (near if margin < WINDOW else fails).append((b, k, g, o, margin))
    return exact, near, fails


def run_case(sv, inp, seed=0, step=0, request_base=0):
    tok = sv.draft_sample(inp.logits, inp.row_index, inp.temperature, seed=seed, step=step,
                          request_base=request_base)
    torch.cuda.synchronize()
    ex, near, fails = compare_draft(workloads.logits_numpy(inp.logits), inp.row_index.cpu().numpy(),
                                    inp.temperature.cpu().numpy(), tok.cpu().numpy(), seed, step, request_base)
    say("  %d exact, %d near-threshold, %d failures" % (ex, len(near), len(fails)))
    assert not fails, fails[:5]
    return tok


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 70001), (torch.float32, 33000),
                                     (torch.bfloat16, 4096 * 8 * 2 + 77)])
def test_parity_mixed_temperatures(sv, dtype, V):
    """Several 8-segment chunks per row, a ragged last segment, shared rows."""
    say("case: draft sampling B12 K5 N40 V%d %s" % (V, dtype))
    inp = workloads.drafter_inputs(12, 5, 40, V, dtype, seed=V % 97, device="cuda")
    for step in range(3):
        run_case(sv, inp, seed=11, step=step, request_base=5)


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 20003), (torch.float32, 1023), (torch.bfloat16, 9),
                                     (torch.float32, 1)])
def test_scalar_path_and_tiny_rows(sv, dtype, V):
    say("case: draft sampling scalar path V%d %s" % (V, dtype))
    inp = workloads.drafter_inputs(6, 4, 10, V, dtype, seed=V, device="cuda", temps=(0.0, 0.7, 1.3))
    run_case(sv, inp, seed=2, step=1)
    # rows inside a wider buffer (row stride > V)
    wide = torch.full((inp.N, V + 24), -30.0, dtype=dtype, device="cuda")
    wide[:, :V] = inp.logits
    tok_w = sv.draft_sample(wide[:, :V], inp.row_index, inp.temperature, seed=2, step=1)
    tok = sv.draft_sample(inp.logits, inp.row_index, inp.temperature, seed=2, step=1)
    assert torch.equal(tok, tok_w)


def test_invalid_inputs(sv):
    say("case: draft sampling invalid inputs")
    inp = workloads.drafter_inputs(5, 3, 6, 300, torch.float32, seed=4, device="cuda", temps=(1.0,))
    ri = inp.row_index.clone()
    T = inp.temperature.clone()
    lg = inp.logits.clone()
    ri[0, 1] = -1
    ri[0, 2] = 6
    T[1] = float("nan")
    T[2] = -1.0
    lg[5] = -float("inf")
    ri[3, :] = 5
    tok = sv.draft_sample(lg, ri, T, seed=3).cpu().numpy()
    ref = oracle.draft_sample(lg.cpu().numpy(), ri.cpu().numpy(), T.cpu().numpy(), seed=3)
    assert tok[0, 1] == -1 and tok[0, 2] == -1 and tok[0, 0] >= 0
    assert (tok[1] == -1).all() and (tok[2] == -1).all() and (tok[3] == -1).all()
    np.testing.assert_array_equal(tok, ref.tokens)
    # no rows at all
    empty = torch.empty(0, 300, dtype=torch.float32, device="cuda")
    tok = sv.draft_sample(empty, ri, inp.temperature).cpu().numpy()
    assert (tok == -1).all()


def test_output_law_through_the_gpu(sv):
    """300000 requests draw K = 3 positions from rows 0, 1, 2 of a V = 64
    table at T = 0.8: each position's tokens follow softmax(row / T)."""
    say("case: draft sampling chi-square through the GPU")
    rng = np.random.default_rng(8)
    lg = (1.5 * rng.standard_normal((3, 64))).astype(np.float32)
    B = 300_000
    ri = torch.arange(3, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    tok = sv.draft_sample(torch.from_numpy(lg).cuda(), ri, torch.full((B,), 0.8, device="cuda"),
                          seed=6).cpu().numpy()
    pv = [chi2_pvalue(np.bincount(tok[:, k], minlength=64), softmax_rows(lg[k], 0.8)) for k in range(3)]
    say("  p-values", pv)
    assert min(pv) >= 1e-4


def test_chained_after_expand_full_size(sv):
    """B=256, K=8, V=151936 bf16: an expansion of the headline batch shape,
    then the draft tokens sampled from drafter logits [N_out, V] at its
    new-token indices; 8 requests (64 positions) against the oracle and
    run-to-run bit-identical."""
    say("case: expand -> draft sampling, B256 K8 V151936")
    B, K, V = 256, 8, workloads.QWEN3_VOCAB
    e = workloads.expand_inputs(B=B, K=K, H=16, seed=3, device="cuda")
    out = sv.expand(e.in_token_ids, e.in_positions, e.in_start, e.accepted, e.bonus, K, e.mask_id)
    nti = out.new_token_indices
    g = workloads._gen(5, "cuda")
    logits = workloads.zipf_logits(e.N_out, V, g, "cuda").to(torch.bfloat16)
    T = torch.tensor([0.0, 0.6, 1.0], device="cuda")[torch.randint(0, 3, (B,), generator=g, device="cuda")]
    tok = sv.draft_sample(logits, nti, T, seed=9, step=4)
    tok2 = sv.draft_sample(logits, nti, T, seed=9, step=4)
    torch.cuda.synchronize()
    assert torch.equal(tok, tok2)
    tok, nti_h, T_h = tok.cpu().numpy(), nti.cpu().numpy(), T.cpu().numpy()
    rng = np.random.default_rng(1)
    ex = nf = 0
    for b in sorted(rng.choice(B, 8, replace=False)):
        rows = nti_h[b]
        sub = workloads.logits_numpy(logits[torch.from_numpy(rows.astype(np.int64)).cuda()])
        e_, near, fails = compare_draft(sub, np.arange(K, dtype=np.int32).reshape(1, K), T_h[b:b + 1],
                                        tok[b:b + 1], seed=9, step=4, request_base=int(b))
        assert not fails, (b, fails)
        ex += e_
        nf += len(near)
    say("  64 positions: %d exact, %d near-threshold" % (ex, nf))
