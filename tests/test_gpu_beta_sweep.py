"""The acceptance-rate sweep on the GPU: B=1024 requests, K=8, V=201088 bf16,
T = 1, draft q = (1 - lam) p + lam softmax(N(0, 1)) with lam tuned so the
per-token acceptance lands at beta = 0.5, 0.8 and 0.9; 100 verification steps
each on the same logits with the draft tokens redrawn per step.

Checks (explainer page, section "一轮能赚多少": a round yields
(1 - beta^(gamma+1)) / (1 - beta) tokens on average at acceptance beta):
  * the measured mean tokens per round equals the exact expectation of these
    rows, mean_b sum_{j=0..K} prod_{i<j} alpha_{b,i} with alpha = sum min(p, q),
    within 4 standard errors;
  * it equals the closed form at the measured beta_hat within 4 standard errors
    plus the gap the spread of alpha across rows puts between the closed form
    and the exact expectation;
  * beta_hat lands within 0.03 of its target;
  * steps 0 and 99 match the oracle on every request, and a planned
    early-exit cut and the dynamic exit of the same steps are bit-identical
    to one pass.
"""
import sys
import time

import numpy as np
import pytest
import torch

import workloads
from parity import Report, compare
from stats_helpers import expected_tokens_per_round

pytestmark = pytest.mark.gpu

B, K, V = 1024, 8, workloads.GPT_OSS_VOCAB
STEPS = 100


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def row_alpha(inp, rows=None):
    """alpha = sum_v min(p, q) of every draft position (library softmax on the
    rounded logits), [B, K] float64."""
    out = torch.empty(inp.B, inp.K, dtype=torch.float64, device=inp.target.device)
    for b0 in range(0, inp.B, 64):
        b1 = min(inp.B, b0 + 64)
        T = inp.temperature[b0:b1].reshape(-1, 1, 1)
        p = torch.softmax(inp.target[b0:b1, :inp.K].float() / T, dim=2)
        q = torch.softmax(inp.draft[b0:b1, :inp.K].float() / T, dim=2)
        out[b0:b1] = torch.minimum(p, q).sum(dim=2, dtype=torch.float64)
    return out


def tuned_lambda(beta, device):
    tv = workloads.total_variation_noise(V, rows=16, seed=7, device=device)
    lam = (1.0 - beta) / tv
    probe = workloads.verify_beta_sweep(lam, seed=99, device=device, B=32)
    alpha = float(row_alpha(probe).mean())
    return lam * (1.0 - beta) / (1.0 - alpha)  # one re-tuning pass


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rejection_sampling_verify_03_amd as m
    return m


@pytest.mark.parametrize("beta", [0.5, 0.8, 0.9])
def test_beta_sweep_closed_form(sv, beta):
    say("case: beta sweep B1024 K8 V201088, beta %.1f" % beta)
    dev = torch.device("cuda")
    lam = tuned_lambda(beta, dev)
    inp = workloads.verify_beta_sweep(lam, seed=int(beta * 10), device=dev, B=B, K=K, V=V)
    alpha = row_alpha(inp)
    exact = torch.ones(B, dtype=torch.float64, device=dev)
    run = torch.ones(B, dtype=torch.float64, device=dev)
    for j in range(K):
        run = run * alpha[:, j]
        exact += run
    exact_mean = float(exact.mean())
    ws = sv.make_workspace(B, K, V, dev)
    acc_all = []
    gpu_ms = 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tl = dl = None
    for s in range(STEPS):
        x = inp.draft_tokens if s == 0 else workloads.redraw_tokens(inp, seed=1000 + s)
        check = s in (0, STEPS - 1)
        e0.record()
        acc, tok, dbg = sv.verify(inp.target, inp.draft, x, inp.temperature, seed=3, step=s, workspace=ws,
                                  debug=check)
        e1.record()
        torch.cuda.synchronize()
        gpu_ms += e0.elapsed_time(e1)
        acc_all.append(acc.cpu().numpy())
        if check:
            # a planned early-exit cut of the same step: bit-identical outputs
            surv = sv.survival_from_accepted(np.concatenate(acc_all), K)
            mask = sv.spec_verify_plan_phases(K, surv, 1.0, 0.2) or 0b1000
            acc2, tok2, _ = sv.verify(inp.target, inp.draft, x, inp.temperature, seed=3, step=s, workspace=ws,
                                      phase_starts=mask)
            acc3, tok3, _ = sv.verify(inp.target, inp.draft, x, inp.temperature, seed=3, step=s, workspace=ws,
                                      phase_starts=sv.SPEC_PHASES_DYNAMIC)
            torch.cuda.synchronize()
            assert torch.equal(acc, acc2) and torch.equal(tok, tok2), (s, mask)
            assert torch.equal(acc, acc3) and torch.equal(tok, tok3), (s, "dynamic")
            if tl is None:
                tl, dl = workloads.logits_numpy(inp.target), workloads.logits_numpy(inp.draft)
            rep = Report()
            t0 = time.time()
            compare(tl, dl, x.cpu().numpy(), inp.temperature.cpu().numpy(), acc.cpu().numpy(), tok.cpu().numpy(),
                    dbg.cpu().numpy(), seed=3, step=s, report=rep)
            say("  step %d, every request (one pass = cut %#x): %s (oracle %.1f s)"
                % (s, mask, rep.summary(), time.time() - t0))
            assert rep.ok(), rep.failures[:5]
    del tl, dl
    a = np.stack(acc_all).astype(np.float64)  # [STEPS, B]
    assert (a >= 0).all() and (a <= K).all()
    tokens = a + 1.0
    mean_tok = float(tokens.mean())
    se = float(tokens.std()) / np.sqrt(tokens.size)
    beta_hat = float(a.sum() / np.minimum(a + 1, K).sum())
    closed = expected_tokens_per_round(beta_hat, K)
    hetero = abs(exact_mean - expected_tokens_per_round(float(alpha.mean()), K))
    say("  lam %.4f  beta_hat %.4f  mean tokens %.4f (se %.4f)  exact %.4f  closed form %.4f  alpha spread gap %.4f"
        % (lam, beta_hat, mean_tok, se, exact_mean, closed, hetero))
    ms = gpu_ms / STEPS
    say("  verify %.1f us/step -> %.2fM verified positions/s" % (ms * 1e3, B * K / ms / 1e3))
    assert abs(mean_tok - exact_mean) < 4 * se
    assert abs(mean_tok - closed) < 4 * se + hetero + 1e-3
    assert abs(beta_hat - beta) < 0.03
