"""The device's Philox4x32-10 streams against the oracle's, through the
public C ABI, on more than 10^6 counters.

The explainer page ("修正拒绝采样") draws one `random.random()` per accept
test and one per resample; here those draws come from a counter-based
generator keyed on (seed, request, position, step), implemented once on each
side.  The oracle's copy is pinned by the published known-answer vectors
(tests/test_oracle_philox.py); this file checks the device's copy against it
wherever the counter words can reach -- all four words, both key halves, the
request index wrapping past 2^32 -- using inputs whose outputs are a closed
form of the uniform:

* drafting stream (counter word 3 = 1, word 0): V equal logits make the
  inverse CDF the integer part of u * V, so a draft token IS the top
  log2(V) bits of the uniform (V = 4096 on 2^20 positions, V = 2^20 and
  V = 2^24 -- every bit -- on fewer);
* verification stream (word 3 = 0): with shared uniform target rows, a
  request with K_b drafts accepts positions 0..K_b-2 for sure (q = p there)
  and position j = K_b - 1 iff u_j < m / V (a draft row uniform over its
  first m tokens), then emits floor(u'_{K_b} V) (bonus, all accepted) or
  m + floor(u'_j (V - m)) (residual, uniform over the tokens the draft row
  leaves out); K_b = 0 emits floor(u'_0 V).  That exposes word 0 (one
  comparison) and word 1 (ten bits) of every request, at every position
  0..63.
"""
import sys

import numpy as np
import pytest
import torch

import philox_cases

pytestmark = pytest.mark.gpu

M32 = philox_cases.M32
SEEDS = [0, 1, M32, 1 << 32, (1 << 63) | 5, (1 << 64) - 1, 0x0123456789ABCDEF, 0xFEDCBA9876543210]
STEPS = [0, 1, 99, 1 << 16, 1 << 31, M32 - 1, M32, 0x5A5A5A5A]


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import rejection_sampling_verify_03_amd as m
    return m


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def draft_case(sv, V, B, K, seed, step, request_base, dtype=torch.float32):
    logits = torch.zeros(1, V, dtype=dtype, device="cuda")
    row_index = torch.zeros(B, K, dtype=torch.int32, device="cuda")
    T = torch.ones(B, dtype=torch.float32, device="cuda")
    tok = sv.draft_sample(logits, row_index, T, seed=seed, step=step, request_base=request_base)
    torch.cuda.synchronize()
    want = philox_cases.draft_expected(seed, step, request_base, B, K, V)
    got = tok.cpu().numpy().astype(np.int64)
    bad = np.argwhere(got != want)
    assert bad.size == 0, ("drafting stream", V, seed, step, request_base, bad[:5].tolist(),
                           [(int(got[i, j]), int(want[i, j])) for i, j in bad[:5]])
    return B * K


def test_drafting_stream_against_oracle(sv):
    say("case: drafting stream, equal-logit rows, 2^20 positions at V=4096")
    n = 0
    bases = [0, 1, (1 << 31) - 700, M32 - 511, 123456789, 1 << 20, M32, 77]
    for i in range(8):
        n += draft_case(sv, 4096, 1024, 128, SEEDS[i], STEPS[i], bases[i])
    say("  %d counters: top 12 bits of every uniform" % n)
    assert n >= 1 << 20
    say("case: drafting stream, V=2^20 and V=2^24 (every bit)")
    draft_case(sv, 1 << 20, 64, 64, SEEDS[6], STEPS[4], M32 - 31)
    draft_case(sv, 1 << 24, 16, 16, SEEDS[7], STEPS[5], 3, dtype=torch.bfloat16)


def verify_case(sv, rng, B, K, V, seed, step, request_base):
    dev = torch.device("cuda")
    c = philox_cases.VerifyCase(rng, B, K, V)
    acc, tok, _ = sv.verify(torch.from_numpy(c.target).to(dev).expand(B, K + 1, V),
                            torch.from_numpy(c.drows).to(dev), torch.from_numpy(c.x).to(dev),
                            torch.ones(B, dtype=torch.float32, device=dev), seed=seed, step=step,
                            request_base=request_base, draft_row_index=torch.from_numpy(c.ridx).to(dev),
                            num_drafts=torch.from_numpy(c.kb).to(dev))
    torch.cuda.synchronize()
    acc, tok = acc.cpu().numpy(), tok.cpu().numpy()
    want_a, want_y, accept = c.expected(seed, step, request_base)
    bad = np.nonzero(acc != want_a)[0]
    assert bad.size == 0, ("accepted counts", seed, step, request_base, bad[:5].tolist(),
                           acc[bad[:5]].tolist(), want_a[bad[:5]].tolist())
    y = tok[np.arange(B), want_a]
    bad = np.nonzero(y != want_y)[0]
    assert bad.size == 0, ("emitted tokens", seed, step, request_base, bad[:5].tolist(),
                           y[bad[:5]].tolist(), want_y[bad[:5]].tolist())
    for b in range(min(B, 256)):  # the accepted prefix and the -1 padding
        a = want_a[b]
        assert list(tok[b, :a]) == list(c.x[b, :a]) and (tok[b, a + 1:] == -1).all(), b
    return B, int((c.kb > 0).sum()), int(accept.sum())


def test_verification_stream_against_oracle(sv):
    say("case: verification stream, uniform rows, ragged K_b in 0..63, 2^19 requests")
    rng = np.random.default_rng(2024)
    bases = [0, M32 - 8191, 1 << 31, 5, 999_999, M32 - 1, 1 << 24, 31337]
    n = tests = acc = 0
    for i in range(32):
        r = verify_case(sv, rng, 16384, 63, 1024, SEEDS[i % 8], STEPS[(i * 3) % 8], bases[(i * 5) % 8])
        n += r[0]
        tests += r[1]
        acc += r[2]
    say("  %d requests: %d word-0 accept tests (%d accepted), %d word-1 draws" % (n, tests, acc, n))
    # every request used one word-1 draw and (K_b > 0) one word-0 comparison
    assert n + tests >= 1_000_000
