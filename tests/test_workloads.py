"""The seeded input recipes build what they say (shapes, laws, determinism)."""
import numpy as np
import torch

import workloads
from stats_helpers import softmax_rows


def test_tiny_recipe_shapes_and_determinism():
    a = workloads.verify_tiny(seed=0)
    b = workloads.verify_tiny(seed=0)
    assert a.target.shape == (4, 5, 1024) and a.target.dtype == torch.float32
    assert a.draft_tokens.shape == (4, 4) and a.draft_tokens.dtype == torch.int32
    assert torch.equal(a.target, b.target) and torch.equal(a.draft_tokens, b.draft_tokens)
    c = workloads.verify_tiny(seed=1)
    assert not torch.equal(a.target, c.target)
    # N(0, 2) target, draft noise N(0, 0.5)
    assert abs(float(a.target.std()) - 2.0) < 0.05
    assert abs(float((a.draft - a.target).std()) - 0.5) < 0.02


def test_zipf_profile():
    g = torch.Generator().manual_seed(0)
    z = workloads.zipf_logits(8, 5000, g, "cpu")
    s = torch.sort(z, dim=1, descending=True).values.mean(0)
    r = torch.arange(1, 5001, dtype=torch.float32)
    # sorted logits follow -1.1 ln r up to the N(0, 0.3) noise (which inflates the top)
    mid = slice(100, 4000)
    slope = np.polyfit(np.log(r[mid].numpy()), s[mid].numpy(), 1)[0]
    assert abs(slope + 1.1) < 0.05
    # each row is a permutation: not sorted
    assert not torch.all(z[:, 1:] <= z[:, :-1])


def test_mixture_recipe_and_tokens():
    inp = workloads.mixture_inputs("t", 24, 3, 2000, torch.bfloat16, 0, "cpu", temps=(0.0, 0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.6)
    T = inp.temperature.numpy()
    assert set(np.unique(T)) <= {0.0, np.float32(0.6), 1.0}
    lam = inp.lam.numpy()
    assert (lam >= 0.05).all() and (lam <= 0.6).all()
    x = inp.draft_tokens.numpy()
    d = inp.draft.float().numpy()
    for b in range(inp.B):
        if T[b] == 0:
            assert (x[b] == np.argmax(d[b, :3], axis=1)).all()
    # acceptance of the mixture: sum min(p, q) = 1 - lam * TV(p, r) roughly in [0.45, 1)
    t = inp.target.float().numpy()
    for b in range(inp.B):
        if T[b] > 0:
            p = softmax_rows(t[b, 0], T[b])
            q = softmax_rows(d[b, 0], T[b])
            alpha = np.minimum(p, q).sum()
            assert 0.4 < alpha < 1.0


def test_expand_recipe():
    e = workloads.expand_inputs(B=512, K=8, H=32, seed=0)
    assert e.N_in == 512 * 9 and e.N_out == 512 * 16
    acc = e.accepted.numpy()
    assert acc.min() >= 0 and acc.max() <= 8 and len(np.unique(acc)) == 9
    pos = e.in_positions.numpy().reshape(512, 9)
    assert (np.diff(pos, axis=1) == 1).all() and pos[:, 0].min() >= 0 and pos[:, 0].max() < 16384
    ids = e.in_token_ids.numpy()
    assert ids.min() >= 0 and ids.max() < 201088
    assert e.mask_id == 201088
