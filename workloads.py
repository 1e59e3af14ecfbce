"""Seeded synthetic inputs for the verification and expansion workloads.

This module only BUILDS inputs: logits, draft tokens, temperatures, accepted
counts, positions and hidden rows.  It holds none of the verification or
expansion arithmetic, and both the HIP path and the CPU oracle consume exactly
the tensors it returns.  Everything runs in torch on the requested device with
a seeded ``torch.Generator`` (the same seed on the same device gives the same
tensors).

The pages measure end to end on public benchmarks with trained models; none of
that is available here, so these recipes stand in for them with the shapes and
value distributions of the pages' workloads:

* a GPT-OSS-sized vocabulary (V = 201088) and a Qwen3-family vocabulary
  (V = 151936), K in {4, 5, 8} drafts per request;
* "Zipf" target rows: the sorted rank r gets logit -1.1 ln r + N(0, 0.3),
  then an independent random permutation per row;
* draft rows as target plus Gaussian noise, or as the mixture
  q = (1 - lam) p_T + lam softmax(N(0, 1)) stored as T ln q;
* draft tokens drawn from the (rounded) draft distribution by the Gumbel-max
  trick, or the draft argmax for greedy requests.

N(mu, s) always means mean mu and STANDARD DEVIATION s.
"""
import torch

GPT_OSS_VOCAB = 201088
QWEN3_VOCAB = 151936
HIDDEN_GPT_OSS_20B = 2880


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def zipf_logits(rows, V, g, device, slope=1.1, noise=0.3, batch=256):
    """[rows, V] float32: rank r (1-based) gets -slope*ln r + N(0, noise), then
    a random permutation per row."""
    base = -slope * torch.log(torch.arange(1, V + 1, device=device, dtype=torch.float32))
    out = torch.empty(rows, V, device=device, dtype=torch.float32)
    for r0 in range(0, rows, batch):
        r1 = min(rows, r0 + batch)
        n = r1 - r0
        vals = base.unsqueeze(0) + noise * torch.randn(n, V, generator=g, device=device)
        perm = torch.argsort(torch.rand(n, V, generator=g, device=device), dim=1)
        out[r0:r1].scatter_(1, perm, vals)
    return out


def gumbel_argmax(logits, g, batch=128):
    """One draw per row from softmax(logits) by the Gumbel-max trick, in
    float64: with float32 uniforms the largest Gumbel values -- the ones that
    pick the winner among ~1e5 tokens -- sit on a coarse grid (the uniforms'
    2^-24 spacing next to 1) and over-weight the likeliest tokens.  -inf logits
    are never drawn."""
    rows, V = logits.shape
    out = torch.empty(rows, dtype=torch.int64, device=logits.device)
    tiny = torch.finfo(torch.float64).tiny
    for r0 in range(0, rows, batch):
        r1 = min(rows, r0 + batch)
        u = torch.rand(r1 - r0, V, generator=g, device=logits.device, dtype=torch.float64).clamp_min_(tiny)
        gumbel = -torch.log(-torch.log(u))
        out[r0:r1] = torch.argmax(logits[r0:r1].double() + gumbel, dim=1)
    return out


def _mixture_log_density(base_f32, noise_f32, lam):
    """log((1 - lam) softmax(base) + lam softmax(noise)) per row (lam per row)."""
    lam = lam.reshape(-1, 1)
    lp = torch.log_softmax(base_f32, dim=1)
    ln = torch.log_softmax(noise_f32, dim=1)
    return torch.logaddexp(torch.log1p(-lam) + lp, torch.log(lam) + ln)


class VerifyInputs:
    """Inputs of one verification step.

    target: [B, K+1, V] (float32 or bfloat16), draft: [B, K+1, V] (row K is
    present but never read), draft_tokens: [B, K] int32, temperature: [B] f32.
    """

    def __init__(self, name, target, draft, draft_tokens, temperature, seed, step=0, lam=None):
        self.name = name
        self.target = target
        self.draft = draft
        self.draft_tokens = draft_tokens
        self.temperature = temperature
        self.seed = seed
        self.step = step
        self.lam = lam
        self.B, self.K1, self.V = target.shape
        self.K = self.K1 - 1

    @property
    def dtype(self):
        return self.target.dtype

    def bytes_per_logit(self):
        return self.target.element_size()


def _draw_tokens(draft, temperature, K, g):
    """Draft tokens: x ~ softmax(draft/T) for T > 0, argmax(draft) for T = 0."""
    B, _, V = draft.shape
    rows = draft[:, :K, :].reshape(B * K, V).float()
    T = temperature.repeat_interleave(K).to(rows.device)
    scaled = torch.where(T.reshape(-1, 1) > 0, rows / T.clamp_min(1e-30).reshape(-1, 1), rows)
    sampled = gumbel_argmax(scaled, g)
    greedy = torch.argmax(rows, dim=1)
    x = torch.where(T > 0, sampled, greedy)
    return x.reshape(B, K).to(torch.int32)


def noisy_draft_inputs(name, B, K, V, dtype, seed, device, recipe, target_std=2.0, draft_noise=0.5,
                       temperature=1.0, temps=None, offset=0.0):
    """Target rows from ``recipe`` ("gauss": i.i.d. N(0, target_std); "zipf"),
    draft rows = target + N(0, draft_noise), both shifted by ``offset`` (a
    shift leaves every softmax unchanged); a single temperature, or one per
    request drawn uniformly from ``temps``."""
    g = _gen(seed, device)
    if recipe == "gauss":
        t = target_std * torch.randn(B * (K + 1), V, generator=g, device=device)
    elif recipe == "zipf":
        t = zipf_logits(B * (K + 1), V, g, device)
    else:
        raise ValueError(recipe)
    d = t + draft_noise * torch.randn(B * (K + 1), V, generator=g, device=device)
    target = (t + offset).reshape(B, K + 1, V).to(dtype)
    draft = (d + offset).reshape(B, K + 1, V).to(dtype)
    del t, d
    if temps is None:
        temp = torch.full((B,), float(temperature), dtype=torch.float32, device=device)
    else:
        tt = torch.tensor(temps, dtype=torch.float32, device=device)
        temp = tt[torch.randint(0, len(temps), (B,), generator=g, device=device)].contiguous()
    x = _draw_tokens(draft, temp, K, g)
    return VerifyInputs(name, target, draft, x, temp, seed)


def mixture_inputs(name, B, K, V, dtype, seed, device, temps, lam_lo=None, lam_hi=None, lam=None,
                   batch_requests=32):
    """Zipf target rows; per request a temperature drawn uniformly from
    ``temps`` and a mixture weight lam (uniform in [lam_lo, lam_hi], or fixed);
    q = (1 - lam) softmax(target / T') + lam softmax(N(0, 1)) with T' = T for
    sampled requests and T' = 1 for greedy ones; draft logits = T ln q for
    T > 0 and ln q for T = 0."""
    g = _gen(seed, device)
    temps_t = torch.tensor(temps, dtype=torch.float32, device=device)
    temperature = temps_t[torch.randint(0, len(temps), (B,), generator=g, device=device)]
    if lam is None:
        lam_b = lam_lo + (lam_hi - lam_lo) * torch.rand(B, generator=g, device=device)
    else:
        lam_b = torch.full((B,), float(lam), device=device)
    target = torch.empty(B, K + 1, V, dtype=dtype, device=device)
    draft = torch.empty(B, K + 1, V, dtype=dtype, device=device)
    for b0 in range(0, B, batch_requests):
        b1 = min(B, b0 + batch_requests)
        nb = b1 - b0
        t = zipf_logits(nb * (K + 1), V, g, device).reshape(nb, K + 1, V)
        target[b0:b1] = t.to(dtype)
        t = target[b0:b1].float()  # the rounded logits define p
        T = temperature[b0:b1]
        Tp = torch.where(T > 0, T, torch.ones_like(T))
        base = (t / Tp.reshape(-1, 1, 1)).reshape(nb * (K + 1), V)
        noise = torch.randn(nb * (K + 1), V, generator=g, device=device)
        lq = _mixture_log_density(base, noise, lam_b[b0:b1].repeat_interleave(K + 1))
        lq = lq.reshape(nb, K + 1, V)
        Td = torch.where(T > 0, T, torch.ones_like(T))
        draft[b0:b1] = (Td.reshape(-1, 1, 1) * lq).to(dtype)
        del t, base, noise, lq
    x = _draw_tokens(draft, temperature, K, g)
    return VerifyInputs(name, target, draft, x, temperature, seed, lam=lam_b)


# ----------------------------------------------------------- named workloads
def verify_tiny(seed=0, device="cpu"):
    """B=4, K=4, V=1024 fp32; target N(0, 2) i.i.d.; draft = target + N(0, 0.5);
    temperature 1."""
    return noisy_draft_inputs("tiny B4 K4 V1024 fp32", 4, 4, 1024, torch.float32, seed, device,
                              "gauss", target_std=2.0, draft_noise=0.5)


def verify_gptoss(seed=0, device="cpu"):
    """B=64, K=5, V=201088 bf16; Zipf target; draft = target + N(0, 0.7); T = 1."""
    return noisy_draft_inputs("gpt-oss vocab B64 K5 V201088 bf16", 64, 5, GPT_OSS_VOCAB,
                              torch.bfloat16, seed, device, "zipf", draft_noise=0.7)


def verify_headline(seed=0, device="cpu", B=256, K=8, V=QWEN3_VOCAB):
    """B=256, K=8, V=151936 bf16; Zipf target; T per request from {0, 0.6, 1};
    mixture draft with lam ~ U[0.05, 0.6]."""
    return mixture_inputs("headline B%d K%d V%d bf16 mixed-T" % (B, K, V), B, K, V, torch.bfloat16,
                          seed, device, temps=(0.0, 0.6, 1.0), lam_lo=0.05, lam_hi=0.6)


def total_variation_noise(V, rows, seed, device, T=1.0):
    """Mean total-variation distance between Zipf p (at temperature T) and
    softmax(N(0, 1)) over ``rows`` sample rows: the acceptance of the
    mixture draft is 1 - lam * TV, so lam = (1 - beta) / TV."""
    g = _gen(seed, device)
    t = zipf_logits(rows, V, g, device).to(torch.bfloat16).float()
    p = torch.softmax(t / T, dim=1)
    r = torch.softmax(torch.randn(rows, V, generator=g, device=device), dim=1)
    return float(0.5 * (p - r).abs().sum(dim=1).mean())


def verify_beta_sweep(lam, seed=0, device="cpu", B=1024, K=8, V=GPT_OSS_VOCAB):
    """B=1024, K=8, V=201088 bf16, T = 1, one mixture weight lam for every
    request (tuned so that the per-token acceptance lands at a target beta)."""
    return mixture_inputs("beta sweep B%d K%d V%d bf16 lam=%.4f" % (B, K, V, lam), B, K, V,
                          torch.bfloat16, seed, device, temps=(1.0,), lam=lam)


def redraw_tokens(inp, seed):
    """Fresh draft tokens for another step of the same logits."""
    g = _gen(seed, inp.target.device)
    return _draw_tokens(inp.draft, inp.temperature, inp.K, g)


class ExpandInputs:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def expand_inputs(B=512, K=8, H=HIDDEN_GPT_OSS_20B, vocab=GPT_OSS_VOCAB, seed=0, device="cpu",
                  n_per_request=None, max_offset=16384, mask_id=None, accepted=None):
    """Verify-batch outputs feeding one expansion: n_b = K + 1 input slots per
    request (or ``n_per_request`` [B]), accepted counts uniform in 0..n_b-1,
    int32 token ids and bonus tokens uniform in [0, vocab), int64 positions
    off_b + j with off_b uniform in [0, max_offset), bf16 N(0, 1) hidden rows
    of width H and a bf16 N(0, 1) mask placeholder row; MASK id = vocab."""
    g = _gen(seed, device)
    if n_per_request is None:
        n = torch.full((B,), K + 1, dtype=torch.int64, device=device)
    else:
        n = torch.as_tensor(n_per_request, dtype=torch.int64, device=device)
    in_start = torch.zeros(B + 1, dtype=torch.int64, device=device)
    in_start[1:] = torch.cumsum(n, 0)
    N_in = int(in_start[-1])
    if accepted is None:
        acc = torch.floor(torch.rand(B, generator=g, device=device) * n.double()).to(torch.int64)
    else:
        acc = torch.as_tensor(accepted, dtype=torch.int64, device=device)
    ids = torch.randint(0, vocab, (N_in,), generator=g, device=device, dtype=torch.int64)
    bonus = torch.randint(0, vocab, (B,), generator=g, device=device, dtype=torch.int64)
    off = torch.randint(0, max_offset, (B,), generator=g, device=device, dtype=torch.int64)
    req = torch.repeat_interleave(torch.arange(B, device=device), n)
    j = torch.arange(N_in, device=device) - in_start[:-1][req]
    pos = off[req] + j
    hidden = torch.randn(N_in, H, generator=g, device=device).to(torch.bfloat16)
    mask_hidden = torch.randn(H, generator=g, device=device).to(torch.bfloat16)
    return ExpandInputs(
        B=B, K=K, H=H, N_in=N_in, N_out=N_in + B * (K - 1),
        in_token_ids=ids.to(torch.int32), in_positions=pos, in_start=in_start.to(torch.int32),
        accepted=acc.to(torch.int32), bonus=bonus.to(torch.int32),
        mask_id=int(vocab if mask_id is None else mask_id),
        target_hidden=hidden, mask_hidden=mask_hidden)


def step_expand_inputs(inp, H=HIDDEN_GPT_OSS_20B, seed=0, block_size=16, max_offset=16384):
    """The expansion batch of one verification step of ``inp`` (a
    VerifyInputs on a device): per request the K+1 verified slots [last
    token, x_0..x_{K-1}] with the last token uniform in [0, V), int64
    positions off_b + j with off_b uniform in [0, max_offset), bf16 N(0, 1)
    hidden rows of width H and mask row, MASK id = the GPT-OSS vocabulary
    size, and a paged-KV block table of ``block_size``-slot blocks covering
    every position the expansion can produce."""
    dev = inp.target.device
    B, K, V = inp.B, inp.K, inp.V
    g = _gen(seed + 1, dev)
    last = torch.randint(0, V, (B, 1), generator=g, device=dev, dtype=torch.int32)
    in_ids = torch.cat([last, inp.draft_tokens], dim=1).reshape(-1).contiguous()
    off = torch.randint(0, max_offset, (B, 1), generator=g, device=dev, dtype=torch.int64)
    in_pos = (off + torch.arange(K + 1, device=dev)).reshape(-1).contiguous()
    in_start = (torch.arange(B + 1, device=dev, dtype=torch.int32) * (K + 1)).contiguous()
    hidden = torch.randn(B * (K + 1), H, generator=g, device=dev).to(torch.bfloat16)
    mask_hidden = torch.randn(H, generator=g, device=dev).to(torch.bfloat16)
    table = block_tables(B, (max_offset + 2 * K + 2) // block_size + 1, seed=seed + 2, device=dev)
    return ExpandInputs(B=B, K=K, H=H, N_in=B * (K + 1), N_out=B * (2 * K), in_token_ids=in_ids,
                        in_positions=in_pos, in_start=in_start, target_hidden=hidden, mask_hidden=mask_hidden,
                        mask_id=GPT_OSS_VOCAB, block_table=table, block_size=block_size)


class DraftInputs:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def drafter_inputs(B, K, N, V, dtype, seed, device, temps=(0.0, 0.6, 1.0), offset=0.0):
    """Drafter logits [N, V] (Zipf rows, as the target recipe, shifted by
    ``offset``), K row indices per request drawn uniformly from [0, N) (the
    new-token indices stand-in), and a temperature per request drawn uniformly
    from ``temps``."""
    g = _gen(seed, device)
    logits = (zipf_logits(N, V, g, device) + offset).to(dtype)
    row_index = torch.randint(0, N, (B, K), generator=g, device=device, dtype=torch.int64).to(torch.int32)
    t = torch.tensor(temps, dtype=torch.float32, device=device)
    temperature = t[torch.randint(0, len(temps), (B,), generator=g, device=device)]
    return DraftInputs(B=B, K=K, N=N, V=V, logits=logits, row_index=row_index.contiguous(),
                       temperature=temperature.contiguous())


def block_tables(B, max_blocks, seed, device="cpu", unmapped_fraction=0.0):
    """A synthetic paged-KV block table [B, max_blocks] int32: every entry a
    distinct physical block (a random permutation of 0..B*max_blocks-1), and
    a ``unmapped_fraction`` of entries set to -1 (no block)."""
    g = _gen(seed, device)
    perm = torch.randperm(B * max_blocks, generator=g, device=device).to(torch.int32).reshape(B, max_blocks)
    if unmapped_fraction > 0:
        drop = torch.rand(B, max_blocks, generator=g, device=device) < unmapped_fraction
        perm = torch.where(drop, torch.full_like(perm, -1), perm)
    return perm.contiguous()


def bf16_bits(t):
    """uint16 numpy view of a bfloat16 tensor (copied to the CPU)."""
    import numpy as np
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def logits_numpy(t):
    """Logits as the oracle takes them: float32 array or bf16 bit patterns."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().float().contiguous().numpy()


__all__ = [n for n in dir() if not n.startswith("_") and n != "torch"]
