"""The allocation-free verification entry point (spec_verify_launch_noalloc,
for callers that cannot allocate) against spec_verify_launch through the C
ABI: the same outputs bit for bit on two calls in a row on the GPU's shared
scratch array, the second with a smaller batch (stale contents of the first
must not leak into it), one pass and early-exit phases; a shape beyond the
array is refused before anything is enqueued."""
import sys

import pytest
import torch

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


def both(sv, inp, seed, step, phase_starts=0):
    """(accepted, tokens, debug) of spec_verify_launch and of the
    allocation-free call on the same inputs."""
    res = []
    for noalloc in (False, True):
        B, K = inp.draft_tokens.shape
        acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        tok = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
        dbg = torch.full((B, K, 2), -7.0, dtype=torch.float32, device="cuda")
        ws = None if noalloc else sv.make_workspace(B, K, inp.V)
        a = sv.verify_args(inp.target, inp.draft, inp.draft_tokens, inp.temperature, acc, tok, dbg, ws,
                           seed=seed, step=step, phase_starts=phase_starts)
        launch = sv.spec_verify_launch_noalloc if noalloc else sv.spec_verify_launch
        assert launch(a, torch.cuda.current_stream().cuda_stream) == sv.SPEC_OK
        torch.cuda.synchronize()
        res.append((acc, tok, dbg))
    return res


def test_noalloc_matches_the_workspace_call(sv):
    big = workloads.verify_headline(seed=3, device="cuda")  # B=256, K=8, V=151936 bf16, mixed T
    small = workloads.mixture_inputs("small", 12, 5, 40000, torch.bfloat16, 4, "cuda", temps=(0.0, 0.6, 1.0),
                                     lam_lo=0.05, lam_hi=0.6)
    need = sv.spec_verify_workspace_bytes(big.B, big.K, big.V)
    say("case: no-alloc verify, headline batch then a smaller one (workspace %d of %d bytes)"
        % (need, sv.SPEC_NOALLOC_SCRATCH_BYTES))
    assert need <= sv.SPEC_NOALLOC_SCRATCH_BYTES
    # the dynamic exit first: the array is still all zero bytes on the library's first call through this
    # entry point (its launch counter at 0), which must not pass for records of the launch
    for inp, seed, step, cut in ((big, 5, 2, sv.SPEC_PHASES_DYNAMIC), (big, 1, 0, 0), (small, 2, 5, 0),
                                 (big, 3, 7, 0b1000), (small, 4, 1, 0b100), (big, 8, 2, sv.SPEC_PHASES_DYNAMIC),
                                 (small, 6, 3, sv.SPEC_PHASES_DYNAMIC)):
        (a1, t1, d1), (a2, t2, d2) = both(sv, inp, seed, step, cut)
        assert torch.equal(a1, a2) and torch.equal(t1, t2) and torch.equal(d1, d2), (inp.name, seed, step, cut)
        assert (a1 >= 0).all()
        say("  %s seed %d step %d cut %#x: identical" % (inp.name, seed, step, cut))


def test_noalloc_refuses_shapes_beyond_its_array(sv):
    say("case: no-alloc verify, shapes beyond the scratch array")
    B, K, V = 4096, 8, 201088
    assert sv.spec_verify_workspace_bytes(B, K, V) > sv.SPEC_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(B, K, dtype=torch.int32, device="cuda")
    T = torch.ones(B, device="cuda")
    t = torch.zeros(1, K + 1, V, dtype=torch.bfloat16, device="cuda").expand(B, K + 1, V)
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
    a = sv.verify_args(t, t, x, T, acc, tok, None, None)
    assert sv.spec_verify_launch_noalloc(a, torch.cuda.current_stream().cuda_stream) == sv.SPEC_EWORKSPACE
    torch.cuda.synchronize()
    assert (acc == -7).all() and (tok == -7).all()  # nothing was enqueued


def test_noalloc_under_graph_capture(sv):
    """The caller it is for: a verification captured in a HIP graph with no
    allocation inside the capture (the workspace is the library's own array)
    and replayed four times, with eager work and an output reset between the
    replays; every replay equals the eager call, phased and one pass."""
    say("case: no-alloc verify captured in a graph")
    inp = workloads.mixture_inputs("graph", 32, 8, 32768, torch.bfloat16, 21, "cuda", temps=(0.0, 0.6, 1.0),
                                   lam_lo=0.05, lam_hi=0.6)
    B, K = 32, 8
    for cut in (0, 0b100100, sv.SPEC_PHASES_DYNAMIC):
        acc = torch.empty(B, dtype=torch.int32, device="cuda")
        tok = torch.empty(B, K + 1, dtype=torch.int32, device="cuda")
        a = sv.verify_args(inp.target, inp.draft, inp.draft_tokens, inp.temperature, acc, tok, None, None,
                           seed=4, step=9, phase_starts=cut)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            assert sv.spec_verify_launch_noalloc(a, s.cuda_stream) == sv.SPEC_OK
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        eager = (acc.clone(), tok.clone())
        g = torch.cuda.CUDAGraph()
        acc.fill_(-5)
        tok.fill_(-5)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            assert sv.spec_verify_launch_noalloc(a, torch.cuda.current_stream().cuda_stream) == sv.SPEC_OK
        for rep in range(4):
            x = torch.randn(1 << 20, device="cuda")
            float(x.sum())
            acc.fill_(-5)
            tok.fill_(-5)
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(acc, eager[0]) and torch.equal(tok, eager[1]), (cut, rep)
        say("  cut %#x: 4 replays identical to the eager call" % cut)
