"""Pins of the oracle's Philox4x32-10 stream and its uniform mapping."""
import json
import os

import numpy as np

import oracle
import philox_cases

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox_known_answer_vectors():
    with open(os.path.join(GOLDEN, "philox_kat.json")) as f:
        kat = json.load(f)
    for v in kat["vectors"]:
        ctr = [int(x, 16) for x in v["ctr"]]
        key = [int(x, 16) for x in v["key"]]
        want = [int(x, 16) for x in v["out"]]
        got = [int(x) for x in oracle.philox4x32_10(ctr, key)]
        assert got == want, (v, [hex(x) for x in got])


def test_uniform_mapping_is_exact_24_bit():
    assert oracle.uniform(0) == 0.0
    assert oracle.uniform(0xFF) == 0.0  # the low 8 bits are dropped
    assert oracle.uniform(0x100) == 2.0 ** -24
    top = oracle.uniform(0xFFFFFFFF)
    assert top == (2 ** 24 - 1) / 2 ** 24 and top < 1.0
    ws = np.random.default_rng(1).integers(0, 2 ** 32, 1000, dtype=np.uint64)
    for w in ws[:50]:
        u = oracle.uniform(int(w))
        assert u * 2 ** 24 == float(int(w) >> 8)


def test_counter_layout_of_verification_draws():
    """Word 0 of counter {request, row, step, 0} under key {seed lo, seed hi}
    drives the accept test of that row and word 1 its sampling draw: a request
    whose only row is evaluated exposes both through the trace."""
    import ctypes
    seed, step, req, row = 0x0123456789ABCDEF, 7, 5, 0
    ua, us = ctypes.c_double(), ctypes.c_double()
    L = oracle.lib()
    L.oracle_verify_uniforms.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                         ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    L.oracle_verify_uniforms(seed, step, req, row, ctypes.byref(ua), ctypes.byref(us))
    out = oracle.philox4x32_10([req, row, step, 0], [seed & 0xFFFFFFFF, seed >> 32])
    assert ua.value == (int(out[0]) >> 8) / 2 ** 24
    assert us.value == (int(out[1]) >> 8) / 2 ** 24
    # and oracle_verify consumes exactly those: a one-request, K=1 case whose
    # draft never matches p's support is always rejected, so the trace holds
    # the accept draw and the sampling draw of row 0 at request_base + 0
    V = 4
    t = np.full((1, 2, V), -np.inf, np.float32)
    t[0, :, 0] = 0.0
    d = np.full((1, 2, V), -np.inf, np.float32)
    d[0, :, 3] = 0.0
    r = oracle.verify(t, d, [[3]], [1.0], seed=seed, step=step, request_base=req)
    assert r.accepted[0] == 0 and r.tokens[0, 0] == 0
    assert r.trace[0, 0, 0] == ua.value and r.trace[0, 0, 2] == us.value


def test_device_stream_cases_match_the_oracle():
    """The closed forms the device-versus-oracle stream test expects
    (philox_cases) are the oracle's own outputs on those inputs: draft tokens
    over equal logits, and verification over uniform target rows with
    restricted draft rows, ragged counts and wrapping request indices."""
    for seed, step, base in ((0, 0, 0), ((1 << 64) - 1, 0xFFFFFFFF, 0xFFFFFFFF - 20), (1 << 32, 99, 7)):
        want = philox_cases.draft_expected(seed, step, base, 40, 9, 4096)
        r = oracle.draft_sample(np.zeros((1, 4096), np.float32), np.zeros((40, 9), np.int32),
                                np.ones(40, np.float32), seed=seed, step=step, request_base=base)
        assert np.array_equal(r.tokens, want)
    rng = np.random.default_rng(5)
    for seed, step, base in ((3, 1, 0), (0xFEDCBA9876543210, 1 << 31, 0xFFFFFFFF - 30)):
        c = philox_cases.VerifyCase(rng, 60, 63, 1024)
        want_a, want_y, _ = c.expected(seed, step, base)
        draft = c.drows[c.ridx]  # the row table gathered into [B, K, V]
        r = oracle.verify(c.target, draft, c.x, np.ones(c.B, np.float32), seed=seed, step=step,
                          request_base=base, num_drafts=c.kb, debug=False, trace=False)
        assert np.array_equal(r.accepted, want_a)
        assert np.array_equal(r.tokens[np.arange(c.B), want_a], want_y)
