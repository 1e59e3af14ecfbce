"""CPU oracle for speculative-decoding verification and P-EAGLE batch expansion.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the CPU
baseline leg of the benchmark may import this module; the product library never
does.  It wraps ``libspecoracle.so`` (plain scalar C in double precision, built
by ``oracle/build.py``) with ctypes over numpy arrays.

Pinning status of each function (what fixes it other than itself):
  * ``philox4x32_10`` / ``uniform``: published Philox known-answer vectors.
  * ``verify``: distribution-preservation chi-square (the explainer page,
    section "修正拒绝采样", theorem), the expected-tokens closed form (section
    "一轮能赚多少", with its printed table), exhaustive enumeration of all 2^24
    uniform codes on a V=4, K=2 case, and special cases (identical p and q,
    disjoint supports, one-hot targets, greedy argmax ties, V=1, K=1).
  * ``expand``: the invariants the P-EAGLE page fixes (mask partition,
    injective mapping, counts, positions, start indices), a hand-worked
    fixture, and the hidden-state fill written out row by row from the page's
    description.  The order of slots inside a request's window is a reading of the page
    and is pinned only by those invariants and the hand-worked fixture.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# SPEC_ORACLE_LIB names another build of the same sources (e.g. one with
# sanitizers, see build.py); default: the in-tree build
_LIB_PATH = os.environ.get("SPEC_ORACLE_LIB") or os.path.join(HERE, "libspecoracle.so")
_lib = None

F32, BF16 = 0, 1


class VerifyArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("target", ctypes.c_void_p), ("t_req_stride", ctypes.c_int64), ("t_row_stride", ctypes.c_int64),
        ("draft", ctypes.c_void_p), ("d_req_stride", ctypes.c_int64), ("d_row_stride", ctypes.c_int64),
        ("draft_tokens", ctypes.c_void_p), ("temperature", ctypes.c_void_p),
        ("seed", ctypes.c_uint64), ("step", ctypes.c_uint32), ("request_base", ctypes.c_uint32),
        ("uniforms", ctypes.c_void_p),
        ("accepted", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p),
        ("debug_probs", ctypes.c_void_p), ("trace", ctypes.c_void_p),
        ("mutation", ctypes.c_int32), ("nthreads", ctypes.c_int32), ("num_drafts", ctypes.c_void_p),
    ]


class ExpandArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("H", ctypes.c_int32), ("N_in", ctypes.c_int32),
        ("in_token_ids", ctypes.c_void_p), ("in_positions", ctypes.c_void_p),
        ("in_start", ctypes.c_void_p), ("accepted", ctypes.c_void_p), ("bonus", ctypes.c_void_p),
        ("mask_id", ctypes.c_int32),
        ("target_hidden", ctypes.c_void_p), ("hidden_row_stride", ctypes.c_int64),
        ("mask_hidden", ctypes.c_void_p),
        ("out_token_ids", ctypes.c_void_p), ("out_positions", ctypes.c_void_p),
        ("rejected_mask", ctypes.c_void_p), ("masked_mask", ctypes.c_void_p),
        ("new_token_indices", ctypes.c_void_p), ("hidden_map", ctypes.c_void_p),
        ("out_start", ctypes.c_void_p), ("out_hidden", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("bt_row_stride", ctypes.c_int64),
        ("max_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32), ("slot_mapping", ctypes.c_void_p),
    ]


class DraftArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("N", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("logits", ctypes.c_void_p), ("row_stride", ctypes.c_int64),
        ("row_index", ctypes.c_void_p), ("temperature", ctypes.c_void_p),
        ("seed", ctypes.c_uint64), ("step", ctypes.c_uint32), ("request_base", ctypes.c_uint32),
        ("tokens", ctypes.c_void_p), ("trace", ctypes.c_void_p), ("mutation", ctypes.c_int32),
    ]


def lib():
    """Load (building first if absent) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _build
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_uniform.argtypes = [ctypes.c_uint32]
        L.oracle_uniform.restype = ctypes.c_double
        L.oracle_accept.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
        L.oracle_accept.restype = ctypes.c_int
        L.oracle_invcdf.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_double]
        L.oracle_invcdf.restype = ctypes.c_int
        L.oracle_residual.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
        L.oracle_residual.restype = ctypes.c_int
        L.oracle_softmax.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                     ctypes.c_void_p]
        L.oracle_softmax.restype = ctypes.c_int
        L.oracle_argmax.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int]
        L.oracle_argmax.restype = ctypes.c_int
        L.oracle_scaled_max_in_range.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float]
        L.oracle_scaled_max_in_range.restype = ctypes.c_int
        L.oracle_accept_many.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_void_p]
        L.oracle_invcdf_many.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_void_p]
        L.oracle_verify.argtypes = [ctypes.POINTER(VerifyArgs)]
        L.oracle_verify.restype = ctypes.c_int
        L.oracle_sampling_weights.argtypes = [ctypes.POINTER(VerifyArgs), ctypes.c_int, ctypes.c_int,
                                              ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_sampling_weights.restype = ctypes.c_int
        L.oracle_expand.argtypes = [ctypes.POINTER(ExpandArgs)]
        L.oracle_expand.restype = ctypes.c_int
        L.oracle_draft_sample.argtypes = [ctypes.POINTER(DraftArgs)]
        L.oracle_draft_sample.restype = ctypes.c_int
        L.oracle_draft_uniform.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                           ctypes.c_void_p]
        L.oracle_draft_uniforms_many.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.oracle_verify_uniforms_many.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ primitives
def philox4x32_10(ctr, key):
    c = _c(ctr, np.uint32)
    k = _c(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(word):
    return lib().oracle_uniform(int(word) & 0xFFFFFFFF)


def accept(p_x, q_x, u):
    return bool(lib().oracle_accept(float(p_x), float(q_x), float(u)))


def accept_many(p_x, q_x, words):
    w = _c(words, np.uint32)
    out = np.zeros(w.shape[0], np.uint8)
    lib().oracle_accept_many(float(p_x), float(q_x), _ptr(w), w.shape[0], _ptr(out))
    return out


def invcdf(w, W, u):
    w = _c(w, np.float64)
    return lib().oracle_invcdf(_ptr(w), w.shape[0], float(W), float(u))


def invcdf_many(w, W, words):
    w = _c(w, np.float64)
    ws = _c(words, np.uint32)
    out = np.zeros(ws.shape[0], np.int32)
    lib().oracle_invcdf_many(_ptr(w), w.shape[0], float(W), _ptr(ws), ws.shape[0], _ptr(out))
    return out


def residual(p, q):
    p = _c(p, np.float64)
    q = _c(q, np.float64)
    w = np.zeros_like(p)
    W = ctypes.c_double(0.0)
    fb = lib().oracle_residual(_ptr(p), _ptr(q), p.shape[0], _ptr(w), ctypes.byref(W))
    return w, W.value, bool(fb)


def _logit_buffer(logits):
    """Return (contiguous array, dtype code).  bf16 logits are passed as their
    uint16 bit patterns; fp32 as float32."""
    a = np.asarray(logits)
    if a.dtype == np.uint16:
        return np.ascontiguousarray(a), BF16
    return np.ascontiguousarray(a, dtype=np.float32), F32


def softmax(logits, T):
    row, dt = _logit_buffer(logits)
    out = np.zeros(row.shape[-1], np.float64)
    rc = lib().oracle_softmax(_ptr(row), dt, row.shape[-1], float(T), _ptr(out))
    if rc != 0:
        raise ValueError("softmax undefined for this row/temperature")
    return out


def argmax(logits):
    row, dt = _logit_buffer(logits)
    return lib().oracle_argmax(_ptr(row), dt, row.shape[-1])


def scaled_max_in_range(logits, T):
    """True if the row's largest logit is finite and its scaled reference
    ceil(max * log2(e) / T) is an exact fp32 integer (|ref| <= 2^24): the
    range in which a sampled row's softmax is computed at all."""
    row, dt = _logit_buffer(logits)
    return bool(lib().oracle_scaled_max_in_range(_ptr(row), dt, row.shape[-1], float(T)))


# ---------------------------------------------------------------------- verify
class VerifyResult:
    def __init__(self, accepted, tokens, debug_probs, trace, n_bad):
        self.accepted = accepted
        self.tokens = tokens
        self.debug_probs = debug_probs
        self.trace = trace
        self.n_bad = n_bad


def _verify_struct(target, draft, draft_tokens, temperature, seed, step, request_base,
                   uniforms, mutation, nthreads, keep, num_drafts=None):
    t, dt = _logit_buffer(target)
    d, dd = _logit_buffer(draft)
    if dt != dd:
        raise ValueError("target and draft logits must share a dtype")
    Bt, K1, V = t.shape
    K = K1 - 1
    x = _c(draft_tokens, np.int32)
    B = x.shape[0]
    if Bt not in (1, B) or d.ndim != 3 or d.shape[0] not in (1, B) or d.shape[1] < K or d.shape[2] != V:
        raise ValueError("target must be [B or 1, K+1, V] and draft [B or 1, >=K, V]")
    x = x.reshape(B, K)
    T = _c(temperature, np.float32).reshape(B)
    u = None if uniforms is None else _c(uniforms, np.float64).reshape(B, K + 1, 2)
    keep.extend([t, d, x, T, u])
    a = VerifyArgs()
    a.B, a.K, a.V, a.dtype = B, K, V, dt
    # a leading dimension of 1 shares the same rows across every request
    a.target, a.t_req_stride, a.t_row_stride = _ptr(t), (K1 * V if Bt == B else 0), V
    a.draft, a.d_req_stride, a.d_row_stride = _ptr(d), (d.shape[1] * V if d.shape[0] == B else 0), V
    a.draft_tokens, a.temperature = _ptr(x), _ptr(T)
    a.seed, a.step, a.request_base = int(seed) & (2**64 - 1), int(step) & 0xFFFFFFFF, int(request_base)
    a.uniforms = _ptr(u)
    a.mutation, a.nthreads = int(mutation), int(nthreads)
    if num_drafts is not None:
        nd = _c(num_drafts, np.int32).reshape(B)
        keep.append(nd)
        a.num_drafts = _ptr(nd)
    else:
        a.num_drafts = None
    return a, B, K, V


def verify(target, draft, draft_tokens, temperature, seed=0, step=0, request_base=0,
           uniforms=None, debug=True, trace=True, mutation=0, nthreads=0, num_drafts=None):
    """Run the oracle verification.

    target: [B, K+1, V] float32 logits, or uint16 bf16 bit patterns; a leading
    dimension of 1 shares the rows across all B requests (B from draft_tokens).
    draft:  [B or 1, >=K, V] same dtype.  draft_tokens: [B, K] int.  temperature: [B].
    uniforms: optional [B, K+1, 2] override of the Philox draws.
    num_drafts: optional [B] ragged draft counts K_b <= K (bonus at row K_b).
    Returns a VerifyResult (accepted [B], tokens [B, K+1], debug_probs [B, K, 2],
    trace [B, K+1, 3] = (u_accept, threshold, u_sample), n_bad).
    """
    keep = []
    a, B, K, V = _verify_struct(target, draft, draft_tokens, temperature, seed, step, request_base,
                                uniforms, mutation, nthreads, keep, num_drafts)
    acc = np.zeros(B, np.int32)
    tok = np.zeros((B, K + 1), np.int32)
    dbg = np.zeros((B, K, 2), np.float32) if debug else None
    trc = np.zeros((B, K + 1, 3), np.float64) if trace else None
    a.accepted, a.out_tokens, a.debug_probs, a.trace = _ptr(acc), _ptr(tok), _ptr(dbg), _ptr(trc)
    rc = lib().oracle_verify(ctypes.byref(a))
    if rc < 0:
        raise ValueError("oracle_verify rejected its arguments")
    return VerifyResult(acc, tok, dbg, trc, rc)


def sampling_weights(target, draft, draft_tokens, temperature, b, j, mutation=0, num_drafts=None):
    """The weights (and their sum) the oracle samples from at row j of request b."""
    keep = []
    a, B, K, V = _verify_struct(target, draft, draft_tokens, temperature, 0, 0, 0, None,
                                mutation, 1, keep, num_drafts)
    w = np.zeros(V, np.float64)
    W = ctypes.c_double(0.0)
    rc = lib().oracle_sampling_weights(ctypes.byref(a), int(b), int(j), _ptr(w), ctypes.byref(W))
    if rc != 0:
        raise ValueError("no sampling weights for this request/row")
    return w, W.value


# ---------------------------------------------------------------------- expand
class ExpandResult:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def expand(in_token_ids, in_positions, in_start, accepted, bonus, K, mask_id,
           target_hidden=None, mask_hidden=None, hidden_fill=None, block_table=None, block_size=0):
    """Run the oracle expansion.  target_hidden: [N_in, H] uint16 (bf16 bits);
    mask_hidden: [H] uint16.  Output rows never written keep ``hidden_fill``
    (default 0xFFFF) so tests can check that every row was written once.
    block_table: [B, max_blocks] int32 with block_size > 0 adds the KV-cache
    slot mapping (``slot_mapping``, -7 where unwritten)."""
    ids = _c(in_token_ids, np.int32)
    pos = _c(in_positions, np.int64)
    st = _c(in_start, np.int32)
    acc = _c(accepted, np.int32)
    bon = _c(bonus, np.int32)
    B = acc.shape[0]
    N_in = ids.shape[0]
    N_out = N_in + B * (K - 1)
    r = ExpandResult(
        out_token_ids=np.full(N_out, -7, np.int32), out_positions=np.full(N_out, -7, np.int64),
        rejected_mask=np.full(N_out, 7, np.uint8), masked_mask=np.full(N_out, 7, np.uint8),
        new_token_indices=np.full((B, K), -7, np.int32), hidden_map=np.full(N_in, -7, np.int32),
        out_start=np.full(B + 1, -7, np.int32), out_hidden=None, n_bad=0, slot_mapping=None)
    a = ExpandArgs()
    a.B, a.K, a.N_in, a.mask_id = B, int(K), N_in, int(mask_id)
    a.in_token_ids, a.in_positions, a.in_start, a.accepted, a.bonus = (
        _ptr(ids), _ptr(pos), _ptr(st), _ptr(acc), _ptr(bon))
    keep = []
    if target_hidden is not None:
        th = _c(target_hidden, np.uint16)
        mh = _c(mask_hidden, np.uint16)
        H = th.shape[1]
        fill = 0xFFFF if hidden_fill is None else hidden_fill
        r.out_hidden = np.full((N_out, H), fill, np.uint16)
        keep += [th, mh]
        a.H, a.target_hidden, a.hidden_row_stride, a.mask_hidden = H, _ptr(th), H, _ptr(mh)
        a.out_hidden = _ptr(r.out_hidden)
    else:
        a.H, a.target_hidden, a.hidden_row_stride, a.mask_hidden, a.out_hidden = 0, None, 0, None, None
    if block_table is not None:
        bt = _c(block_table, np.int32)
        keep.append(bt)
        r.slot_mapping = np.full(N_out, -7, np.int64)
        a.block_table, a.bt_row_stride, a.max_blocks, a.block_size = _ptr(bt), bt.shape[1], bt.shape[1], int(block_size)
        a.slot_mapping = _ptr(r.slot_mapping)
    else:
        a.block_table, a.bt_row_stride, a.max_blocks, a.block_size, a.slot_mapping = None, 0, 0, 0, None
    a.out_token_ids, a.out_positions = _ptr(r.out_token_ids), _ptr(r.out_positions)
    a.rejected_mask, a.masked_mask = _ptr(r.rejected_mask), _ptr(r.masked_mask)
    a.new_token_indices, a.hidden_map, a.out_start = (
        _ptr(r.new_token_indices), _ptr(r.hidden_map), _ptr(r.out_start))
    rc = lib().oracle_expand(ctypes.byref(a))
    if rc < 0:
        raise ValueError("oracle_expand rejected its arguments (%d)" % rc)
    r.n_bad = rc
    return r


# ---------------------------------------------------------------- draft sampling
class DraftResult:
    def __init__(self, tokens, trace, n_bad):
        self.tokens = tokens
        self.trace = trace
        self.n_bad = n_bad


def draft_uniform(seed, step, request, position):
    u = ctypes.c_double(0.0)
    lib().oracle_draft_uniform(int(seed) & (2**64 - 1), int(step) & 0xFFFFFFFF, int(request), int(position),
                               ctypes.byref(u))
    return u.value


def draft_uniforms(seed, step, requests, positions):
    """draft_uniform for arrays of (global request, position) pairs."""
    r = _c(np.asarray(requests, dtype=np.int64) & 0xFFFFFFFF, np.uint32)
    k = _c(np.asarray(positions, dtype=np.int64) & 0xFFFFFFFF, np.uint32)
    if r.shape != k.shape:
        raise ValueError("requests and positions must have one shape")
    u = np.zeros(r.shape, np.float64)
    lib().oracle_draft_uniforms_many(int(seed) & (2**64 - 1), int(step) & 0xFFFFFFFF, _ptr(r), _ptr(k), r.size,
                                     _ptr(u))
    return u


def verify_uniforms(seed, step, requests, rows):
    """The verification's two uniforms (accept test, sampling draw) of each
    (global request, row) pair: arrays (u_accept, u_sample)."""
    r = _c(np.asarray(requests, dtype=np.int64) & 0xFFFFFFFF, np.uint32)
    k = _c(np.asarray(rows, dtype=np.int64) & 0xFFFFFFFF, np.uint32)
    if r.shape != k.shape:
        raise ValueError("requests and rows must have one shape")
    ua = np.zeros(r.shape, np.float64)
    us = np.zeros(r.shape, np.float64)
    lib().oracle_verify_uniforms_many(int(seed) & (2**64 - 1), int(step) & 0xFFFFFFFF, _ptr(r), _ptr(k), r.size,
                                      _ptr(ua), _ptr(us))
    return ua, us


def draft_sample(logits, row_index, temperature, seed=0, step=0, request_base=0, mutation=0):
    """Draft tokens sampled at rows row_index [B, K] of logits [N, V] (float32,
    or uint16 bf16 bit patterns).  Returns a DraftResult (tokens [B, K],
    trace [B, K] = the uniform of each draw, n_bad)."""
    lg, dt = _logit_buffer(logits)
    if lg.ndim != 2:
        raise ValueError("logits must be [N, V]")
    ri = _c(row_index, np.int32)
    B, K = ri.shape
    T = _c(temperature, np.float32).reshape(B)
    tok = np.zeros((B, K), np.int32)
    trc = np.zeros((B, K), np.float64)
    a = DraftArgs()
    a.B, a.K, a.V, a.N, a.dtype = B, K, lg.shape[1], lg.shape[0], dt
    a.logits, a.row_stride, a.row_index, a.temperature = _ptr(lg), lg.shape[1], _ptr(ri), _ptr(T)
    a.seed, a.step, a.request_base = int(seed) & (2**64 - 1), int(step) & 0xFFFFFFFF, int(request_base)
    a.tokens, a.trace, a.mutation = _ptr(tok), _ptr(trc), int(mutation)
    rc = lib().oracle_draft_sample(ctypes.byref(a))
    if rc < 0:
        raise ValueError("oracle_draft_sample rejected its arguments")
    return DraftResult(tok, trc, rc)
