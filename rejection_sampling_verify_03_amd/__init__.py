"""Python binding of ``libspecverify.so``: the C ABI in ``include/spec_verify.h``.

Argument marshalling only.  Every step of verification and expansion runs in
the library's HIP kernels; torch supplies device memory and the stream.  There
is no fallback: if the library has not been built (``build.py``) importing the
binding raises.

Same names as the C ABI: ``spec_verify_workspace_bytes``,
``spec_verify_launch``, ``spec_expand_launch``, ``spec_status_string``; plus two convenience wrappers, ``verify`` and
``expand``, that allocate the outputs and call the launchers on torch's current
stream.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libspecverify.so")

SPEC_OK, SPEC_EINVAL, SPEC_EDTYPE, SPEC_EALIGN, SPEC_EWORKSPACE, SPEC_ELAUNCH = 0, -1, -2, -3, -4, -5
SPEC_F32, SPEC_BF16 = 0, 1
SPEC_MAX_K = 63
SPEC_MAX_V = 2147418112  # 2^31 - 2^16
SPEC_NOALLOC_SCRATCH_BYTES = 16 << 20
SPEC_PHASES_DYNAMIC = 1  # phase_starts value: decisions inside the row pass (dynamic early exit)

EXPORTED = ("spec_verify_workspace_bytes", "spec_verify_plan_phases", "spec_verify_phase_cost",
            "spec_verify_launch", "spec_verify_launch_noalloc",
            "spec_expand_launch", "spec_expand_hidden_launch", "spec_verify_expand_launch",
            "spec_draft_workspace_bytes",
            "spec_draft_sample_launch", "spec_shard_workspace_bytes", "spec_shard_stats_launch",
            "spec_shard_phase_launch", "spec_shard_decide_launch", "spec_shard_draw_launch",
            "spec_workspace_error", "spec_status_string")


class SpecVerifyArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("target_logits", ctypes.c_void_p), ("t_req_stride", ctypes.c_int64), ("t_row_stride", ctypes.c_int64),
        ("draft_logits", ctypes.c_void_p), ("d_req_stride", ctypes.c_int64), ("d_row_stride", ctypes.c_int64),
        ("draft_tokens", ctypes.c_void_p), ("temperature", ctypes.c_void_p),
        ("seed", ctypes.c_uint64), ("step", ctypes.c_uint32), ("request_base", ctypes.c_uint32),
        ("accepted_counts", ctypes.c_void_p), ("output_tokens", ctypes.c_void_p),
        ("debug_probs", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("phase_event", ctypes.c_void_p), ("phase_starts", ctypes.c_uint64),
        ("draft_row_index", ctypes.c_void_p), ("draft_rows", ctypes.c_int32),
        ("num_drafts", ctypes.c_void_p), ("draft_stats", ctypes.c_void_p),
    ]


class SpecExpandArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("H", ctypes.c_int32), ("N_in", ctypes.c_int32),
        ("in_token_ids", ctypes.c_void_p), ("in_positions", ctypes.c_void_p), ("in_start", ctypes.c_void_p),
        ("accepted_counts", ctypes.c_void_p), ("bonus_tokens", ctypes.c_void_p),
        ("verify_output_tokens", ctypes.c_void_p),
        ("mask_token_id", ctypes.c_int32),
        ("target_hidden", ctypes.c_void_p), ("hidden_row_stride", ctypes.c_int64),
        ("mask_hidden", ctypes.c_void_p),
        ("out_token_ids", ctypes.c_void_p), ("out_positions", ctypes.c_void_p),
        ("rejected_mask", ctypes.c_void_p), ("masked_mask", ctypes.c_void_p),
        ("new_token_indices", ctypes.c_void_p), ("hidden_map", ctypes.c_void_p),
        ("out_start", ctypes.c_void_p), ("out_hidden", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("bt_row_stride", ctypes.c_int64),
        ("max_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32), ("slot_mapping", ctypes.c_void_p),
    ]


class SpecDraftArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("N", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("logits", ctypes.c_void_p), ("row_stride", ctypes.c_int64),
        ("row_index", ctypes.c_void_p), ("temperature", ctypes.c_void_p),
        ("seed", ctypes.c_uint64), ("step", ctypes.c_uint32), ("request_base", ctypes.c_uint32),
        ("tokens", ctypes.c_void_p), ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("stats_out", ctypes.c_void_p),
    ]


DRAFT_STATS_BYTES = 16  # one record per (request, position)


class SpecShardArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("G", ctypes.c_int32), ("g", ctypes.c_int32), ("v0", ctypes.c_int32), ("Vs", ctypes.c_int32),
        ("target_logits", ctypes.c_void_p), ("t_req_stride", ctypes.c_int64), ("t_row_stride", ctypes.c_int64),
        ("draft_logits", ctypes.c_void_p), ("d_req_stride", ctypes.c_int64), ("d_row_stride", ctypes.c_int64),
        ("draft_tokens", ctypes.c_void_p), ("temperature", ctypes.c_void_p),
        ("seed", ctypes.c_uint64), ("step", ctypes.c_uint32), ("request_base", ctypes.c_uint32),
        ("records", ctypes.c_void_p), ("masses", ctypes.c_void_p),
        ("accepted_counts", ctypes.c_void_p), ("output_tokens", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("num_drafts", ctypes.c_void_p), ("draft_row_index", ctypes.c_void_p), ("draft_rows", ctypes.c_int32),
        ("phase_starts", ctypes.c_uint64), ("phase", ctypes.c_int32),
    ]


def _load():
    # torch ships its own HIP runtime under the same SONAME as the system one;
    # loading torch first makes this library bind to that single runtime
    # instead of pulling in a second copy.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libspecverify.so is not built (expected at %s); run rejection_sampling_verify_03_amd/build.py "
            "or __graft_entry__.build()" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    L.spec_verify_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    L.spec_verify_workspace_bytes.restype = ctypes.c_size_t
    L.spec_verify_plan_phases.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_double), ctypes.c_double,
                                          ctypes.c_double]
    L.spec_verify_plan_phases.restype = ctypes.c_uint64
    L.spec_verify_phase_cost.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    L.spec_verify_phase_cost.restype = ctypes.c_double
    L.spec_verify_launch.argtypes = [ctypes.POINTER(SpecVerifyArgs), ctypes.c_void_p]
    L.spec_verify_launch.restype = ctypes.c_int
    L.spec_verify_launch_noalloc.argtypes = [ctypes.POINTER(SpecVerifyArgs), ctypes.c_void_p]
    L.spec_verify_launch_noalloc.restype = ctypes.c_int
    L.spec_workspace_error.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    L.spec_workspace_error.restype = ctypes.c_int
    L.spec_expand_launch.argtypes = [ctypes.POINTER(SpecExpandArgs), ctypes.c_void_p]
    L.spec_expand_launch.restype = ctypes.c_int
    L.spec_verify_expand_launch.argtypes = [ctypes.POINTER(SpecVerifyArgs), ctypes.POINTER(SpecExpandArgs),
                                            ctypes.c_void_p]
    L.spec_verify_expand_launch.restype = ctypes.c_int
    L.spec_expand_hidden_launch.argtypes = [ctypes.POINTER(SpecExpandArgs), ctypes.c_void_p]
    L.spec_expand_hidden_launch.restype = ctypes.c_int
    L.spec_draft_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    L.spec_draft_workspace_bytes.restype = ctypes.c_size_t
    L.spec_draft_sample_launch.argtypes = [ctypes.POINTER(SpecDraftArgs), ctypes.c_void_p]
    L.spec_draft_sample_launch.restype = ctypes.c_int
    L.spec_shard_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    L.spec_shard_workspace_bytes.restype = ctypes.c_size_t
    for name in ("spec_shard_stats_launch", "spec_shard_phase_launch", "spec_shard_decide_launch",
                 "spec_shard_draw_launch"):
        getattr(L, name).argtypes = [ctypes.POINTER(SpecShardArgs), ctypes.c_void_p]
        getattr(L, name).restype = ctypes.c_int
    L.spec_status_string.argtypes = [ctypes.c_int]
    L.spec_status_string.restype = ctypes.c_char_p
    return L


lib = _load()


class SpecError(RuntimeError):
    def __init__(self, status):
        super().__init__(spec_status_string(status))
        self.status = status


# ----------------------------------------------------------------- raw C ABI
def spec_verify_workspace_bytes(B, K, V):
    return int(lib.spec_verify_workspace_bytes(int(B), int(K), int(V)))


def spec_verify_plan_phases(K, survival, sampled_fraction, phase_cost):
    """survival: K+1 floats, survival[k] = probability that a request reaches
    draft position k.  Returns the phase_starts bit mask (0 = one pass)."""
    arr = (ctypes.c_double * (int(K) + 1))(*[float(v) for v in survival])
    return int(lib.spec_verify_plan_phases(int(K), arr, float(sampled_fraction), float(phase_cost)))


def spec_verify_phase_cost(B, K, V, dtype=SPEC_BF16):
    """The price of one early-exit phase boundary for a batch of this shape,
    in row-units (the planner's unit); -1 for an invalid shape."""
    return float(lib.spec_verify_phase_cost(int(B), int(K), int(V), int(dtype)))


def plan_phases(B, K, V, survival, sampled_fraction, dtype=SPEC_BF16):
    """The phase_starts mask the planner picks for this batch shape and
    acceptance curve, with the boundary priced by spec_verify_phase_cost."""
    return spec_verify_plan_phases(K, survival, sampled_fraction, spec_verify_phase_cost(B, K, V, dtype))


def survival_from_accepted(accepted, K):
    """survival[k] = fraction of valid requests whose first k drafts were
    accepted, from a batch of accepted counts (any iterable of ints)."""
    a = [int(v) for v in accepted if int(v) >= 0]
    n = max(len(a), 1)
    return [sum(1 for v in a if v >= k) / n for k in range(int(K) + 1)]


def spec_verify_launch(args, stream_ptr):
    """args: a SpecVerifyArgs; stream_ptr: hipStream_t as an int (0 = null stream)."""
    return int(lib.spec_verify_launch(ctypes.byref(args), stream_ptr))


def spec_verify_launch_noalloc(args, stream_ptr):
    """The same verification with the library's own per-GPU scratch array as
    its workspace (args.workspace ignored); allocates nothing."""
    return int(lib.spec_verify_launch_noalloc(ctypes.byref(args), stream_ptr))


def spec_workspace_error(workspace, stream_ptr=0):
    """Invalid requests of the last verification on this workspace (a device
    tensor or pointer); waits for the stream.  Negative: a spec_status."""
    ptr = workspace.data_ptr() if hasattr(workspace, "data_ptr") else workspace
    return int(lib.spec_workspace_error(ptr, stream_ptr))


def spec_expand_launch(args, stream_ptr):
    return int(lib.spec_expand_launch(ctypes.byref(args), stream_ptr))


def spec_verify_expand_launch(verify_args_, expand_args_, stream_ptr):
    """The verification and the expansion of its outputs as one chained call."""
    return int(lib.spec_verify_expand_launch(ctypes.byref(verify_args_), ctypes.byref(expand_args_), stream_ptr))


def spec_expand_hidden_launch(args, stream_ptr):
    return int(lib.spec_expand_hidden_launch(ctypes.byref(args), stream_ptr))


def spec_draft_workspace_bytes(B, K, V):
    return int(lib.spec_draft_workspace_bytes(int(B), int(K), int(V)))


def spec_draft_sample_launch(args, stream_ptr):
    return int(lib.spec_draft_sample_launch(ctypes.byref(args), stream_ptr))


def spec_shard_workspace_bytes(B, K, Vs):
    return int(lib.spec_shard_workspace_bytes(int(B), int(K), int(Vs)))


def spec_shard_stats_launch(args, stream_ptr):
    return int(lib.spec_shard_stats_launch(ctypes.byref(args), stream_ptr))


def spec_shard_phase_launch(args, stream_ptr):
    return int(lib.spec_shard_phase_launch(ctypes.byref(args), stream_ptr))


def spec_shard_decide_launch(args, stream_ptr):
    return int(lib.spec_shard_decide_launch(ctypes.byref(args), stream_ptr))


def spec_shard_draw_launch(args, stream_ptr):
    return int(lib.spec_shard_draw_launch(ctypes.byref(args), stream_ptr))


def spec_status_string(status):
    return lib.spec_status_string(int(status)).decode()


# ------------------------------------------------------- torch conveniences
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _logit_dtype(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    if t.dtype == torch.float32:
        return SPEC_F32
    raise TypeError("logits must be bfloat16 or float32, got %s" % t.dtype)


def _check_dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def make_workspace(B, K, V, device="cuda"):
    """A workspace large enough for verifications of this shape (no
    initialisation needed; torch's allocations are 256-byte aligned)."""
    torch = _torch()
    n = spec_verify_workspace_bytes(B, K, V)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def verify_args(target, draft, draft_tokens, temperature, accepted, tokens, debug, workspace,
                seed=0, step=0, request_base=0, phase_event=None, phase_starts=0, draft_row_index=None,
                num_drafts=None, draft_stats=None):
    """Fill a SpecVerifyArgs from tensors (no copies).

    With draft_row_index [B, K] int32, draft is a 2-D [N, V] buffer (e.g. the
    drafter's logits) and draft row k of request b is its row
    draft_row_index[b, k].

    target [B or broadcast, K+1, V] and draft [B or broadcast, >=K, V] with a
    unit innermost stride; a request stride of 0 (expanded tensor) shares rows.
    """
    _check_dev(target, draft, draft_tokens, temperature, accepted, tokens, debug, workspace)
    B, K = draft_tokens.shape
    V = target.shape[-1]
    if target.stride(-1) != 1 or draft.stride(-1) != 1:
        raise ValueError("logits rows must be contiguous")
    if draft_tokens.dtype != _torch().int32 or not draft_tokens.is_contiguous():
        raise ValueError("draft_tokens must be contiguous int32 [B, K]")
    if temperature.dtype != _torch().float32 or not temperature.is_contiguous():
        raise ValueError("temperature must be contiguous float32 [B]")
    a = SpecVerifyArgs()
    a.B, a.K, a.V, a.dtype = B, K, V, _logit_dtype(target)
    if draft.dtype != target.dtype:
        raise TypeError("target and draft logits must share a dtype")
    a.target_logits = target.data_ptr()
    a.t_req_stride = target.stride(0) if target.shape[0] == B and B > 1 else 0
    a.t_row_stride = target.stride(1)
    a.draft_logits = draft.data_ptr()
    if draft_row_index is not None:
        _check_dev(draft_row_index)
        if draft.dim() != 2:
            raise ValueError("with a draft row table the draft logits are [N, V]")
        if draft_row_index.dtype != _torch().int32 or not draft_row_index.is_contiguous() or \
                tuple(draft_row_index.shape) != (B, K):
            raise ValueError("draft_row_index must be contiguous int32 [B, K]")
        a.d_req_stride, a.d_row_stride = 0, draft.stride(0)
        a.draft_row_index, a.draft_rows = draft_row_index.data_ptr(), draft.shape[0]
    else:
        a.d_req_stride = draft.stride(0) if draft.shape[0] == B and B > 1 else 0
        a.d_row_stride = draft.stride(1)
        a.draft_row_index, a.draft_rows = None, 0
    a.draft_tokens = draft_tokens.data_ptr()
    a.temperature = temperature.data_ptr()
    a.seed, a.step, a.request_base = int(seed) & (2 ** 64 - 1), int(step) & 0xFFFFFFFF, int(request_base)
    a.accepted_counts = accepted.data_ptr()
    a.output_tokens = tokens.data_ptr()
    a.debug_probs = debug.data_ptr() if debug is not None else None
    # workspace None: for spec_verify_launch_noalloc, which brings its own
    a.workspace = workspace.data_ptr() if workspace is not None else None
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.phase_event = phase_event
    a.phase_starts = int(phase_starts)
    if num_drafts is not None:
        _check_dev(num_drafts)
        if num_drafts.dtype != _torch().int32 or not num_drafts.is_contiguous() or num_drafts.numel() != B:
            raise ValueError("num_drafts must be contiguous int32 [B]")
        a.num_drafts = num_drafts.data_ptr()
    else:
        a.num_drafts = None
    if draft_stats is not None:
        _check_dev(draft_stats)
        if draft_stats.numel() * draft_stats.element_size() < B * K * DRAFT_STATS_BYTES:
            raise ValueError("draft_stats must hold [B, K] records of %d bytes" % DRAFT_STATS_BYTES)
        a.draft_stats = draft_stats.data_ptr()
    else:
        a.draft_stats = None
    return a


def verify(target, draft, draft_tokens, temperature, seed=0, step=0, request_base=0, debug=False,
           workspace=None, stream=None, phase_starts=0, draft_row_index=None, num_drafts=None, draft_stats=None):
    """One verification step on torch's current stream.  Returns
    (accepted_counts [B] int32, output_tokens [B, K+1] int32, debug_probs
    [B, K, 2] float32 or None)."""
    torch = _torch()
    B, K = draft_tokens.shape
    V = target.shape[-1]
    dev = target.device
    accepted = torch.empty(B, dtype=torch.int32, device=dev)
    tokens = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    dbg = torch.empty(B, K, 2, dtype=torch.float32, device=dev) if debug else None
    ws = workspace if workspace is not None else make_workspace(B, K, V, dev)
    a = verify_args(target, draft, draft_tokens, temperature, accepted, tokens, dbg, ws, seed, step,
                    request_base, phase_starts=phase_starts, draft_row_index=draft_row_index,
                    num_drafts=num_drafts, draft_stats=draft_stats)
    rc = spec_verify_launch(a, _stream_ptr(stream))
    if rc != SPEC_OK:
        raise SpecError(rc)
    return accepted, tokens, dbg


class ExpandOutputs:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def expand_outputs(B, K, N_in, H, device, with_hidden=True, with_slots=False):
    torch = _torch()
    N_out = N_in + B * (K - 1)
    return ExpandOutputs(
        slot_mapping=torch.empty(N_out, dtype=torch.int64, device=device) if with_slots else None,
        out_token_ids=torch.empty(N_out, dtype=torch.int32, device=device),
        out_positions=torch.empty(N_out, dtype=torch.int64, device=device),
        rejected_mask=torch.empty(N_out, dtype=torch.uint8, device=device),
        masked_mask=torch.empty(N_out, dtype=torch.uint8, device=device),
        new_token_indices=torch.empty(B, K, dtype=torch.int32, device=device),
        hidden_map=torch.empty(N_in, dtype=torch.int32, device=device),
        out_start=torch.empty(B + 1, dtype=torch.int32, device=device),
        out_hidden=torch.empty(N_out, H, dtype=torch.bfloat16, device=device) if with_hidden else None)


def expand_args(in_token_ids, in_positions, in_start, accepted, bonus, K, mask_id, target_hidden,
                mask_hidden, out, verify_tokens=None, block_table=None, block_size=0):
    """bonus: [B] int32, or None with verify_tokens = the [B, K+1] output
    tokens of a verification (the bonus is then read at the accepted count).
    block_table: [B, max_blocks] int32 (row stride free, unit column stride)
    with block_size, when out.slot_mapping is given."""
    torch = _torch()
    _check_dev(in_token_ids, in_positions, in_start, accepted, bonus, target_hidden, mask_hidden)
    for t, dt in ((in_token_ids, torch.int32), (in_positions, torch.int64), (in_start, torch.int32),
                  (accepted, torch.int32), (bonus, torch.int32), (verify_tokens, torch.int32)):
        if t is not None and (t.dtype != dt or not t.is_contiguous()):
            raise ValueError("expected contiguous %s" % dt)
    a = SpecExpandArgs()
    B = accepted.shape[0]
    a.B, a.K, a.N_in, a.mask_token_id = B, int(K), in_token_ids.shape[0], int(mask_id)
    a.in_token_ids, a.in_positions, a.in_start = (in_token_ids.data_ptr(), in_positions.data_ptr(),
                                                   in_start.data_ptr())
    a.accepted_counts = accepted.data_ptr()
    a.bonus_tokens = bonus.data_ptr() if bonus is not None else None
    a.verify_output_tokens = verify_tokens.data_ptr() if verify_tokens is not None else None
    if out.out_hidden is not None:
        if target_hidden.dtype != torch.bfloat16 or target_hidden.stride(-1) != 1:
            raise ValueError("target_hidden must be bfloat16 with contiguous rows")
        a.H = target_hidden.shape[1]
        a.target_hidden = target_hidden.data_ptr()
        a.hidden_row_stride = target_hidden.stride(0)
        a.mask_hidden = mask_hidden.contiguous().data_ptr()
        a.out_hidden = out.out_hidden.data_ptr()
    else:
        a.H, a.target_hidden, a.hidden_row_stride, a.mask_hidden, a.out_hidden = 0, None, 0, None, None
    if getattr(out, "slot_mapping", None) is not None:
        if block_table is None or block_table.dtype != torch.int32 or block_table.stride(-1) != 1:
            raise ValueError("slot mapping needs an int32 block table with unit column stride")
        _check_dev(block_table)
        a.block_table = block_table.data_ptr()
        a.bt_row_stride = block_table.stride(0)
        a.max_blocks = block_table.shape[1]
        a.block_size = int(block_size)
        a.slot_mapping = out.slot_mapping.data_ptr()
    else:
        a.block_table, a.bt_row_stride, a.max_blocks, a.block_size, a.slot_mapping = None, 0, 0, 0, None
    a.out_token_ids, a.out_positions = out.out_token_ids.data_ptr(), out.out_positions.data_ptr()
    a.rejected_mask, a.masked_mask = out.rejected_mask.data_ptr(), out.masked_mask.data_ptr()
    a.new_token_indices, a.hidden_map = out.new_token_indices.data_ptr(), out.hidden_map.data_ptr()
    a.out_start = out.out_start.data_ptr()
    return a


def expand(in_token_ids, in_positions, in_start, accepted, bonus, K, mask_id, target_hidden=None,
           mask_hidden=None, stream=None, out=None, verify_tokens=None, block_table=None, block_size=0):
    """One expansion on torch's current stream; returns an ExpandOutputs
    (with slot_mapping when a block table is given)."""
    B = accepted.shape[0]
    H = target_hidden.shape[1] if target_hidden is not None else 0
    if out is None:
        out = expand_outputs(B, K, in_token_ids.shape[0], H, accepted.device,
                             with_hidden=target_hidden is not None, with_slots=block_table is not None)
    a = expand_args(in_token_ids, in_positions, in_start, accepted, bonus, K, mask_id, target_hidden,
                    mask_hidden, out, verify_tokens, block_table=block_table, block_size=block_size)
    rc = spec_expand_launch(a, _stream_ptr(stream))
    if rc != SPEC_OK:
        raise SpecError(rc)
    return out


# ------------------------------------------------------------ draft sampling
def draft_args(logits, row_index, temperature, tokens, workspace, seed=0, step=0, request_base=0, stats_out=None):
    """Fill a SpecDraftArgs: logits [N, V] (unit column stride), row_index
    [B, K] int32, temperature [B] float32, tokens [B, K] int32 out."""
    torch = _torch()
    _check_dev(logits, row_index, temperature, tokens, workspace)
    if logits.dim() != 2 or logits.stride(-1) != 1:
        raise ValueError("logits must be [N, V] with contiguous rows")
    for t, dt in ((row_index, torch.int32), (temperature, torch.float32), (tokens, torch.int32)):
        if t.dtype != dt or not t.is_contiguous():
            raise ValueError("expected contiguous %s" % dt)
    a = SpecDraftArgs()
    B, K = row_index.shape
    a.B, a.K, a.V, a.N, a.dtype = B, K, logits.shape[1], logits.shape[0], _logit_dtype(logits)
    a.logits, a.row_stride = logits.data_ptr(), logits.stride(0)
    a.row_index, a.temperature, a.tokens = row_index.data_ptr(), temperature.data_ptr(), tokens.data_ptr()
    a.seed, a.step, a.request_base = int(seed) & (2 ** 64 - 1), int(step) & 0xFFFFFFFF, int(request_base)
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    if stats_out is not None:
        _check_dev(stats_out)
        if stats_out.numel() * stats_out.element_size() < B * K * DRAFT_STATS_BYTES:
            raise ValueError("stats_out must hold [B, K] records of %d bytes" % DRAFT_STATS_BYTES)
        a.stats_out = stats_out.data_ptr()
    else:
        a.stats_out = None
    return a


def draft_stats_buffer(B, K, device="cuda"):
    """Device memory for the [B, K] draft statistics records."""
    return _torch().empty(B * K * DRAFT_STATS_BYTES, dtype=_torch().uint8, device=device)


def draft_sample(logits, row_index, temperature, seed=0, step=0, request_base=0, workspace=None, stream=None,
                 stats_out=None):
    """Draft tokens [B, K] int32 sampled at rows row_index of logits, on
    torch's current stream (and, with stats_out, the rows' statistics for
    the verification of these tokens)."""
    torch = _torch()
    B, K = row_index.shape
    dev = logits.device
    tokens = torch.empty(B, K, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(spec_draft_workspace_bytes(B, K, logits.shape[1]), 16), dtype=torch.uint8,
                                device=dev)
    a = draft_args(logits, row_index, temperature, tokens, workspace, seed, step, request_base, stats_out)
    rc = spec_draft_sample_launch(a, _stream_ptr(stream))
    if rc != SPEC_OK:
        raise SpecError(rc)
    return tokens


# ---------------------------------------------------- vocab-sharded verify
SHARD_RECORD_BYTES = 32


def phase_count(K, phase_starts):
    """Phases of a phase_starts cut of positions 0..K (1 for one pass)."""
    return 1 + sum(1 for k in range(1, int(K) + 1) if (int(phase_starts) >> k) & 1)


class ShardSetup:
    """Argument blocks of the G shards of one vocab-sharded verification and
    the arrays they exchange (records, masses) and write (per-shard accepted
    counts [G, B], output tokens [G, B, K+1])."""

    def __init__(self, shards, records, masses, acc, tok, stream_ptr, phases=1):
        self.shards, self.records, self.masses = shards, records, masses
        self.acc, self.tok, self.stream_ptr = acc, tok, stream_ptr
        self.phases = phases

    def launch(self, stage, h, phase=0):
        """Enqueue stage 0 (statistics of a phase), 1 (decisions), 2 (draw)
        or 3 (the accept tests of a phase before the last) of shard h."""
        launch = (spec_shard_stats_launch, spec_shard_decide_launch, spec_shard_draw_launch,
                  spec_shard_phase_launch)[stage]
        a = self.shards[h][0]
        a.phase = int(phase)
        rc = launch(a, self.stream_ptr)
        if rc != SPEC_OK:
            raise SpecError(rc)

    def schedule(self):
        """The (stage, phase) launches of one verification in order; each is
        run on every shard before the next (an exchange between them)."""
        out = []
        for p in range(self.phases):
            out.append((0, p))
            if p + 1 < self.phases:
                out.append((3, p))
        return out + [(1, 0), (2, 0)]

    def run(self):
        """Every stage of every shard, in stage order (the exchanges between
        stages are the shared arrays)."""
        for stage, p in self.schedule():
            for h in range(len(self.shards)):
                self.launch(stage, h, p)


def shard_setup(target, draft, draft_tokens, temperature, G, seed=0, step=0, request_base=0, bounds=None,
                stream=None, phase_starts=0, num_drafts=None, draft_row_index=None):
    """The argument blocks of a verification with the vocabulary split over G
    shards (bounds: G+1 slice boundaries, default as equal as possible), each
    shard reading only its slice of the logits, with their workspaces and
    exchange arrays allocated here.  With draft_row_index [B, K] int32, draft
    is a 2-D [N, V] buffer of draft rows (each shard reads its slice of
    them); num_drafts [B] int32: ragged draft counts; phase_starts: early
    exit as for verify()."""
    torch = _torch()
    B, K = draft_tokens.shape
    V = target.shape[-1]
    dev = target.device
    if bounds is None:
        bounds = [(V * h) // G for h in range(G + 1)]
    if len(bounds) != G + 1 or bounds[0] != 0 or bounds[-1] != V:
        raise ValueError("bounds must run from 0 to V in G steps")
    R = 2 * K + 1
    records = torch.empty(G * B * R * SHARD_RECORD_BYTES, dtype=torch.uint8, device=dev)
    masses = torch.empty(G * B * 2, dtype=torch.float64, device=dev)
    acc = torch.empty(G, B, dtype=torch.int32, device=dev)
    tok = torch.empty(G, B, K + 1, dtype=torch.int32, device=dev)
    shards = []
    for h in range(G):
        v0, v1 = bounds[h], bounds[h + 1]
        ws = torch.empty(max(spec_shard_workspace_bytes(B, K, v1 - v0), 16), dtype=torch.uint8, device=dev)
        t, d = target[..., v0:v1], draft[..., v0:v1]
        a = SpecShardArgs()
        a.B, a.K, a.V, a.dtype, a.G, a.g, a.v0, a.Vs = B, K, V, _logit_dtype(target), G, h, v0, v1 - v0
        a.target_logits = t.data_ptr()
        a.t_req_stride = target.stride(0) if target.shape[0] == B and B > 1 else 0
        a.t_row_stride = target.stride(1)
        a.draft_logits = d.data_ptr()
        a.d_req_stride = draft.stride(0) if draft.shape[0] == B and B > 1 else 0
        a.d_row_stride = draft.stride(1)
        a.draft_tokens, a.temperature = draft_tokens.data_ptr(), temperature.data_ptr()
        a.seed, a.step, a.request_base = int(seed) & (2 ** 64 - 1), int(step) & 0xFFFFFFFF, int(request_base)
        a.records, a.masses = records.data_ptr(), masses.data_ptr()
        a.accepted_counts, a.output_tokens = acc[h].data_ptr(), tok[h].data_ptr()
        a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
        if draft_row_index is not None:
            a.d_req_stride, a.d_row_stride = 0, draft.stride(0)
            a.draft_row_index, a.draft_rows = draft_row_index.data_ptr(), draft.shape[0]
        else:
            a.draft_row_index, a.draft_rows = None, 0
        a.num_drafts = num_drafts.data_ptr() if num_drafts is not None else None
        a.phase_starts, a.phase = int(phase_starts), 0
        shards.append((a, ws))
    return ShardSetup(shards, records, masses, acc, tok, _stream_ptr(stream), phase_count(K, phase_starts))


def verify_sharded(target, draft, draft_tokens, temperature, G, seed=0, step=0, request_base=0, bounds=None,
                   stream=None, phase_starts=0, num_drafts=None, draft_row_index=None):
    """The verification with the vocabulary split over G shards, each stage of
    each shard launched through the C ABI on one GPU; the exchanges between
    shards are the shared record and mass arrays, and the last one (the
    sampled token, -1 on every shard but its owner) an element-wise maximum.
    bounds: G+1 slice boundaries (default: as equal as possible).  Returns
    (accepted [B], output_tokens [B, K+1], per-shard accepted counts [G, B])."""
    st = shard_setup(target, draft, draft_tokens, temperature, G, seed=seed, step=step, request_base=request_base,
                     bounds=bounds, stream=stream, phase_starts=phase_starts, num_drafts=num_drafts,
                     draft_row_index=draft_row_index)
    st.run()
    return st.acc[0].clone(), st.tok.max(dim=0).values, st.acc
