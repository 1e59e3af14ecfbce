"""The C-ABI library loads, exports every entry point its header declares, and
rejects bad arguments synchronously (no GPU work is enqueued by these calls)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


@pytest.fixture(scope="module")
def sv():
    lib = os.path.join(ROOT, "rejection_sampling_verify_03_amd", "libspecverify.so")
    if not os.path.exists(lib):
        subprocess.run(["python", os.path.join(ROOT, "rejection_sampling_verify_03_amd", "build.py"), "-q"],
                       check=True)
    import rejection_sampling_verify_03_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(spec_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    assert {"spec_verify_launch", "spec_expand_launch"} <= set(fns)


def test_every_declared_symbol_is_exported(sv):
    L = ctypes.CDLL(sv.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(sv.EXPORTED) == set(declared_functions())


def test_struct_layouts_match_the_header(sv, tmp_path):
    """Every field offset and struct size of the binding's ctypes mirrors
    equals what a C compiler makes of include/spec_verify.h."""
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "spec_verify.h"', 'int main(void) {']
    for cname, py in (("spec_verify_args", sv.SpecVerifyArgs), ("spec_expand_args", sv.SpecExpandArgs),
                      ("spec_draft_args", sv.SpecDraftArgs), ("spec_shard_args", sv.SpecShardArgs)):
        lines.append('printf("%s size %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in py._fields_:
            lines.append('printf("%s %s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in (("spec_verify_args", sv.SpecVerifyArgs), ("spec_expand_args", sv.SpecExpandArgs),
                      ("spec_draft_args", sv.SpecDraftArgs), ("spec_shard_args", sv.SpecShardArgs)):
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_workspace_sizing(sv):
    assert sv.spec_verify_workspace_bytes(0, 1, 1) > 0 or sv.spec_verify_workspace_bytes(0, 1, 1) == 0
    assert sv.spec_verify_workspace_bytes(4, 0, 10) == 0
    assert sv.spec_verify_workspace_bytes(4, 64, 10) == 0
    assert sv.spec_verify_workspace_bytes(4, 4, 0) == 0
    assert sv.spec_verify_workspace_bytes(4, 4, sv.SPEC_MAX_V + 1) == 0
    assert sv.spec_verify_workspace_bytes(1, 1, sv.SPEC_MAX_V) > 0
    small = sv.spec_verify_workspace_bytes(4, 4, 1024)
    big = sv.spec_verify_workspace_bytes(256, 8, 151936)
    assert 0 < small < big
    assert big % 256 == 0
    # grows with every dimension
    assert sv.spec_verify_workspace_bytes(257, 8, 151936) > big
    assert sv.spec_verify_workspace_bytes(256, 9, 151936) > big
    assert sv.spec_verify_workspace_bytes(256, 8, 200000) > big


def _valid_verify_args(sv, B=2, K=3, V=64):
    a = sv.SpecVerifyArgs()
    a.B, a.K, a.V, a.dtype = B, K, V, sv.SPEC_BF16
    fake = 0x10000  # never dereferenced: every call below fails validation first
    a.target_logits, a.t_req_stride, a.t_row_stride = fake, (K + 1) * V, V
    a.draft_logits, a.d_req_stride, a.d_row_stride = fake, (K + 1) * V, V
    a.draft_tokens = a.temperature = a.accepted_counts = a.output_tokens = fake
    a.workspace = fake
    a.workspace_bytes = 0  # too small on purpose
    return a


def test_verify_argument_errors(sv):
    launch = lambda a: sv.spec_verify_launch(a, None)
    a = _valid_verify_args(sv)
    assert launch(a) == sv.SPEC_EWORKSPACE
    for field, value, want in [("K", 0, sv.SPEC_EINVAL), ("K", 64, sv.SPEC_EINVAL), ("V", 0, sv.SPEC_EINVAL),
                               ("B", -1, sv.SPEC_EINVAL), ("dtype", 5, sv.SPEC_EDTYPE),
                               ("V", sv.SPEC_MAX_V + 1, sv.SPEC_EINVAL),
                               ("t_row_stride", 63, sv.SPEC_EINVAL), ("d_row_stride", 10, sv.SPEC_EINVAL),
                               ("t_req_stride", 64, sv.SPEC_EINVAL), ("d_req_stride", 5, sv.SPEC_EINVAL),
                               ("target_logits", None, sv.SPEC_EINVAL), ("draft_tokens", None, sv.SPEC_EINVAL),
                               ("temperature", None, sv.SPEC_EINVAL), ("workspace", None, sv.SPEC_EINVAL),
                               ("output_tokens", None, sv.SPEC_EINVAL), ("workspace", 0x10008, sv.SPEC_EALIGN),
                               ("draft_stats", 0x10008, sv.SPEC_EALIGN), ("draft_stats", 0x10010, sv.SPEC_EWORKSPACE)]:
        a = _valid_verify_args(sv)
        setattr(a, field, value)
        assert launch(a) == want, (field, value)
    # early-exit phases: bit 0 with another bit, or a bit above K, is rejected (K = 3 here); bits
    # 1..K pass validation, and so does bit 0 alone (the dynamic early exit)
    for mask, want in [(3, sv.SPEC_EINVAL), (1 | (1 << 2), sv.SPEC_EINVAL), (1 << 4, sv.SPEC_EINVAL),
                       (1 << 63, sv.SPEC_EINVAL), ((1 << 1) | (1 << 3), sv.SPEC_EWORKSPACE),
                       (sv.SPEC_PHASES_DYNAMIC, sv.SPEC_EWORKSPACE)]:
        a = _valid_verify_args(sv)
        a.phase_starts = mask
        assert launch(a) == want, mask
    # a draft row table: its row count must not be negative, and the request stride is unused
    a = _valid_verify_args(sv)
    a.draft_row_index, a.draft_rows = 0x10000, -1
    assert launch(a) == sv.SPEC_EINVAL
    a = _valid_verify_args(sv)
    a.draft_row_index, a.draft_rows, a.d_req_stride = 0x10000, 10, 5
    assert launch(a) == sv.SPEC_EWORKSPACE
    # request stride 0 (shared rows) is accepted by validation
    a = _valid_verify_args(sv)
    a.t_req_stride = a.d_req_stride = 0
    assert launch(a) == sv.SPEC_EWORKSPACE
    # a batch whose grids exceed one dispatch (2^32 work-items): refused before anything is enqueued,
    # with every other check passed (the workspace size included)
    for B, K, V, dyn in [(1_000_000, 8, 151936, False), (9_000_000, 1, 8, False), (300_000, 8, 151936, True)]:
        a = _valid_verify_args(sv, B=B, K=K, V=V)
        a.workspace_bytes = sv.spec_verify_workspace_bytes(B, K, V)
        a.phase_starts = sv.SPEC_PHASES_DYNAMIC if dyn else 0
        assert a.workspace_bytes > 0
        assert launch(a) == sv.SPEC_EINVAL, (B, K, V, dyn)
    # B = 0 is a no-op
    a = _valid_verify_args(sv)
    a.B = 0
    assert launch(a) == sv.SPEC_OK
    assert sv.lib.spec_verify_launch(None, None) == sv.SPEC_EINVAL


def test_expand_argument_errors(sv):
    fake = 0x10000

    def args():
        a = sv.SpecExpandArgs()
        a.B, a.K, a.H, a.N_in = 2, 3, 8, 8
        for f in ("in_token_ids", "in_positions", "in_start", "accepted_counts", "bonus_tokens",
                  "out_token_ids", "out_positions", "rejected_mask", "masked_mask", "new_token_indices",
                  "hidden_map", "out_start"):
            setattr(a, f, fake)
        a.out_hidden = None
        return a

    launch = lambda a: sv.spec_expand_launch(a, None)
    for field, value in [("K", 0), ("B", -1), ("H", -1), ("N_in", -1), ("in_start", None),
                         ("accepted_counts", None), ("bonus_tokens", None), ("out_start", None),
                         ("new_token_indices", None), ("in_token_ids", None)]:
        a = args()
        setattr(a, field, value)
        assert launch(a) == sv.SPEC_EINVAL, field
    a = args()
    a.verify_output_tokens = fake  # two bonus sources
    assert launch(a) == sv.SPEC_EINVAL
    a = args()
    a.out_hidden, a.target_hidden, a.mask_hidden, a.hidden_row_stride = fake, fake, fake, 4  # stride < H
    assert launch(a) == sv.SPEC_EINVAL
    a = args()
    a.out_hidden, a.target_hidden, a.mask_hidden, a.hidden_row_stride = fake, fake, None, 8
    assert launch(a) == sv.SPEC_EINVAL
    a = args()
    a.B, a.N_in, a.K = 2, 2 ** 31 - 2, 3  # N_out overflows int32
    assert launch(a) == sv.SPEC_EINVAL
    a = args()
    a.B, a.N_in, a.K = 20_000_000, 20_000_000, 1  # a workgroup per request: more work-items than one dispatch
    assert launch(a) == sv.SPEC_EINVAL
    a = args()
    a.B = 0
    assert launch(a) == sv.SPEC_OK


def test_verify_expand_argument_errors(sv):
    fake = 0x10000  # never dereferenced: every call below fails validation first
    v = _valid_verify_args(sv)
    v.workspace_bytes = 1 << 40  # passes the size check; no call below gets to the launch

    def expand_for(v):
        a = sv.SpecExpandArgs()
        a.B, a.K, a.H, a.N_in = v.B, v.K, 8, v.B * (v.K + 1)
        for f in ("in_token_ids", "in_positions", "in_start", "out_token_ids", "out_positions", "rejected_mask",
                  "masked_mask", "new_token_indices", "hidden_map", "out_start"):
            setattr(a, f, fake)
        a.accepted_counts, a.verify_output_tokens = v.accepted_counts, v.output_tokens
        a.out_hidden = None
        return a

    launch = lambda v, e: sv.lib.spec_verify_expand_launch(ctypes.byref(v), ctypes.byref(e), None)
    small = _valid_verify_args(sv)
    assert launch(small, expand_for(small)) == sv.SPEC_EWORKSPACE  # the verification's own status
    e = expand_for(v)
    e.K = v.K + 1
    assert launch(v, e) == sv.SPEC_EINVAL
    e = expand_for(v)
    e.B, e.N_in = v.B + 1, (v.B + 1) * (v.K + 1)
    assert launch(v, e) == sv.SPEC_EINVAL
    e = expand_for(v)
    e.accepted_counts = fake + 64  # not the verification's counts
    assert launch(v, e) == sv.SPEC_EINVAL
    e = expand_for(v)
    e.verify_output_tokens, e.bonus_tokens = None, fake  # bonus not from the verification
    assert launch(v, e) == sv.SPEC_EINVAL
    e = expand_for(v)
    e.out_start = None  # the expansion's own argument error
    assert launch(v, e) == sv.SPEC_EINVAL
    v0, e0 = _valid_verify_args(sv), expand_for(v)
    v0.B = e0.B = 0
    assert launch(v0, e0) == sv.SPEC_OK
    assert sv.lib.spec_verify_expand_launch(None, None, None) == sv.SPEC_EINVAL


def test_status_strings(sv):
    for code in (0, -1, -2, -3, -4, -5):
        assert sv.spec_status_string(code).startswith("SPEC_")
    assert "unknown" in sv.spec_status_string(42)


def test_workspace_error_rejects_a_null_workspace(sv):
    # rejected before any HIP call, so this runs without a GPU
    assert sv.spec_workspace_error(0, 0) == sv.SPEC_EINVAL


def test_expand_hidden_argument_errors(sv):
    fake = 0x10000
    a = sv.SpecExpandArgs()
    a.B, a.K, a.H, a.N_in = 2, 3, 8, 8
    a.in_start = a.target_hidden = a.mask_hidden = a.out_hidden = fake
    a.hidden_row_stride = 8
    launch = lambda a: sv.spec_expand_hidden_launch(a, None)
    for field, value in [("K", 0), ("B", -1), ("H", -1), ("N_in", -1), ("in_start", None), ("out_hidden", None),
                         ("mask_hidden", None), ("target_hidden", None), ("hidden_row_stride", 7)]:
        b = sv.SpecExpandArgs.from_buffer_copy(a)
        setattr(b, field, value)
        assert launch(b) == sv.SPEC_EINVAL, field
    b = sv.SpecExpandArgs.from_buffer_copy(a)
    b.H = 0  # nothing to gather
    assert launch(b) == sv.SPEC_OK
    assert sv.lib.spec_expand_hidden_launch(None, None) == sv.SPEC_EINVAL


def test_draft_argument_errors(sv):
    fake = 0x10000  # never dereferenced: every call below fails validation first

    def args():
        a = sv.SpecDraftArgs()
        a.B, a.K, a.V, a.N, a.dtype = 2, 3, 100, 8, sv.SPEC_BF16
        a.logits, a.row_stride = fake, 100
        a.row_index = a.temperature = a.tokens = a.workspace = fake
        a.workspace_bytes = 0  # too small on purpose
        return a

    launch = lambda a: sv.spec_draft_sample_launch(a, None)
    assert launch(args()) == sv.SPEC_EWORKSPACE
    for field, value, want in [("K", 0, sv.SPEC_EINVAL), ("V", 0, sv.SPEC_EINVAL), ("B", -1, sv.SPEC_EINVAL),
                               ("V", sv.SPEC_MAX_V + 1, sv.SPEC_EINVAL),
                               ("N", -1, sv.SPEC_EINVAL), ("dtype", 7, sv.SPEC_EDTYPE),
                               ("row_stride", 99, sv.SPEC_EINVAL), ("row_index", None, sv.SPEC_EINVAL),
                               ("temperature", None, sv.SPEC_EINVAL), ("tokens", None, sv.SPEC_EINVAL),
                               ("logits", None, sv.SPEC_EINVAL), ("workspace", None, sv.SPEC_EINVAL),
                               ("workspace", 0x10004, sv.SPEC_EALIGN), ("stats_out", 0x10004, sv.SPEC_EALIGN),
                               ("stats_out", 0x10010, sv.SPEC_EWORKSPACE)]:
        a = args()
        setattr(a, field, value)
        assert launch(a) == want, (field, value)
    a = args()
    a.B = 0
    assert launch(a) == sv.SPEC_OK
    # more statistics work-items than one dispatch holds, every other check passed
    a = args()
    a.B, a.K, a.V, a.row_stride = 2_000_000, 8, 151936, 151936
    a.workspace_bytes = sv.spec_draft_workspace_bytes(a.B, a.K, a.V)
    assert launch(a) == sv.SPEC_EINVAL
    assert sv.lib.spec_draft_sample_launch(None, None) == sv.SPEC_EINVAL
    # workspace: one 16-byte statistic per (request, position, 4096-logit segment), 256-byte rounded
    assert sv.spec_draft_workspace_bytes(2, 3, 100) == 256
    assert sv.spec_draft_workspace_bytes(256, 8, 151936) == 256 * 8 * 38 * 16
    assert sv.spec_draft_workspace_bytes(1, 0, 10) == 0
    assert sv.spec_draft_workspace_bytes(1, 1, sv.SPEC_MAX_V + 1) == 0


def test_shard_argument_errors(sv):
    fake = 0x10000

    def args():
        a = sv.SpecShardArgs()
        a.B, a.K, a.V, a.dtype, a.G, a.g, a.v0, a.Vs = 2, 3, 100, sv.SPEC_BF16, 2, 1, 50, 50
        a.target_logits, a.t_req_stride, a.t_row_stride = fake, 400, 100
        a.draft_logits, a.d_req_stride, a.d_row_stride = fake, 400, 100
        a.draft_tokens = a.temperature = a.records = a.masses = fake
        a.accepted_counts = a.output_tokens = a.workspace = fake
        a.workspace_bytes = 0
        return a

    for launch in (sv.spec_shard_stats_launch, sv.spec_shard_decide_launch, sv.spec_shard_draw_launch,
                   sv.spec_shard_phase_launch):
        if launch is sv.spec_shard_phase_launch:  # needs a phase that is not the last
            a = args()
            a.phase_starts = 1 << 2
            assert launch(a, None) == sv.SPEC_EWORKSPACE
            a.phase = 1
            assert launch(a, None) == sv.SPEC_EINVAL
            a.phase_starts = 0
            a.phase = 0
            assert launch(a, None) == sv.SPEC_EINVAL
            continue
        assert launch(args(), None) == sv.SPEC_EWORKSPACE
        for field, value, want in [("G", 0, sv.SPEC_EINVAL), ("g", 2, sv.SPEC_EINVAL), ("g", -1, sv.SPEC_EINVAL),
                                   ("Vs", 0, sv.SPEC_EINVAL), ("v0", 51, sv.SPEC_EINVAL), ("v0", -1, sv.SPEC_EINVAL),
                                   ("K", 64, sv.SPEC_EINVAL), ("dtype", 3, sv.SPEC_EDTYPE),
                                   ("V", sv.SPEC_MAX_V + 1, sv.SPEC_EINVAL),
                                   ("t_row_stride", 49, sv.SPEC_EINVAL), ("records", None, sv.SPEC_EINVAL),
                                   ("masses", None, sv.SPEC_EINVAL), ("workspace", 0x10008, sv.SPEC_EALIGN),
                                   ("phase_starts", 1, sv.SPEC_EINVAL), ("phase_starts", 1 << 4, sv.SPEC_EINVAL),
                                   ("phase", 1, sv.SPEC_EINVAL), ("phase", -1, sv.SPEC_EINVAL),
                                   ("draft_rows", -1, sv.SPEC_EWORKSPACE)]:
            a = args()
            setattr(a, field, value)
            assert launch(a, None) == want, (launch, field, value)
    # a draft row table with a negative row count
    a = args()
    a.draft_row_index, a.draft_rows = fake, -1
    assert sv.spec_shard_stats_launch(a, None) == sv.SPEC_EINVAL
    # more statistics work-items than one dispatch holds, every other check passed
    a = args()
    a.B, a.K, a.t_req_stride, a.d_req_stride = 200_000, 63, 64 * 100, 64 * 100
    a.workspace_bytes = sv.spec_shard_workspace_bytes(a.B, a.K, a.Vs)
    for launch in (sv.spec_shard_stats_launch, sv.spec_shard_decide_launch, sv.spec_shard_draw_launch):
        assert launch(a, None) == sv.SPEC_EINVAL
    # decision records, segment sums and the request state between phases
    assert sv.spec_shard_workspace_bytes(2, 3, 50) == 256 + 256 + 256
    assert sv.spec_shard_workspace_bytes(1, 1, sv.SPEC_MAX_V + 1) == 0
    assert sv.spec_shard_workspace_bytes(256, 8, 37984) == 256 * 64 + 256 * 10 * 16 + 256 * 4


def test_noalloc_argument_errors(sv):
    """The allocation-free entry point refuses bad shapes, and shapes whose
    workspace exceeds its scratch array, on the host before anything runs."""
    assert sv.lib.spec_verify_launch_noalloc(None, None) == sv.SPEC_EINVAL
    a = sv.SpecVerifyArgs()
    a.B, a.K, a.V, a.dtype = 4, 0, 100, sv.SPEC_BF16
    assert sv.spec_verify_launch_noalloc(a, 0) == sv.SPEC_EINVAL
    a.K = 8
    a.B, a.V = 4096, 201088
    assert sv.spec_verify_workspace_bytes(4096, 8, 201088) > sv.SPEC_NOALLOC_SCRATCH_BYTES
    assert sv.spec_verify_launch_noalloc(a, 0) == sv.SPEC_EWORKSPACE
    a.B = 0
    a.dtype = 7
    assert sv.spec_verify_launch_noalloc(a, 0) == sv.SPEC_EDTYPE
