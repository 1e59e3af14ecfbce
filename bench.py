"""Benchmark of one speculative-decoding hot-path step on one MI355X.

A step = one verification of the headline batch (B=256 requests, K=8 drafts,
V=151936 bf16 logits, temperatures drawn from {0, 0.6, 1}, mixture drafts)
followed by the P-EAGLE expansion of the same batch (hidden width 2880, the
bonus read from the verification's output tokens, KV-cache slot mapping
through a 16-slot-per-block table), enqueued through the C ABI on torch's
current stream as one chained call (spec_verify_expand_launch: the expansion
runs inside the verification's sampling stage; --separate-expand enqueues it
as its own call).  Inputs are generated once on the GPU and stay resident in
HBM; each timed step uses a new Philox step counter.

By default the verification reads its rows in early-exit phases (rows of a
phase only for requests whose earlier drafts were all accepted), cut by the
library's planner from the acceptance curve of 8 untimed one-pass steps with
the phase boundary priced for the batch shape (spec_verify_phase_cost); the
outputs are identical to one pass (--early-exit off).

Prints one JSON line: verified draft positions per second (B*K per step,
wall clock over the timed steps); the roofline of the dominant stage (the row
statistics of verification: its row-pass kernels and, with phases, the
decisions between them), timed with HIP events on the launch stream
(created without the system-scope fence, see TimingEvent) on every
--event-every-th timed step (at least 10 of them), against the logit bytes
those steps read under the plan, against the method's sequential minimum,
and -- for the row pass as one launch over every row -- against the
algorithmic bytes of the parallel formulation; and the CPU oracle timed on
the host's cores over whole steps of the same batch (and on one core).

Side measurements, outside the timed steps (each timed with HIP events):
draft-token sampling at the step's new-token indices (draft_sampling), one
GPU's share of a 4-way vocab-sharded verification of the same batch
(shard_share_tp4), a whole P-EAGLE round -- draft sampling, then the chained
verification and expansion -- with and without the sampler's row statistics
handed to the verification (peagle_round), and the other workloads (configs): the GPT-OSS vocabulary
batch (B=64, K=5, V=201088) and the expansion alone (B=512, K=8, H=2880),
each rotating over input copies that together exceed the 256 MB Infinity
Cache, and the large batch (B=1024, K=8, V=201088, acceptance ~0.8).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E

_HIP = None


def _hip_runtime():
    """The HIP runtime torch has loaded (one copy per process: its streams are
    that runtime's objects)."""
    global _HIP
    if _HIP is None:
        import ctypes
        import re
        with open("/proc/self/maps") as f:
            paths = sorted(set(re.findall(r"\S*/libamdhip64\.so\S*", f.read())))
        if len(paths) != 1:
            raise RuntimeError("expected one HIP runtime in the process, found %r" % (paths,))
        h = ctypes.CDLL(paths[0])
        h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        h.hipEventDestroy.argtypes = [ctypes.c_void_p]
        h.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        _HIP = h
    return _HIP


class TimingEvent:
    """A HIP timing event without the system-scope fence
    (hipEventDisableSystemFence).  A default timing event writes back and
    invalidates the caches when it is recorded, which costs the GPU time of its
    own: ~5 µs per headline step with a start event and the library's phase
    event (166.7 µs per step without events, 172.1 with torch's events on every
    step, 168.7-169.4 with these).  The events only time work; outputs are read
    after a device synchronisation, and each kernel's completion releases its
    writes to the next one on the device."""
    _FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        self._c = ctypes
        self._hip = _hip_runtime()
        self.h = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.h), self._FLAGS)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)
        self.cuda_event = self.h.value  # the handle the C ABI takes as hipEvent_t

    def record(self, stream):
        rc = self._hip.hipEventRecord(self.h, self._c.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def wait_on(self, stream):
        """Make `stream` wait for this event."""
        rc = self._hip.hipStreamWaitEvent(self._c.c_void_p(stream.cuda_stream), self.h, 0)
        if rc != 0:
            raise RuntimeError("hipStreamWaitEvent failed: %d" % rc)

    def elapsed_time(self, end):
        ms = self._c.c_float()
        rc = self._hip.hipEventElapsedTime(self._c.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def __del__(self):
        # at interpreter exit the runtime may already be gone: leave the event to it
        if sys.is_finalizing() or not getattr(self, "h", None) or not self.h.value:
            return
        self._hip.hipEventDestroy(self.h)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=None,
                    help="record the HIP events that time the stages on every N-th timed step only (each event "
                         "record costs GPU time of its own; 1 = every step); default: at most 8, and at least "
                         "10 timed steps with events")
    ap.add_argument("--separate-expand", action="store_true",
                    help="enqueue the expansion as its own call after the verification instead of the chained "
                         "call that runs it inside the verification's sampling stage")
    ap.add_argument("--overlap", action="store_true",
                    help="gather the expansion's hidden rows on a second stream while the verification's sampling "
                         "stage runs (measured slower: the gather competes with the segment sums for HBM)")
    ap.add_argument("--no-draft-sampling", action="store_true",
                    help="skip the separate measurement of draft-token sampling at the new-token indices")
    ap.add_argument("--no-shard-share", action="store_true",
                    help="skip the separate measurement of one GPU's share of a 4-way vocab-sharded verification")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU-seconds of oracle work for the CPU baseline")
    ap.add_argument("--early-exit", choices=("plan", "off", "dynamic"), default="plan",
                    help="plan: read rows in phases planned from the acceptance of the warmup steps; "
                         "off: one pass over every row; dynamic: decisions inside the row pass (no plan; the "
                         "rows read are not counted, so frac is left out)")
    ap.add_argument("--phase-starts", type=int, default=None,
                    help="with --early-exit plan: use this phase mask (bit k starts a phase at draft position k) "
                         "instead of the one planned from the acceptance curve")
    ap.add_argument("--only", choices=("all", "headline", "gptoss", "expand", "large"), default="all",
                    help="run only the headline step, or only one of the side workloads (for profiling runs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the side workloads (GPT-OSS vocabulary batch, expansion alone, large batch)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy 1 GiB device to device once (a plain copy kernel of known "
                         "size, to scale hardware byte counters)")
    return ap.parse_args()


def algorithmic_verify_bytes(B, K, V, es, temps):
    """Bytes the parallel formulation must read once: every target row 0..K,
    and draft rows 0..K-1 of sampled (T > 0) requests; plus draft tokens and
    temperatures in, accepted counts and output tokens out."""
    n_sampled = int((temps > 0).sum())
    logits = B * (K + 1) * V * es + n_sampled * K * V * es
    return logits + B * K * 4 + B * 4 + B * 4 + B * (K + 1) * 4


def one_pass_logit_bytes(B, K, V, es, temps):
    """Logit bytes of the row pass without early exit: every target row 0..K
    and the draft rows 0..K-1 of sampled requests."""
    return B * (K + 1) * V * es + int((temps > 0).sum()) * K * V * es


def phased_logit_bytes(acc, temps, mask, K, V, es):
    """Logit bytes the row stage reads under the phase cut `mask` (0 = one
    pass) for one step with accepted counts `acc`: a request reads the rows of
    every phase up to the one holding its stopping position (all of them when
    its data is invalid only under one pass)."""
    starts = [0] + [k for k in range(1, K + 1) if (mask >> k) & 1]
    ends = starts[1:] + [K + 1]
    total = 0
    for a, t in zip(acc, temps):
        a = K if a < 0 else int(a)
        for s, e in zip(starts, ends):
            if s > a:
                break
            total += (e - s) + ((min(e, K) - s) if t > 0 else 0)
    return total * V * es


def draft_sampling(sv, torch, np, out, temperature, B, K, V, seed, dev, reps=50):
    """Draft tokens sampled from drafter logits [N_out, V] bf16 (Zipf rows) at
    the expansion's new-token indices, timed apart from the step with HIP
    events; bytes = every sampled row once plus the one segment the draw
    re-reads for a T > 0 position."""
    import workloads
    n_out = out.out_token_ids.shape[0]
    g = workloads._gen(seed + 3, dev)
    logits = workloads.zipf_logits(n_out, V, g, dev).to(torch.bfloat16)
    tokens = torch.empty(B, K, dtype=torch.int32, device=dev)
    ws = torch.empty(sv.spec_draft_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    args = [sv.draft_args(logits, out.new_token_indices, temperature, tokens, ws, seed=seed, step=i)
            for i in range(reps)]
    for a in args[:5]:
        assert sv.spec_draft_sample_launch(a, stream.cuda_stream) == sv.SPEC_OK
    e0, e1 = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    e0.record(stream)
    for a in args:
        assert sv.spec_draft_sample_launch(a, stream.cuda_stream) == sv.SPEC_OK
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    n_sampled = int((temperature > 0).sum())
    nbytes = B * K * V * 2 + n_sampled * K * 4096 * 2
    del logits
    return {"workload": "drafter logits [%d, %d] bf16, B=%d requests x K=%d new-token indices" % (n_out, V, B, K),
            "ms": ms, "positions_per_s": B * K / (ms * 1e-3), "bytes": nbytes,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}


def shard_share(sv, torch, inp, seed, G=4, reps=50, phase_starts=0):
    """One GPU's share of a tensor-parallel verification of the headline batch
    over G vocabulary shards: shard 0's stages (statistics over its slice --
    per early-exit phase, with the phase's accept tests between phases --,
    decisions from every shard's records, draw) on its slice, held as a
    contiguous tensor as a tensor-parallel GPU would hold it, timed with HIP
    events after one run of every shard has filled the exchanged records and
    masses (the same step each rep, so the work is the same).  Bytes: the
    slice of every row the plan reads, once."""
    import numpy as np
    B, K, V = inp.B, inp.K, inp.V
    st = sv.shard_setup(inp.target, inp.draft, inp.draft_tokens, inp.temperature, G, seed=seed, step=0,
                        phase_starts=phase_starts)
    st.run()
    torch.cuda.synchronize()
    acc = st.acc[0].cpu().numpy()
    stream = torch.cuda.current_stream()
    # a tensor-parallel GPU holds its slice as a tensor of its own: shard 0
    # reads contiguous copies [B, K+1, Vs] (the same values as the view)
    a0 = st.shards[0][0]
    t0 = inp.target[..., a0.v0:a0.v0 + a0.Vs].contiguous()
    d0 = inp.draft[..., a0.v0:a0.v0 + a0.Vs].contiguous()
    a0.target_logits, a0.t_req_stride, a0.t_row_stride = t0.data_ptr(), t0.stride(0), t0.stride(1)
    a0.draft_logits, a0.d_req_stride, a0.d_row_stride = d0.data_ptr(), d0.stride(0), d0.stride(1)
    sched = st.schedule()

    def share():
        for stage, p in sched:
            st.launch(stage, 0, p)

    for _ in range(5):
        share()
    e0, e1 = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        share()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    Vs = a0.Vs
    temps = inp.temperature.cpu().numpy()
    nbytes = phased_logit_bytes(acc, temps, phase_starts, K, Vs, 2)
    del t0, d0
    return {"workload": "shard 0 of %d: its slice [%d, %d, %d] bf16 of the headline batch, contiguous%s"
                        % (G, B, K + 1, Vs, ", early-exit phases %#x" % phase_starts if phase_starts else ""),
            "launches": len(sched), "ms": ms, "positions_per_s": B * K / (ms * 1e-3), "bytes": nbytes,
            "GBps": nbytes / (ms * 1e-3) / 1e9, "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "one_pass_bytes": one_pass_logit_bytes(B, K, Vs, 2, temps)}


def sequential_logit_bytes(acc, temps, K, V, es):
    """The method's own minimum: rows 0..a of the target and, for sampled
    requests, draft rows 0..min(a, K-1)."""
    rows = sum((int(a) + 1) + (min(int(a) + 1, K) if t > 0 else 0) for a, t in zip(acc, temps) if a >= 0)
    return rows * V * es


NOMINAL_ROW_GBS = 6800.0  # the row pass's one-pass streaming rate (the planner's price unit)
PLAN_STEPS = 8  # one-pass steps whose accepted counts give the survival curve


def algorithmic_expand_bytes(B, K, H, n_in):
    """Hidden rows read and written once, metadata in and out, and the slot
    mapping (one block-table entry read and one int64 slot written per output
    slot)."""
    n_out = n_in + B * (K - 1)
    hidden = n_in * H * 2 + H * 2 + n_out * H * 2
    meta_in = n_in * (4 + 8) + (B + 1) * 4 + B * 4 + B * 4
    meta_out = n_out * (4 + 8 + 1 + 1) + B * K * 4 + n_in * 4 + (B + 1) * 4
    slots = n_out * (4 + 8)
    return hidden + meta_in + meta_out + slots


ROWPASS_SOURCES = ["rejection_sampling_verify_03_amd/csrc/verify.hip", "rejection_sampling_verify_03_amd/csrc/device_common.hpp",
                   "rejection_sampling_verify_03_amd/csrc/verify_layout.hpp",
                   "rejection_sampling_verify_03_amd/csrc/verify_kernels.hpp",
                   "rejection_sampling_verify_03_amd/csrc/rowpass.hpp",
                   "rejection_sampling_verify_03_amd/csrc/decision.hpp"]
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "verify_rowstats_traffic.md")


def rowpass_source_hash():
    """Hash of the row-pass sources as code: comments and whitespace are left
    out, so that a reworded comment does not set the committed counters
    aside."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ROWPASS_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)                # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(phase_starts):
    """HBM bytes per step of the row-statistics stage under this phase plan,
    from the committed counter summary, with the provenance: (bytes or None,
    {"summary", "source_sha256", "matches_sources"}).  The bytes are None when
    the summary holds none for the plan or the row-pass sources changed since
    those counters were taken."""
    import re
    src = rowpass_source_hash()
    prov = {"summary": os.path.relpath(TRAFFIC_SUMMARY, ROOT), "source_sha256": src, "matches_sources": False}
    try:
        text = open(TRAFFIC_SUMMARY).read()
    except OSError:
        return None, prov
    for m in re.finditer(r"traffic_bytes_per_step: (\d+) phase_starts: (\d+) source_sha256: ([0-9a-f]+)", text):
        if int(m.group(2)) == phase_starts and m.group(3) == src:
            prov["matches_sources"] = True
            return int(m.group(1)), prov
    return None, prov


def event_steps(torch, stream, launch, n):
    """Run launch(i, (start, stage_end, end) or None) for i < n twice: once
    with only an event pair around the whole loop (the step time), then with
    an event triple around every step (the stage times: row statistics, and
    the rest).  Returns (ms per step, [stage ms], [rest ms])."""
    a, b = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(n):
        launch(i, None)
    b.record(stream)
    torch.cuda.synchronize()
    ev = [[TimingEvent() for _ in range(3)] for _ in range(n)]
    for e3 in ev:  # create the underlying HIP events before the loop
        for e in e3:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(n):
        launch(i, ev[i])
    torch.cuda.synchronize()
    return (a.elapsed_time(b) / n, [e[0].elapsed_time(e[1]) for e in ev], [e[1].elapsed_time(e[2]) for e in ev])


def verify_config(sv, torch, np, name, copies, steps=20, seed=0):
    """One verification per step of a side workload through spec_verify_launch,
    rotating over `copies` (VerifyInputs with the same values in different
    buffers, so that a step's rows are not left in the Infinity Cache by the
    step before), rows read in the phases the planner picks for this shape
    from 8 one-pass steps; the one-pass timing beside it."""
    inp = copies[0]
    B, K, V = inp.B, inp.K, inp.V
    es = inp.bytes_per_logit()
    dev = inp.target.device
    temps = inp.temperature.cpu().numpy()
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ws = sv.make_workspace(B, K, V, dev)
    stream = torch.cuda.current_stream()
    args = [sv.verify_args(c.target, c.draft, c.draft_tokens, c.temperature, acc, tok, None, ws, seed=seed)
            for c in copies]
    mask = {"m": 0}

    def launch(i, ev):
        a = args[i % len(args)]
        a.step = i & 0xFFFFFFFF
        a.phase_starts = mask["m"]
        a.phase_event = ev[1].cuda_event if ev else None
        if ev:
            ev[0].record(stream)
        rc = sv.spec_verify_launch(a, stream.cuda_stream)
        if rc != sv.SPEC_OK:
            raise sv.SpecError(rc)
        if ev:
            ev[2].record(stream)

    accs = []
    for i in range(PLAN_STEPS):
        launch(5_000_000 + i, None)
        torch.cuda.synchronize()
        accs.extend(acc.cpu().tolist())
    surv = sv.survival_from_accepted(accs, K)
    frac_sampled = float((temps > 0).mean())
    cost = sv.spec_verify_phase_cost(B, K, V, sv.SPEC_BF16 if es == 2 else sv.SPEC_F32)
    planned = sv.spec_verify_plan_phases(K, surv, frac_sampled, cost)
    out = {"workload": name, "B": B, "K": K, "V": V, "dtype": "bf16" if es == 2 else "f32",
           "input_copies": len(copies), "steps": steps}
    res = {}
    dyn = sv.SPEC_PHASES_DYNAMIC
    for m in sorted({0, planned, dyn}):
        mask["m"] = m
        for i in range(3):
            launch(6_000_000 + i, None)
        ms, k1, k2 = event_steps(torch, stream, launch, steps)
        read = []
        seq = []
        for i in range(steps):  # outputs depend only on (seed, step): the rows each timed step read
            launch(i, None)
            a_np = acc.cpu().numpy()
            # the dynamic exit's rows depend on timing: no exact count (the sequential minimum bounds it)
            read.append(phased_logit_bytes(a_np, temps, m, K, V, es) if m != dyn else float("nan"))
            seq.append(sequential_logit_bytes(a_np, temps, K, V, es))
        stage = float(np.mean(k1))
        res[m] = {"ms_per_step": ms, "row_stage_ms": stage, "row_stage_p10_p90": [float(np.percentile(k1, 10)),
                                                                                   float(np.percentile(k1, 90))],
                  "sampling_stage_ms": float(np.mean(k2)), "read_bytes": float(np.mean(read)),
                  "seq_bytes": float(np.mean(seq)), "mean_accepted": float(acc.float().mean())}
    alg = one_pass_logit_bytes(B, K, V, es, temps)
    p = res[planned]
    out.update({
        "plan": {"phase_starts": planned, "phases": [0] + [k for k in range(1, K + 1) if (planned >> k) & 1],
                 "survival": [round(v, 4) for v in surv], "phase_cost_rows": round(cost, 4)},
        "ms_per_step": p["ms_per_step"], "positions_per_s": B * K / (p["ms_per_step"] * 1e-3),
        "row_stage_ms": p["row_stage_ms"], "row_stage_p10_p90": p["row_stage_p10_p90"],
        "algorithmic_bytes": alg, "plan_read_bytes": p["read_bytes"], "sequential_min_bytes": p["seq_bytes"],
        "frac": p["read_bytes"] / (p["row_stage_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "frac_seq_min": p["seq_bytes"] / (p["row_stage_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "one_pass": {"ms_per_step": res[0]["ms_per_step"], "row_stage_ms": res[0]["row_stage_ms"],
                     "frac": alg / (res[0]["row_stage_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "dynamic": {"ms_per_step": res[dyn]["ms_per_step"], "row_stage_ms": res[dyn]["row_stage_ms"],
                    "frac_seq_min": res[dyn]["seq_bytes"] / (res[dyn]["row_stage_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "positions_per_s": B * K / (res[dyn]["ms_per_step"] * 1e-3)},
        "plan_is_fastest": p["ms_per_step"] <= min(r["ms_per_step"] for r in res.values()),
        "mean_accepted": p["mean_accepted"]})
    return out


def expand_config(sv, torch, B=512, K=8, H=2880, copies=8, steps=48, seed=0):
    """spec_expand_launch alone on the expansion workload (B=512, K=8,
    H=2880, accepted counts uniform in 0..K), rotating over `copies` input and
    output buffers (~74 MB per copy); bytes: hidden rows read and written
    once, the mask row, metadata in and out."""
    import workloads
    dev = torch.device("cuda")
    e = workloads.expand_inputs(B=B, K=K, H=H, seed=seed, device=dev)
    stream = torch.cuda.current_stream()
    args = []
    keep = []
    for c in range(copies):
        th = e.target_hidden.clone()
        out = sv.expand_outputs(B, K, e.N_in, H, dev)
        keep.append((th, out))
        args.append(sv.expand_args(e.in_token_ids, e.in_positions, e.in_start, e.accepted, e.bonus, K, e.mask_id,
                                   th, e.mask_hidden, out))

    def launch(i, ev):
        if ev:
            ev[0].record(stream)
        rc = sv.spec_expand_launch(args[i % copies], stream.cuda_stream)
        if rc != sv.SPEC_OK:
            raise sv.SpecError(rc)
        if ev:
            ev[1].record(stream)
            ev[2].record(stream)

    for i in range(copies):
        launch(i, None)
    ms, k1, _ = event_steps(torch, stream, launch, steps)
    nbytes = algorithmic_expand_bytes(B, K, H, e.N_in) - (e.N_in + B * (K - 1)) * 12  # no slot mapping here
    each = float(sum(k1) / len(k1))

    # the practical ceiling of this copy-shaped traffic: a plain device-to-device copy of the output's
    # hidden bytes (torch's copy kernel, the same rotation), timed the same way
    def copy(i, ev):
        if ev:
            ev[0].record(stream)
        keep[i % copies][1].out_hidden.copy_(keep[(i + 1) % copies][1].out_hidden)
        if ev:
            ev[1].record(stream)
            ev[2].record(stream)

    for i in range(copies):
        copy(i, None)
    cms, _, _ = event_steps(torch, stream, copy, steps)
    cbytes = 2 * keep[0][1].out_hidden.numel() * 2
    return {"workload": "P-EAGLE expansion alone: B=%d, K=%d, H=%d bf16, accepted uniform in 0..K" % (B, K, H),
            "input_copies": copies, "launches": steps, "ms_per_launch": ms, "ms_per_launch_events": each,
            "algorithmic_bytes": nbytes, "GBps": nbytes / (ms * 1e-3) / 1e9,
            "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "write_GBps": (e.N_in + B * (K - 1)) * H * 2 / (ms * 1e-3) / 1e9,
            "device_copy": {"what": "torch copy_ of the [%d, %d] bf16 output hidden rows (read and write once)"
                                    % tuple(keep[0][1].out_hidden.shape), "ms": cms, "bytes": cbytes,
                            "GBps": cbytes / (cms * 1e-3) / 1e9,
                            "write_GBps": cbytes / 2 / (cms * 1e-3) / 1e9}}


def peagle_round(sv, torch, np, inp, seed, steps=20):
    """One P-EAGLE round at the headline shape, timed two ways: draft-token
    sampling at the new-token indices of an expanded batch (from drafter rows
    holding the headline's mixture drafts, so the acceptance is the
    headline's), then the chained verification of those tokens against those
    rows (read in place through the row table) with the expansion of its
    outputs.  "rows": the verification's row pass reads the drafter rows;
    "stats": the sampler hands its row statistics to the verification, whose
    row pass then reads the target rows only.  Each way plans its early-exit
    cut with the shape-priced planner from 8 one-pass rounds."""
    import workloads
    B, K, V = inp.B, inp.K, inp.V
    dev = inp.target.device
    ex = workloads.step_expand_inputs(inp, seed=seed)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ws = sv.make_workspace(B, K, V, dev)
    out = sv.expand_outputs(B, K, ex.N_in, ex.H, dev, with_slots=True)
    # the new-token indices of one expansion, and drafter rows there holding the mixture drafts
    first = sv.expand(ex.in_token_ids, ex.in_positions, ex.in_start, torch.zeros(B, dtype=torch.int32, device=dev),
                      inp.draft_tokens[:, 0].contiguous(), K, ex.mask_id)
    nti = first.new_token_indices.clone()
    drafter = torch.zeros(ex.N_out, V, dtype=inp.draft.dtype, device=dev)
    drafter[nti.reshape(-1).long()] = inp.draft[:, :K].reshape(B * K, V)
    x = torch.empty(B, K, dtype=torch.int32, device=dev)
    stats = sv.draft_stats_buffer(B, K, dev)
    dws = torch.empty(sv.spec_draft_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    xa = sv.expand_args(ex.in_token_ids, ex.in_positions, ex.in_start, acc, None, K, ex.mask_id, ex.target_hidden,
                        ex.mask_hidden, out, verify_tokens=tok, block_table=ex.block_table, block_size=ex.block_size)
    temps = inp.temperature.cpu().numpy()
    res = {}
    for way in ("rows", "stats"):
        da = sv.draft_args(drafter, nti, inp.temperature, x, dws, seed=seed + 9,
                           stats_out=stats if way == "stats" else None)
        va = sv.verify_args(inp.target, drafter, x, inp.temperature, acc, tok, None, ws, seed=seed,
                            draft_row_index=nti, draft_stats=stats if way == "stats" else None)
        mask = {"m": 0}

        def launch(i, ev):
            da.step = va.step = i & 0xFFFFFFFF
            va.phase_starts = mask["m"]
            va.phase_event = ev[1].cuda_event if ev else None
            if ev:
                ev[0].record(stream)
            rc = sv.spec_draft_sample_launch(da, sptr)
            if rc == sv.SPEC_OK:
                rc = sv.spec_verify_expand_launch(va, xa, sptr)
            if rc != sv.SPEC_OK:
                raise sv.SpecError(rc)
            if ev:
                ev[2].record(stream)

        accs = []
        for i in range(PLAN_STEPS):
            launch(7_000_000 + i, None)
            torch.cuda.synchronize()
            accs.extend(acc.cpu().tolist())
        surv = sv.survival_from_accepted(accs, K)
        f = 0.0 if way == "stats" else float((temps > 0).mean())  # draft rows the row pass reads
        mask["m"] = sv.spec_verify_plan_phases(K, surv, f, sv.spec_verify_phase_cost(B, K, V, sv.SPEC_BF16))
        for i in range(3):
            launch(8_000_000 + i, None)
        ms, _, _ = event_steps(torch, stream, launch, steps)
        read = []
        for i in range(steps):
            launch(i, None)
            a_np = acc.cpu().numpy()
            t_eff = temps if way == "rows" else np.zeros_like(temps)
            read.append(phased_logit_bytes(a_np, t_eff, mask["m"], K, V, 2))
        res[way] = {"phase_starts": mask["m"], "ms_per_round": ms, "positions_per_s": B * K / (ms * 1e-3),
                    "row_stage_read_bytes": float(np.mean(read)), "mean_accepted": float(acc.float().mean())}
    del drafter
    return {"workload": "P-EAGLE round at the headline shape: draft sampling at the new-token indices "
                        "([%d, %d] bf16 drafter rows), then the chained verify + expand (H=%d)" % (ex.N_out, V, ex.H),
            "rows": res["rows"], "stats": res["stats"],
            "speedup": res["rows"]["ms_per_round"] / res["stats"]["ms_per_round"]}


def side_configs(sv, torch, np, only, seed):
    import workloads
    dev = torch.device("cuda")
    out = {}
    if only in ("all", "gptoss"):
        base = workloads.verify_gptoss(seed=seed, device=dev)
        copies = [base] + [workloads.VerifyInputs(base.name, base.target.clone(), base.draft.clone(),
                                                  base.draft_tokens.clone(), base.temperature.clone(), seed)
                           for _ in range(3)]
        out["gptoss_vocab"] = verify_config(sv, torch, np, "GPT-OSS vocabulary: B=64, K=5, V=201088 bf16, Zipf "
                                            "target, draft = target + N(0, 0.7), T = 1", copies, seed=seed)
        del base, copies
    if only in ("all", "expand"):
        out["expand"] = expand_config(sv, torch, seed=seed)
    if only in ("all", "large"):
        beta = 0.8
        lam = (1.0 - beta) / workloads.total_variation_noise(workloads.GPT_OSS_VOCAB, rows=16, seed=7, device=dev)
        inp = workloads.verify_beta_sweep(lam, seed=8, device=dev)
        r = verify_config(sv, torch, np, "large batch: B=1024, K=8, V=201088 bf16, T = 1, mixture drafts, "
                          "lam = %.4f for acceptance ~%.1f" % (lam, beta), [inp], steps=12, seed=seed)
        r["acceptance_target"] = beta
        out["large_batch"] = r
        del inp
    torch.cuda.empty_cache()
    return out


def host_cpu():
    """The host's CPU model and core counts (logical cores, and those this
    process may run on)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"cpu_model": model, "logical_cores": os.cpu_count(), "usable_cores": usable}


def cpu_baseline(inp, seed, cpu_seconds):
    """The oracle, as it stands, over whole steps of the headline batch on all
    host threads it is given (OMP_NUM_THREADS, else every core)."""
    import numpy as np
    import oracle
    import workloads
    tl = workloads.logits_numpy(inp.target)
    dl = workloads.logits_numpy(inp.draft)
    x = inp.draft_tokens.cpu().numpy()
    T = inp.temperature.cpu().numpy()
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    steps = 0
    wall = 0.0
    cpu0 = time.process_time()
    while True:
        t0 = time.perf_counter()
        oracle.verify(tl, dl, x, T, seed=seed, step=steps, debug=False, trace=False, nthreads=threads)
        wall += time.perf_counter() - t0
        steps += 1
        if time.process_time() - cpu0 >= cpu_seconds or steps >= 50:
            break
    B, K = x.shape
    used = time.process_time() - cpu0
    # the same oracle on one core, over blocks of 16 requests of the same
    # batch (request_base keeps each request's uniforms those of the step)
    one_wall = 0.0
    one_req = 0
    cpu1 = time.process_time()
    while one_req < B and time.process_time() - cpu1 < cpu_seconds / 4:
        r1 = min(B, one_req + 16)
        t0 = time.perf_counter()
        oracle.verify(tl[one_req:r1], dl[one_req:r1], x[one_req:r1], T[one_req:r1], seed=seed, step=0,
                      request_base=one_req, debug=False, trace=False, nthreads=1)
        one_wall += time.perf_counter() - t0
        one_req = r1
    return {"value": steps * B * K / wall, "unit": "positions/s", "cores": threads, "kind": "oracle",
            "host": host_cpu(),
            "sample": "%d whole step(s) of the headline batch (B=%d, K=%d, V=%d), %.1f CPU-s"
                      % (steps, B, K, tl.shape[-1], used),
            "single_core": {"value": one_req * K / one_wall, "unit": "positions/s", "cores": 1,
                            "sample": "requests 0..%d of step 0 of the same batch" % (one_req - 1)}}


def copy_calibration(torch, dev):
    """One 1 GiB device-to-device copy (a plain copy kernel of known size, to
    scale hardware byte counters)."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def headline(args, sv, torch, np, workloads):
    """The timed steps of the headline workload; returns the JSON fields and
    what the side measurements reuse (inputs, expansion outputs)."""
    dev = torch.device("cuda:0")
    inp = workloads.verify_headline(seed=args.seed, device=dev)
    B, K, V = inp.B, inp.K, inp.V
    H = workloads.HIDDEN_GPT_OSS_20B
    # the verify batch feeding the expansion: per request [last token, x_0..x_{K-1}], and a paged
    # KV cache of 16-slot blocks covering every position of the batch
    ex = workloads.step_expand_inputs(inp, H=H, seed=args.seed)
    accepted = torch.empty(B, dtype=torch.int32, device=dev)
    tokens = torch.empty(B, K + 1, dtype=torch.int32, device=dev)
    ws = sv.make_workspace(B, K, V, dev)
    out = sv.expand_outputs(B, K, ex.N_in, H, dev, with_slots=True)
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    ex_args = sv.expand_args(ex.in_token_ids, ex.in_positions, ex.in_start, accepted, None, K, ex.mask_id,
                             ex.target_hidden, ex.mask_hidden, out, verify_tokens=tokens,
                             block_table=ex.block_table, block_size=ex.block_size)

    # events on every `every`-th timed step: at least 10 of them (each event record costs GPU time of its own)
    every = args.event_every if args.event_every else max(1, min(8, args.steps // 10))
    timed_with_events = [i for i in range(args.steps) if i % every == 0]
    ev = [[TimingEvent() for _ in range(4)] for _ in timed_with_events]
    for e4 in ev:  # create the underlying HIP events
        for e in e4:
            e.record(stream)
    torch.cuda.synchronize()

    plan = {"mask": 0}

    # The hidden rows of the expansion depend only on the windows, not on the accepted counts: with
    # --overlap they are gathered on a second stream that starts when the row statistics end (the library
    # records phase_event there), overlapping the verification's sampling stage; the metadata follows the
    # verification on the main stream, and the step ends when both are done.
    overlap = args.overlap
    chained = not (args.overlap or args.separate_expand)
    side = torch.cuda.Stream()
    meta_out = sv.ExpandOutputs(**{**out.__dict__, "out_hidden": None})
    meta_args = sv.expand_args(ex.in_token_ids, ex.in_positions, ex.in_start, accepted, None, K, ex.mask_id,
                               ex.target_hidden, ex.mask_hidden, meta_out, verify_tokens=tokens,
                               block_table=ex.block_table, block_size=ex.block_size)
    untimed_phase = TimingEvent()
    untimed_phase.record(stream)

    # the argument block is built once, as a serving loop would keep it; each step sets its step counter,
    # phase cut and event (rebuilding it in Python every step costs host time the GPU can wait on)
    va = sv.verify_args(inp.target, inp.draft, inp.draft_tokens, inp.temperature, accepted, tokens, None, ws,
                        seed=args.seed, step=0, phase_event=untimed_phase.cuda_event, phase_starts=0)

    def step(i, events=None, row_stage_only=False):
        # events: [before, after the row stage (the library's phase_event), after the sampling
        # stage, after the expansion]; row_stage_only records the first two only
        ph = events[1] if events else untimed_phase
        va.step = i & 0xFFFFFFFF
        # the phase event only where it is used: a timed stage, or the second stream's start
        va.phase_event = ph.cuda_event if (events or overlap) else None
        va.phase_starts = plan["mask"]
        if events:
            events[0].record(stream)
        if row_stage_only:
            events = None
        if chained:  # one call: the expansion runs inside the verification's sampling stage
            rc = sv.spec_verify_expand_launch(va, ex_args, sptr)
            if rc != sv.SPEC_OK:
                raise sv.SpecError(rc)
            if events:
                events[2].record(stream)
            return
        rc = sv.spec_verify_launch(va, sptr)
        if rc != sv.SPEC_OK:
            raise sv.SpecError(rc)
        if overlap:
            ph.wait_on(side)
            rc = sv.spec_expand_hidden_launch(ex_args, side.cuda_stream)
            if rc != sv.SPEC_OK:
                raise sv.SpecError(rc)
        if events:
            events[2].record(stream)
        rc = sv.spec_expand_launch(meta_args if overlap else ex_args, sptr)
        if rc != sv.SPEC_OK:
            raise sv.SpecError(rc)
        if overlap:
            stream.wait_stream(side)
        if events:
            events[3].record(stream)

    temps = inp.temperature.cpu().numpy()
    sampled_fraction = float((temps > 0).mean())
    if args.early_exit == "plan":
        # the accepted counts of a few one-pass steps give the acceptance curve and the phase plan
        # follows from it, as a serving loop would plan from its recent steps; the boundary is priced
        # for this batch shape
        accs = []
        for i in range(PLAN_STEPS):
            step(2_000_000 + i)
            torch.cuda.synchronize()
            accs.extend(accepted.cpu().tolist())
        surv = sv.survival_from_accepted(accs, K)
        cost = sv.spec_verify_phase_cost(B, K, V, sv.SPEC_BF16)
        plan["mask"] = sv.spec_verify_plan_phases(K, surv, sampled_fraction, cost)
        if args.phase_starts is not None:
            plan["planned_mask"] = plan["mask"]
            plan["mask"] = args.phase_starts
        plan["survival"] = [round(v, 4) for v in surv]
        plan["phase_cost_rows"] = round(cost, 4)
    elif args.early_exit == "dynamic":
        plan["mask"] = sv.SPEC_PHASES_DYNAMIC
    for i in range(args.warmup):
        step(1_000_000 + i)
    torch.cuda.synchronize()
    # the timed steps: the row stage is timed on every `every`-th of them with two events (each event
    # record costs GPU time of its own, and these steps are the ones the wall clock times)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, ev[i // every] if i % every == 0 else None, row_stage_only=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    k1 = np.array([e[0].elapsed_time(e[1]) for e in ev])

    if args.copy_calibration:
        copy_calibration(torch, dev)

    # the later stages, on 24 more steps of the same plan with every event
    evs = [[TimingEvent() for _ in range(4)] for _ in range(24)]
    for e4 in evs:  # create the underlying HIP events
        for e in e4:
            e.record(stream)
    for i in range(3):
        step(5_000_000 + i)
    torch.cuda.synchronize()
    for i, e4 in enumerate(evs):
        step(6_000_000 + i, e4)
    torch.cuda.synchronize()
    k2 = np.array([e[1].elapsed_time(e[2]) for e in evs])
    ke = None if chained else np.array([e[2].elapsed_time(e[3]) for e in evs])

    # the row pass as one launch over every row (no early exit), timed the same way on 24 more
    # steps: the kernel's own streaming rate against the parallel formulation's bytes
    alg_bytes = one_pass_logit_bytes(B, K, V, 2, temps)
    saved_mask = plan["mask"]
    plan["mask"] = 0
    for i in range(5):
        step(3_000_000 + i)
    ev1 = [[TimingEvent() for _ in range(4)] for _ in range(24)]
    for e4 in ev1:  # create the underlying HIP events
        for e in e4:
            e.record(stream)
    torch.cuda.synchronize()
    for i, e4 in enumerate(ev1):
        step(4_000_000 + i, e4)
    torch.cuda.synchronize()
    k1o = np.array([e[0].elapsed_time(e[1]) for e in ev1])
    # the dynamic early exit (decisions inside the row pass, no plan) on the step numbers of the timed
    # steps with events, every event recorded
    plan["mask"] = sv.SPEC_PHASES_DYNAMIC
    for i in range(5):
        step(7_000_000 + i)
    evd = [[TimingEvent() for _ in range(4)] for _ in timed_with_events]
    for e4 in evd:  # create the underlying HIP events
        for e in e4:
            e.record(stream)
    torch.cuda.synchronize()
    for i, e4 in zip(timed_with_events, evd):
        step(i, e4)
    torch.cuda.synchronize()
    k1d = np.array([e[0].elapsed_time(e[1]) for e in evd])
    k2d = np.array([e[1].elapsed_time(e[2]) for e in evd])
    plan["mask"] = saved_mask
    gbs = alg_bytes / (float(k1o.mean()) * 1e-3) / 1e9
    one_pass = {"ms": float(k1o.mean()), "ms_median": float(np.median(k1o)), "achieved": gbs,
                "frac": gbs / HBM_PEAK_GBS, "algorithmic_bytes": alg_bytes, "steps": len(ev1)}

    # the timed steps again, untimed (outputs depend only on seed and step), for the rows each one read
    mask = plan["mask"]
    acc_steps = []
    for i in range(args.steps):
        step(i)
        acc_steps.append(accepted.cpu().numpy().copy())
    # the bytes of the steps whose stages the events timed
    dyn_mode = mask == sv.SPEC_PHASES_DYNAMIC
    seq_bytes = float(np.mean([sequential_logit_bytes(acc_steps[i], temps, K, V, 2) for i in timed_with_events]))
    # the dynamic exit's rows depend on timing and are not counted: its frac is taken on the
    # sequential minimum, a lower bound of what it read
    read_bytes = seq_bytes if dyn_mode else float(
        np.mean([phased_logit_bytes(acc_steps[i], temps, mask, K, V, 2) for i in timed_with_events]))
    vbytes = algorithmic_verify_bytes(B, K, V, 2, temps)
    ebytes = algorithmic_expand_bytes(B, K, H, B * (K + 1))
    k1_ms = float(k1.mean())
    achieved = read_bytes / (k1_ms * 1e-3) / 1e9
    acc_np = np.concatenate(acc_steps)
    positions_per_s = B * K / (ms_per_step * 1e-3)
    traffic, traffic_src = measured_traffic(mask)
    line = {
        "metric": "verified draft positions/sec + achieved HBM GB/s at B=256,K=8,V=151936 bf16",
        "value": positions_per_s,
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "headline verify B=256 K=8 V=151936 bf16, T in {0,0.6,1}, mixture drafts "
                               "+ P-EAGLE expand H=2880 with KV slot mapping, chained on the verify outputs",
                   "B": B, "K": K, "V": V, "H": H, "sampled_requests": int((temps > 0).sum()),
                   "expansion": ("chained call: hidden rows and metadata inside the verification's sampling stage"
                                 if chained else "hidden rows on a second stream, overlapping the sampling stage"
                                 if overlap else "its own kernel after the verification")},
        # the dominant stage as run: achieved and frac on the logit bytes the planned phases read;
        # frac_seq_min on the method's sequential minimum (rows 0..a only); the one-pass row kernel
        # against the parallel formulation's algorithmic bytes
        "roofline": {"kernel": "verify_rowstats", "stage": "row statistics (row-pass launches and phase decisions)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "frac_seq_min": seq_bytes / (k1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_from_profiles": traffic_src,
                     "plan_read_bytes": None if dyn_mode else read_bytes, "algorithmic_bytes": alg_bytes,
                     "sequential_min_bytes": seq_bytes, "stage_ms": k1_ms, "one_pass_row_kernel": one_pass},
        "early_exit": {"phase_starts": mask, "phases": [0] + [k for k in range(1, K + 1) if (mask >> k) & 1],
                       **{k: v for k, v in plan.items() if k != "mask"}},
        # the same steps with the dynamic exit: row stage and sampling stage from events on every step
        # (each event costs GPU time: compare with the plan's stages, not with ms_per_step)
        "early_exit_dynamic": {"phase_starts": sv.SPEC_PHASES_DYNAMIC, "steps": len(evd),
                               "row_stage_ms": float(k1d.mean()), "sampling_stage_ms": float(k2d.mean()),
                               "frac_seq_min": seq_bytes / (float(k1d.mean()) * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "kernels_ms": {"timed_steps_with_events": len(timed_with_events), "event_every": every,
                       "verify_row_stage": k1_ms, "later_stages_timed_on": "24 further steps of the same plan",
                       ("sampling_stage_with_expansion" if chained else "verify_decide_and_draw"): float(k2.mean()),
                       **({} if chained else {("expand_metadata_and_join" if overlap else "expand"): float(ke.mean())}),
                       "verify_row_stage_p10_p90": [float(np.percentile(k1, 10)), float(np.percentile(k1, 90))]},
        "emitted_tokens_per_s": float((acc_np + 1).sum()) / args.steps / (ms_per_step * 1e-3),
        "mean_accepted": float(acc_np.mean()),
    }
    if not chained:  # the verification and the expansion timed apart (with the chained call they share a stage)
        line["verify_GBps_algorithmic"] = (read_bytes + vbytes - alg_bytes) / ((k1.mean() + k2.mean()) * 1e-3) / 1e9
        if not overlap:
            line["expand_GBps_algorithmic"] = ebytes / (ke.mean() * 1e-3) / 1e9
    return line, inp, out


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (request sharding is "
              "described in the design notes); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import rejection_sampling_verify_03_amd as sv
    import workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.only not in ("all", "headline"):
        configs = side_configs(sv, torch, np, args.only, args.seed)
        if args.copy_calibration:
            copy_calibration(torch, dev)
        print(json.dumps({"only": args.only, "configs": configs}), flush=True)
        return
    line, inp, out = headline(args, sv, torch, np, workloads)
    B, K, V = inp.B, inp.K, inp.V
    if not args.no_draft_sampling:
        line["draft_sampling"] = draft_sampling(sv, torch, np, out, inp.temperature, B, K, V, args.seed, dev)
    if not args.no_shard_share:
        # the slice's own plan: the headline's acceptance curve, the boundary priced for a
        # [B, K+1, V/4] slice; the headline's cut timed beside it
        G = 4
        Vs = V // G
        cost = sv.spec_verify_phase_cost(B, K, Vs, sv.SPEC_BF16)
        surv = line["early_exit"].get("survival")
        frac_sampled = line["config"]["sampled_requests"] / B
        smask = sv.spec_verify_plan_phases(K, surv, frac_sampled, cost) if surv else 0
        line["shard_share_tp4"] = shard_share(sv, torch, inp, args.seed, G=G, phase_starts=smask)
        line["shard_share_tp4"]["plan"] = {"phase_starts": smask, "phase_cost_rows": round(cost, 4)}
        hmask = line["early_exit"]["phase_starts"]
        if hmask and hmask != smask:
            line["shard_share_tp4_headline_cut"] = shard_share(sv, torch, inp, args.seed, G=G, phase_starts=hmask)
    if not args.no_configs and args.only == "all":
        line["peagle_round"] = peagle_round(sv, torch, np, inp, args.seed)
        line["configs"] = side_configs(sv, torch, np, "all", args.seed)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, args.seed, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
