// verify.hip -- batched modified-rejection-sampling verification on gfx950.
//
// The method (explainer page on speculative decoding, sections "修正拒绝采样"
// and "核心思想"): draft token x_k is accepted with probability
// min(1, p_k(x_k) / q_k(x_k)); at the first rejection a token is resampled from
// normalize(max(0, p - q)); if all K drafts are accepted a bonus token is
// sampled from p_K.  Temperature 0 is the greedy limit (accept iff x_k is the
// target argmax, emit the target argmax where the request stops).
//
// Four kernels in stream order, no host round trip, and no communication
// between workgroups of one kernel but in the dynamic early exit below (each
// kernel boundary makes the previous kernel's writes visible, so no
// cache-maintenance fences; a device atomic counts invalid requests for the
// host to read after the stream):
//
//  verify_rowstats  one 256-thread workgroup per (request, row, chunk of ~32K
//      logits) streams every row the parallel formulation needs exactly once
//      (target rows 0..K and, for sampled requests, draft rows 0..K-1) with
//      non-temporal 16-byte loads, and reduces the chunk to
//      S * 2^M = sum_v 2^(x_v * s - M) (s = log2(e) / T, M an integer-valued
//      reference raised by exact power-of-two rescaling) or, for greedy
//      requests, to (max, lowest argmax).  The chunk holding a position's
//      draft token also records the logit there.
//
//  verify_decide    one workgroup per request merges its row partials in
//      chunk order and evaluates the K accept tests in parallel (one lane per
//      position, Philox uniforms, double-precision p(x), q(x)); a_b is the
//      count of trailing ones of a wavefront ballot.  Writes the outputs but
//      the sampled token, and a decision record.
//
//  verify_segsum    one wave64 workgroup per (request, 4096-logit segment)
//      sums the residual weights max(0, p - q) and the weights of p over its
//      segment of the sampling row(s) (p_a and q_a, or p_K for the bonus).
//      With a chained expansion, more one-wave workgroups at the end of its
//      grid expand this verification's outputs (hidden rows, metadata).
//
//  verify_draw      one 512-thread workgroup per sampled request scans the
//      segment sums for the inverse-CDF crossing of u' * R (one wave, DPP),
//      recomputes the weights of that one segment (one 512-logit block per
//      wave) and finds the token with a wavefront scan; with a chained
//      expansion it also writes the bonus id into the drafter batch.
//
// Early exit (a request stops at its first rejection, same page, section
// "核心思想"): the caller may cut the positions 0..K into phases.  The row
// pass then runs once per phase over the phase's rows, skipping requests that
// already stopped, and verify_phase runs the phase's accept tests in between
// (one workgroup per request), leaving a per-request state for the next
// phase and for the final decision.  Or the row pass takes the decisions
// itself as its rows come in (verify_rowstats_dyn_kernel), with no phases.
#include <float.h>
#include <limits.h>

#include "decision.hpp"
#include "device_common.hpp"
#include "expand_device.hpp"
#include "rowpass.hpp"
#include "sampling.hpp"
#include "verify_kernels.hpp"
#include "verify_layout.hpp"

namespace specv {

// Element offset of draft row k of request b from the draft base: through
// the row table when one is given (entry di), else by the strides.
__device__ __forceinline__ int64_t draft_off(const VerifyParams& P, int b, int k, int di) {
  return P.dridx ? (int64_t)di * P.d_row : (int64_t)b * P.d_req + (int64_t)k * P.d_row;
}

// Row r of request b: target rows 0..K, then draft rows K+1..2K (di: the
// draft row table's entry for it, when there is a table).
template <int ES>
__device__ __forceinline__ const char* row_ptr(const VerifyParams& P, int b, int r, int di = 0) {
  if (r <= P.K) return P.target + ((int64_t)b * P.t_req + (int64_t)r * P.t_row) * ES;
  return P.draft + draft_off(P, b, r - P.K - 1, di) * ES;
}

// The draft row table's entry for position k (k clamped into [0, K); 0
// without a table), loaded unconditionally so it can be issued with other
// loads; and whether it names a row of the buffer.
__device__ __forceinline__ int draft_entry(const VerifyParams& P, int b, int k) {
  const int32_t* t = P.dridx ? P.dridx : P.tokens;  // any readable [B, K] int32 array
  const int v = t[(int64_t)b * P.K + min(max(k, 0), P.K - 1)];
  return P.dridx ? v : 0;
}

__device__ __forceinline__ bool draft_entry_ok(const VerifyParams& P, int di) {
  return !P.dridx || (uint32_t)di < (uint32_t)P.draft_rows;
}

// Drafts K_b of request b (ragged counts, else K), loaded unconditionally so
// it can be issued with other loads; -1 for a count outside [0, K] (the
// request is invalid).
__device__ __forceinline__ int drafts_of(const VerifyParams& P, int b) {
  const int32_t* t = P.num_drafts ? P.num_drafts : reinterpret_cast<const int32_t*>(P.temperature);
  const int v = t[b];
  const int kb = P.num_drafts ? v : P.K;
  return (kb >= 0 && kb <= P.K) ? kb : -1;
}

// State words of the dynamic early exit (see verify_rowstats_dyn_kernel):
// (launch tag << 8) | (2 n + f).
constexpr uint64_t kTagMask = (1ull << 56) - 1;

__device__ __forceinline__ uint64_t dstate_word(uint64_t E, int n, int f) {
  return ((E & kTagMask) << 8) | (uint64_t)(2 * n + f);
}

// (n, f) of a state word in launch E; (0, 0) for a word of another launch or
// one no decision can write (n > K, or a stop at n >= K).
__device__ __forceinline__ void dstate_read(uint64_t w, uint64_t E, int K, int& n, int& f) {
  const int key = (w >> 8) == (E & kTagMask) ? (int)(w & 0xffu) : 0;
  n = key >> 1;
  f = key & 1;
  if (n > K || (f && n >= K)) n = f = 0;
}

// The tag E of a launch: the workspace's launch counter (byte 8, advanced by
// the last kernel of every launch) plus a salt taken from the workspace's
// address.  The counter of a workspace that was never used holds whatever
// the memory held, and two such workspaces -- say two allocations of one
// allocator, each carved from memory a third one used before -- can hold the
// same value while one's record area holds the other's records; the salt
// keeps their launches apart.
__device__ __forceinline__ uint64_t launch_tag(const VerifyParams& P) { return *P.epoch + P.salt; }

// The 48-bit tags of launch E in the words of a record, each odd (so that
// zeroed memory, such as a fresh workspace or the no-alloc array at load,
// never passes for a record of any launch) and each different for any two
// launches less than 2^47 apart, so that a decider that catches a record
// half-written, some words still from an earlier launch, sees the difference
// in every such word: words 0-3 carry record_tag (the low bits of 2E + 1),
// words 4-7 record_tag_b (the same with the higher bits E >> 47 folded in),
// so that a record left whole by an earlier launch repeats all eight tags
// only after 2^94 launches.  With 32-bit tags a record caught half-written
// could pass for one whose other words a launch exactly 2^31 back had left.
constexpr uint64_t kRecTagMask = (1ull << 48) - 1;
__device__ __forceinline__ uint64_t record_tag(uint64_t E) { return (2 * E + 1) & kRecTagMask; }
__device__ __forceinline__ uint64_t record_tag_b(uint64_t E) {
  return ((2 * E + 1) ^ ((E >> 47) << 1)) & kRecTagMask;
}

// Word i of the tagged record of `part` in launch E.
__device__ __forceinline__ uint64_t record_word(const RowPartial& part, int i, uint64_t E) {
  const uint64_t lo = ((uint64_t)(uint32_t)part.idx << 32) | __float_as_uint(part.m);
  const uint64_t hi = (uint64_t)__double_as_longlong(part.s);
  const uint64_t pay = ((i < 4 ? lo : hi) >> (16 * (i & 3))) & 0xffffu;
  return ((i < 4 ? record_tag(E) : record_tag_b(E)) << 16) | pay;
}

// Agent-scope accesses: coherent between workgroups of one launch, whatever
// their XCD (no cache maintenance, no ordering between different words).
__device__ __forceinline__ uint64_t load_coherent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------- decision
// The accept tests of request b over draft positions [lo, hi) (positions
// before lo passed in earlier phases), computed by the whole workgroup.
// Merges the statistics of target rows [lo, thi) and, for a sampled request,
// draft rows [lo, min(thi, K)) into `sh`; thi >= hi.  With known >= 0 no test
// runs and a = known (its rows lo = known, thi = known + 1 are merged for the
// draw).  Returns, in every thread, a in [lo, hi] (hi: every test in range
// passed) or -1 for invalid data (stop_position: the inputs, or a row without
// a usable normaliser where the request stops; rows past the stop do not
// count).  Every draft token and the temperature are checked whatever the
// range, so invalid tokens are caught by the first decision of a request.
// With check_state, a request whose state is not alive returns kNotAlive and
// writes nothing.  With `debug`, writes p_k(x_k), q_k(x_k) of every tested
// position, and zero for: the positions from hi on when the request stopped
// before hi (their rows are never read), with zero_after the positions past
// the stop, positions whose rows have no usable normaliser, and every
// position of an invalid request.
struct DecideShared {
  int64_t qoff[SPEC_MAX_K];     // draft row offsets of the positions
  float m[2 * SPEC_MAX_K + 1];
  double s[2 * SPEC_MAX_K + 1];
  float z[2 * SPEC_MAX_K + 1];  // logit of the row at its position's draft token
  int g[SPEC_MAX_K + 1];
  unsigned char bad[2 * SPEC_MAX_K + 1];  // a merged sampled row without a usable normaliser
  int a;
  int kb;  // drafts of the request
};

// Merge the chunk partials of one row in chunk order, the first batch of 8
// given (loaded by the caller with everything else), later batches loaded 8 at
// a time.  Sampled rows also return the logit at x recorded by the chunk that
// holds x (x outside [0, V) leaves z = 0; such a request is invalid).
constexpr int kPartBatch = 8;

__device__ __forceinline__ void load_partials(const RowPartial* __restrict__ rp, int c0, int C1,
                                              RowPartial q[kPartBatch]) {
#pragma unroll
  for (int i = 0; i < kPartBatch; ++i)
    if (c0 + i < C1) q[i] = rp[c0 + i];
}

template <int ES, bool GREEDY>
__device__ __forceinline__ void merge_row(const VerifyParams& P, const RowPartial* __restrict__ rp,
                                          RowPartial q[kPartBatch], int x, MS& ms, VI& vi, float& z) {
  const int cx = (x >= 0 && x < P.V) ? x / P.chunk1 : -1;
  z = 0.f;
  for (int c0 = 0; c0 < P.C1; c0 += kPartBatch) {
    if (c0 > 0) load_partials(rp, c0, P.C1, q);
#pragma unroll
    for (int i = 0; i < kPartBatch; ++i) {
      const int c = c0 + i;
      if (c >= P.C1) break;
      if (GREEDY) {
        const VI v{q[i].m, q[i].idx};
        vi = c == 0 ? v : vi_pick(vi, v);
      } else {
        const MS v{q[i].m, q[i].s};
        ms = c == 0 ? v : ms_merge(ms, v);
        if (c == cx) z = bits_to_logit<ES>((uint32_t)q[i].idx);
      }
    }
  }
}

constexpr int kNotAlive = -3;  // decide_tests: the request stopped in an earlier phase

template <int ES>
__device__ int decide_tests(const VerifyParams& P, int b, int lo, int hi, int thi, int known, bool invalid,
                            bool debug, bool check_state, DecideShared& sh, bool zero_after = false) {
  const int K = P.K;
  const int tid = threadIdx.x;
  const bool test = known < 0;
  // Every load of the prologue is issued before any result is used: the
  // state (stale and ignored without check_state), the temperature, the
  // tokens, and the first partials of every row the request may need (draft
  // rows too, ignored for a greedy request).
  const int st = P.state[b];
  const float T = P.temperature[b];
  const int kb_ = drafts_of(P, b);
  const int x = P.tokens[(int64_t)b * K + min(tid, K - 1)];
  const int nt = thi - lo;
  const int nd = min(thi, K) - lo;
  const bool row_thread = tid < nt + nd && !invalid;
  const int r = tid < nt ? lo + tid : K + 1 + lo + (tid - nt);
  const int k = tid < nt ? r : r - K - 1;  // position of the row
  const RowPartial* rp = P.rowp + ((int64_t)b * P.R + (row_thread ? r : 0)) * P.C1;
  const int xr = P.tokens[(int64_t)b * K + min(k, K - 1)];
  // with draft statistics a draft row is its sampler's record, not partials
  const bool stat_row = P.dstats != nullptr && tid >= nt;
  RowPartial q[kPartBatch];
  if (row_thread) {
    if (stat_row) q[0] = P.dstats[(int64_t)b * K + min(k, K - 1)];
    else load_partials(rp, 0, P.C1, q);
  }

  const int dix = draft_entry(P, b, tid);
  const bool greedy = (T == 0.0f);
  // positions k >= K_b do not exist: no token, no draft row, no test; target
  // rows up to K_b (the bonus row) exist
  const int kb = max(kb_, 0);
  bool inbad = invalid || kb_ < 0 || !temperature_valid(T) || (tid < kb && (x < 0 || x >= P.V));
  if (!greedy && tid < kb) {
    inbad |= !draft_entry_ok(P, dix);  // a sampled request reads every draft row
    sh.qoff[tid] = draft_off(P, b, tid, dix);
  }
  const bool row_exists = tid < nt ? k <= kb : k < kb;
  if (row_thread && row_exists && (!greedy || tid < nt)) {
    MS ms{0.f, 0.0};
    VI vi{0.f, 0};
    float z;
    if (greedy) {
      merge_row<ES, true>(P, rp, q, -1, ms, vi, z);
      sh.g[r] = vi.i;
    } else {
      if (stat_row) {
        ms = MS{q[0].m, q[0].s};
        z = bits_to_logit<ES>((uint32_t)q[0].idx);
      } else {
        merge_row<ES, false>(P, rp, q, k < kb ? xr : -1, ms, vi, z);
      }
      sh.m[r] = ms.m;
      sh.s[r] = ms.s;
      sh.z[r] = z;
      sh.bad[r] = !row_usable(ms.m, ms.s);
    }
  }
  const bool anybad = __syncthreads_or(inbad) != 0;
  if (check_state && st != kStateAlive) return kNotAlive;  // its partials here were never written
  if (tid < 64) {  // wave 0: one lane per draft position
    // rows of position tid merged here (sampled): target row and draft row
    const bool merged = !greedy && tid >= lo && tid < thi && tid < kb;
    const bool rowbad = merged && (sh.bad[tid] || sh.bad[K + 1 + tid]);
    const bool bonusbad = !greedy && kb >= lo && kb < thi && sh.bad[kb];
    bool acc = tid < lo;
    float dp = 0.f, dq = 0.f;
    if (test && tid >= lo && tid < min(hi, kb) && !anybad && !rowbad) {
      if (greedy)
        acc = (x == sh.g[tid]);
      else
        acc = accept_test(T, sh.z[tid], sh.m[tid], sh.s[tid], sh.z[K + 1 + tid], sh.m[K + 1 + tid],
                          sh.s[K + 1 + tid], P.seed, (uint32_t)b + P.request_base, (uint32_t)tid, P.step, dp, dq);
    }
    // lanes >= min(hi, K_b) fail: a <= min(hi, K_b)
    const int a = stop_position(test, lo, hi, thi, known, kb, acc, rowbad, bonusbad, anybad);
    if (debug && P.debug && tid < K) {
      float* d = P.debug + ((int64_t)b * K + tid) * 2;
      if (a < 0 || (tid >= hi && a < hi) || (zero_after && tid > a) || (rowbad && tid >= lo && tid < hi)) {
        d[0] = 0.f;
        d[1] = 0.f;
      } else if (test && tid >= lo && tid < hi) {
        d[0] = dp;
        d[1] = dq;
      }
    }
    if (tid == 0) {
      sh.a = a;
      sh.kb = kb;
    }
  }
  __syncthreads();
  return sh.a;
}

// The outputs and decision record of request b once its stop a = sh.a is
// known (all threads of the workgroup call it): with `write`, the outputs (all
// but the token the draw samples) and the decision record; `D` (shared) gets
// the record either way.
template <int ES>
__device__ void decide_finish(const VerifyParams& P, int b, bool write, ReqDesc& D, const DecideShared& sh) {
  const int K = P.K;
  const int tid = threadIdx.x;
  const int a = sh.a;
  const float T = P.temperature[b];
  const bool greedy = (T == 0.0f);
  const bool bad = a < 0;
  if (tid < 64) {
    if (write) {
      int32_t* out = P.out_tokens + (int64_t)b * (K + 1);
      for (int j = tid; j <= K; j += 64) {  // K <= 63: one pass
        int tok;
        if (bad || j > a) tok = -1;
        else if (j < a) tok = P.tokens[(int64_t)b * K + j];
        else tok = greedy ? sh.g[a] : -1;  // sampled: written by the draw
        if (!(j == a && !greedy && !bad)) out[j] = tok;
      }
      if (bad && P.debug)  // invalid: no probability is reported
        for (int j = tid; j < K; j += 64) {
          P.debug[((int64_t)b * K + j) * 2 + 0] = 0.f;
          P.debug[((int64_t)b * K + j) * 2 + 1] = 0.f;
        }
      if (tid == 0) {
        P.accepted[b] = a;
        if (bad) atomicAdd(P.err, 1);
      }
    }
    if (tid == 0) {
      ReqDesc d;
      d.a = a;
      d.mode = (bad || greedy) ? kModeNone : (a < sh.kb ? kModeResidual : kModeBonus);
      d.s_hi = d.s_lo = 0.f;
      d.mp = d.sp = d.mq = d.sq = d.u = 0.0;
      d.qoff = 0;
      if (d.mode != kModeNone) {
        temperature_scale(T, d.s_hi, d.s_lo);
        d.mp = (double)sh.m[a];
        d.sp = sh.s[a];
        if (a < sh.kb) {
          d.mq = (double)sh.m[K + 1 + a];
          d.sq = sh.s[K + 1 + a];
          d.qoff = sh.qoff[a];
        }
        const uint32_t k0 = (uint32_t)(P.seed & 0xffffffffu), k1 = (uint32_t)(P.seed >> 32);
        d.u = unit_uniform(philox4x32_10((uint32_t)b + P.request_base, (uint32_t)a, P.step, 0u, k0, k1).w[1]);
      }
      D = d;
      if (write) P.desc[b] = d;
    }
  }
  __syncthreads();
}

// The decision of request b at the sampling stage, computed by the whole
// workgroup into `D` (shared).  With `write`, the request's outputs (all but
// the token the draw samples), its debug rows and its decision record are
// written too.
template <int ES>
__device__ void decide(const VerifyParams& P, int b, bool write, ReqDesc& D) {
  __shared__ DecideShared sh;
  const int K = P.K;
  int lo = 0, known = -1;
  bool invalid = false;
  if (P.dyn) {  // decisions inside the row pass: every test again, from the partials
    const uint64_t E = launch_tag(P);
    int n, f;
    dstate_read(P.dstate[b], E, K, n, f);
    // with f the rows past n may not have been read: test [0, n] only
    const int a = decide_tests<ES>(P, b, 0, f ? n + 1 : K, f ? n + 1 : K + 1, -1, false, write, false, sh, true);
    __syncthreads();
    if (threadIdx.x == 0) {
      // position n passed after all: the state word was not written in this launch
      sh.a = (f && a > n) ? -1 : a;
      if (write) P.dstate[b] = dstate_word(E + 1, 0, 0);  // the next launch starts from nothing
    }
    __syncthreads();
    decide_finish<ES>(P, b, write, D, sh);
    return;
  }
  if (P.phased) {  // rows were read in phases: the request may have stopped earlier
    const int st = P.state[b];
    invalid = st == kStateInvalid;
    if (st >= 0) {
      known = st;
      lo = st;
    } else {
      lo = P.last_lo;
    }
  }
  const int thi = known >= 0 ? known + 1 : K + 1;
  decide_tests<ES>(P, b, lo, K, thi, known, invalid, write, false, sh);
  decide_finish<ES>(P, b, write, D, sh);
}

// Between early-exit phases: the accept tests of the phase's positions
// [ph_lo, ph_lo + ph_nd) for every request still alive; one workgroup per
// request updates its state.
template <int ES>
__global__ __launch_bounds__(kWG) void verify_phase_kernel(VerifyParams P) {
  __shared__ DecideShared sh;
  const int b = blockIdx.x;
  const int lo = P.ph_lo, hi = P.ph_lo + P.ph_nd;
  const int a = decide_tests<ES>(P, b, lo, hi, hi, -1, false, true, P.ph_check != 0, sh);
  if (a == kNotAlive) return;
  if (threadIdx.x == 0) P.state[b] = a < 0 ? kStateInvalid : (a < hi ? a : kStateAlive);
}

template <int ES, bool VEC>
__global__ __launch_bounds__(kWG) void verify_rowstats_kernel(VerifyParams P) {
  // a 3D grid (chunk, row, request), in the order of the linear index, so
  // that no integer division precedes the first load; batches past the
  // grid's 65535 in z use the linear index instead (x then spans every
  // workgroup, which a 3D grid's x only does for one row of one request, where
  // both readings agree)
  int c, lr, b;
  if ((int)gridDim.x == P.C1) {
    c = blockIdx.x;
    lr = blockIdx.y;
    b = blockIdx.z;
  } else {
    const int nr = P.ph_nt + P.ph_rd;
    c = blockIdx.x % P.C1;
    lr = (blockIdx.x / P.C1) % nr;
    b = blockIdx.x / (P.C1 * nr);
  }
  const int r = lr < P.ph_nt ? P.ph_lo + lr : P.K + 1 + P.ph_lo + (lr - P.ph_nt);
  const int k = lr < P.ph_nt ? r : r - P.K - 1;  // position of the row
  // three independent loads, unconditional and all feeding one branch so that
  // they are issued together (the state of a first phase is stale and
  // ignored; position K has no token)
  const float T = P.temperature[b];
  const int st = P.state[b];
  const int xt = P.tokens[(int64_t)b * P.K + min(k, P.K - 1)];
  const int di = draft_entry(P, b, k);
  const int kb = drafts_of(P, b);
  const bool greedy = (T == 0.0f);
  // skip: draft rows of greedy requests (never read), requests that stopped in
  // an earlier phase, rows past the request's drafts (target row > K_b, draft
  // row >= K_b: they do not exist), and rows of a request whose draft count,
  // draft token or draft row entry is out of range (the request is invalid;
  // no statistic is used)
  if ((blockIdx.x | blockIdx.y | blockIdx.z) == 0 && threadIdx.x == 0 && P.ph_lo == 0)
    *P.err = 0;  // counted by the final decision
  const bool skip = (greedy & (r > P.K)) | ((P.ph_check != 0) & (st != kStateAlive)) |
                    ((k < kb) & ((uint32_t)xt >= (uint32_t)P.V)) | ((r > P.K) & !draft_entry_ok(P, di)) |
                    (kb < 0) | ((r <= P.K) & (k > kb)) | ((r > P.K) & (k >= kb));
  if (skip) return;
  const int x = k < kb ? xt : -1;
  const char* row = row_ptr<ES>(P, b, r, di);
  const int e0 = c * P.chunk1;
  const int e1 = min(P.V, e0 + P.chunk1);
  RowPartial part;
  if (greedy) {
    const VI v = block_argmax(chunk_argmax<ES, VEC>(row, e0, e1));
    part.m = v.v;
    part.idx = v.i;
    part.s = 0.0;
  } else {
    // the logit at the position's draft token, recorded by the chunk holding
    // it: loaded unconditionally (clamped into the chunk) and kept as loaded,
    // so that nothing waits for it before the stream below
    const bool has_x = x >= e0 && x < e1;
    const uint32_t zbits = load_bits<ES>(row, min(max(x, e0), e1 - 1));
    float s_hi, s_lo;
    temperature_scale(T, s_hi, s_lo);
    const MS v = block_merge_ms(chunk_stats<ES, VEC>(row, e0, e1, s_hi, s_lo));
    part.m = v.m;
    part.idx = has_x ? (int32_t)zbits : 0;
    part.s = v.s;
  }
  if (threadIdx.x == 0) P.rowp[((int64_t)b * P.R + r) * P.C1 + c] = part;
}

// ------------------------------------------------------ dynamic early exit
// The row pass with the decisions inside it (same page, section "核心思想":
// a request stops at its first rejection).  The grid is position-major:
// block J holds, for every request in order, the chunks of its target row J
// and (sampled, without draft statistics) draft row J, plus one decider slot.
// The decider slot after request g's chunks serves request d = g - dyn_shift
// (mod B): it tests, from the records of this launch, the positions of d from
// the first one not yet known to pass up to J (J - 1 when d's chunks of J come
// after it), in order, and stops at the first position whose records are not
// all there yet, that fails its test, or whose rows have no usable
// normaliser.  The result goes into d's state word with an atomic maximum, so
// it only ever moves forward: (n, 0) positions before n known to pass, (n, 1)
// the request stops at n.  A chunk workgroup of position k > n of a stopped
// request exits at once.  Nothing waits for anything: a decision that finds
// its records incomplete is left to a later decider slot, and a late one only
// costs the rows read meanwhile.  The final decision recomputes every test
// from the plain partials after the launch, so the outputs never depend on
// which rows the deciders let the pass skip.
struct DynShared {
  uint64_t sw;  // the request's state word as the decider read it
  uint64_t swv[kWaves];         // the state word as each wave of a chunk workgroup read it
  unsigned char skipv[kWaves];  // a chunk workgroup's row skipped for its own reasons
  // one record per thread of a decider: (position - p0) * 2 C1 + row kind * C1 + chunk
  float m[kWG];
  int32_t idx[kWG];
  double s[kWG];
  unsigned char ok[kWG];  // all eight words carry this launch's tags
  // merged rows of a decider's window: (position - p0) * 2 + row kind
  float rm[2 * 64];
  double rs[2 * 64];
  float rz[2 * 64];
  int32_t rg[2 * 64];
  unsigned char rok[2 * 64];
};

// The decider slot of request d at block J: one round of loads (the state
// word, the request's scalars and every record of a window of positions
// ending at the last one it may test), then the merges and tests, then one
// atomic maximum that nothing waits for.
template <int ES>
__device__ void dyn_decider(const VerifyParams& P, int J, int g, uint64_t E, DynShared& ds) {
  const int B = P.B, K = P.K, C1 = P.C1;
  int d = g - P.dyn_shift, j = J;
  if (d < 0) {
    d += B;
    j = J - 1;
  }
  const int per = 2 * C1;  // records of a position: its target row and its draft row
  if (j < 0 || per > kWG) return;  // a position's records must fit one round
  const int top = min(j, K - 1);          // the last position that may be tested
  const int w = min(top + 1, kWG / per);  // the window [p0, top] of loaded positions
  const int p0 = top - w + 1;
  const int t = threadIdx.x;
  const float T = P.temperature[d];
  const int kb = drafts_of(P, d);
  if (t == 0) ds.sw = load_coherent(P.dstate + d);  // one value for the whole workgroup
  if (t < w * per) {
    const int p = p0 + t / per, rr = (t / C1) % 2, c = t % C1;
    const int r = rr == 0 ? p : K + 1 + p;
    const uint64_t* wp = P.trec[((int64_t)d * P.R + r) * C1 + c].w;
    uint64_t wv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wv[i] = load_coherent(wp + i);
    const uint64_t tag = record_tag(E), tag_b = record_tag_b(E);
    bool ok = true;
    uint64_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ok = ok && (wv[i] >> 16) == (i < 4 ? tag : tag_b);
      const uint64_t piece = (wv[i] & 0xffffu) << (16 * (i & 3));
      if (i < 4) lo |= piece;
      else hi |= piece;
    }
    ds.ok[t] = ok;
    ds.m[t] = __uint_as_float((uint32_t)lo);
    ds.idx[t] = (int32_t)(uint32_t)(lo >> 32);
    ds.s[t] = __longlong_as_double((long long)hi);
  }
  __syncthreads();
  int n0, f;
  dstate_read(ds.sw, E, K, n0, f);
  const int hi = min(top, kb - 1);  // the last position to test
  // nothing to decide: stopped already, invalid scalars, no position in
  // range, or the first open position outside the window
  if (f || kb < 0 || !temperature_valid(T) || hi < n0 || n0 < p0) return;
  const bool greedy = T == 0.0f;
  if (t < 2 * w) {  // one thread per row of the window: merge its chunks in chunk order
    const int p = p0 + t / 2, rr = t % 2;
    const int base = (t / 2) * per + rr * C1;
    const int x = P.tokens[(int64_t)d * K + p];
    const bool xin = x >= 0 && x < P.V;
    const int cx = xin ? x / P.chunk1 : -1;
    bool ok = xin;
    MS ms{ds.m[base], ds.s[base]};
    VI vi{ds.m[base], ds.idx[base]};
    float z = cx == 0 ? bits_to_logit<ES>((uint32_t)ds.idx[base]) : 0.f;
    for (int c = 0; c < C1; ++c) {
      ok = ok && ds.ok[base + c];
      if (c == 0) continue;
      if (greedy) {
        vi = vi_pick(vi, VI{ds.m[base + c], ds.idx[base + c]});
      } else {
        ms = ms_merge(ms, MS{ds.m[base + c], ds.s[base + c]});
        if (c == cx) z = bits_to_logit<ES>((uint32_t)ds.idx[base + c]);
      }
    }
    ds.rm[t] = ms.m;
    ds.rs[t] = ms.s;
    ds.rz[t] = z;
    ds.rg[t] = vi.i;
    ds.rok[t] = ok;
  }
  __syncthreads();
  if (t < 64) {  // wave 0: lane l tests position n0 + l
    const int p = n0 + t;
    const int np = hi - n0 + 1;
    const bool in = t < np;
    const int i = in ? 2 * (p - p0) : 0;  // its target row in the window (draft row: i + 1)
    const bool need_q = !greedy && !P.dstats;
    const bool complete = in && ds.rok[i] && (!need_q || ds.rok[i + 1]);
    const int x = in ? P.tokens[(int64_t)d * K + p] : 0;
    bool stop = false;  // the request stops here: its test failed, or its rows are unusable
    if (complete) {
      if (greedy) {
        stop = x != ds.rg[i];
      } else {
        float mq, zq;
        double sq;
        if (P.dstats) {
          const RowPartial q = P.dstats[(int64_t)d * K + p];
          mq = q.m;
          sq = q.s;
          zq = bits_to_logit<ES>((uint32_t)q.idx);
        } else {
          mq = ds.rm[i + 1];
          sq = ds.rs[i + 1];
          zq = ds.rz[i + 1];
        }
        float dp, dq;
        stop = !row_usable(ds.rm[i], ds.rs[i]) || !row_usable(mq, sq) ||
               !accept_test(T, ds.rz[i], ds.rm[i], ds.rs[i], zq, mq, sq, P.seed, (uint32_t)d + P.request_base,
                            (uint32_t)p, P.step, dp, dq);
      }
    }
    const uint64_t go = __ballot(complete && !stop);
    const uint64_t done = __ballot(complete);
    const int first = (int)__builtin_ctzll(~go);  // <= np
    if (t == 0) {
      const int n = n0 + first;
      const int fl = (first < np && ((done >> first) & 1u)) ? 1 : 0;
      if (2 * n + fl > 2 * n0 + f)
        __hip_atomic_fetch_max(P.dstate + d, (unsigned long long)dstate_word(E, n, fl), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Chunk c of row r of request b: its partial into rowp and, tagged with the
// launch, into trec (one word per lane of the first eight).
template <int ES, bool VEC>
__device__ __forceinline__ void dyn_chunk(const VerifyParams& P, int b, int r, int c, int x, bool greedy, float T,
                                          int di, uint64_t E) {
  const char* row = row_ptr<ES>(P, b, r, di);
  const int e0 = c * P.chunk1;
  const int e1 = min(P.V, e0 + P.chunk1);
  RowPartial part;
  if (greedy) {
    const VI v = block_argmax(chunk_argmax<ES, VEC>(row, e0, e1));
    part.m = v.v;
    part.idx = v.i;
    part.s = 0.0;
  } else {
    const bool has_x = x >= e0 && x < e1;
    const uint32_t zbits = load_bits<ES>(row, min(max(x, e0), e1 - 1));
    float s_hi, s_lo;
    temperature_scale(T, s_hi, s_lo);
    const MS v = block_merge_ms(chunk_stats<ES, VEC>(row, e0, e1, s_hi, s_lo));
    part.m = v.m;
    part.idx = has_x ? (int32_t)zbits : 0;
    part.s = v.s;
  }
  const int64_t at = ((int64_t)b * P.R + r) * P.C1 + c;
  if (threadIdx.x == 0) P.rowp[at] = part;
  if (threadIdx.x < 8) store_coherent(&P.trec[at].w[threadIdx.x], record_word(part, threadIdx.x, E));
}

// Block J: per request, the chunks of its target row J and (sampled, J <
// K_b, without draft statistics) of its draft row J, one workgroup each, then
// its decider slot.
template <int ES, bool VEC>
__global__ __launch_bounds__(kWG) void verify_rowstats_dyn_kernel(VerifyParams P) {
  __shared__ DynShared ds;
  const int K = P.K, C1 = P.C1;
  // 32-bit index arithmetic (the grid fits, checked on the host): it runs
  // before the first load of every workgroup
  const int wm = (P.dstats ? 1 : 2) * C1 + 1, wl = C1 + 1;
  const int span = P.B * wm;
  const int bid = (int)blockIdx.x;
  const int J = min(bid / span, K);
  const int rem = bid - J * span;
  const int W = J < K ? wm : wl;
  // the roles inside a group rotate with the group, so that no role keeps to
  // one XCD when W is a multiple of the 8 the hardware deals workgroups to
  const int g = rem / W, sl = (rem - g * W + g) % W;
  const uint64_t E = launch_tag(P);
  if (sl == W - 1) {
    dyn_decider<ES>(P, J, g, E, ds);
    return;
  }
  const int b = g, k = J, c = sl % C1;
  const bool draft_row = sl >= C1;
  const int r = draft_row ? K + 1 + k : k;
  // every wave reads the state word, and the waves then agree on the largest
  // value any of them saw: a decision may land between two waves' reads, and
  // the waves must agree on whether to skip (the block reduction below has
  // barriers); the word only moves forward, so the largest is the newest
  const uint64_t sw = load_coherent(P.dstate + b);
  const float T = P.temperature[b];
  const int xt = P.tokens[(int64_t)b * K + min(k, K - 1)];
  const int di = draft_entry(P, b, k);
  const int kb = drafts_of(P, b);
  const bool greedy = (T == 0.0f);
  // skip as the phased pass does (then, below, every row past a known stop)
  const bool skip_rows = (greedy & draft_row) | ((k < kb) & ((uint32_t)xt >= (uint32_t)P.V)) |
                         (draft_row & !draft_entry_ok(P, di)) | (kb < 0) | (!draft_row & (k > kb)) |
                         (draft_row & (k >= kb));
  if ((threadIdx.x & 63) == 0) {
    ds.skipv[threadIdx.x >> 6] = skip_rows;  // first: its loads go out before the state word is awaited
    ds.swv[threadIdx.x >> 6] = sw;
  }
  if (bid == 0 && threadIdx.x == 0) *P.err = 0;  // counted by the final decision
  __syncthreads();
  if (ds.skipv[0]) return;  // the same in every wave: plain inputs
  uint64_t swm = ds.swv[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) swm = max(swm, ds.swv[w]);
  int n, f;
  dstate_read(swm, E, K, n, f);
  if ((f != 0) & (n < k)) return;
  dyn_chunk<ES, VEC>(P, b, r, c, k < kb ? xt : -1, greedy, T, di, E);
}

// ------------------------------------------------------------ sampling weights
// The weight context of a decision record: scale, references and the split
// residual constant c = S_p / S_q (see WeightCtx).
__device__ __forceinline__ WeightCtx make_ctx(const ReqDesc& d) {
  WeightCtx w;
  w.s_hi = d.s_hi;
  w.s_lo = d.s_lo;
  w.negMp = -(float)d.mp;
  w.negMq = -(float)d.mq;
  const double c = d.mode == kModeResidual ? d.sp / d.sq : 0.0;
  w.c_hi = (float)c;
  w.c_lo = (float)(c - (double)w.c_hi);
  return w;
}

// The final decision of every request: outputs (all but the token the draw
// samples), debug rows and the decision record; one workgroup per request.
template <int ES>
__global__ __launch_bounds__(kWG) void verify_decide_kernel(VerifyParams P) {
  __shared__ ReqDesc D;
  decide<ES>(P, blockIdx.x, true, D);
}

// A decision record that calls for a draw (anything else samples nothing).
__device__ __forceinline__ bool desc_samples(const ReqDesc& d, int K) {
  // residual at a rejected position a < K_b <= K; bonus at row a = K_b <= K
  return (d.mode == kModeResidual || d.mode == kModeBonus) && d.a >= 0 && d.a <= K &&
         (d.mode == kModeBonus || d.a < K);
}

// The sums of one 4096-logit segment of one request's sampling row(s): one
// wave64 workgroup per (request, segment), so that the hardware dispatcher
// balances the sampled requests' segments over the compute units (the
// requests that sample nothing exit after reading their decision record).
// The workgroups past B * nseg expand the verification's outputs (a chained
// expansion): hidden rows and metadata of rows g, g + ex_G, ... of request
// b's window, after the decision (accepted counts and greedy tokens are
// written); a sampled request's bonus id is left to the draw, which samples it.
__device__ __forceinline__ void chained_expand(const VerifyParams& P, int t) {
  const ExpandParams& E = P.ex;
  const int b = t / P.ex_G, g = t % P.ex_G;
  const int tid = threadIdx.x;
  const ExpandWindow w = expand_window(E, b);
  if (g == 0 && tid == 0) expand_out_start(E, b, w);
  if (!w.valid) {
    if (g == 0) expand_invalid(E, b, tid, 64);
    return;
  }
  if (E.out_h != nullptr) {
    if (E.vec) expand_copy_rows<true>(E, w, g, P.ex_G, tid, 64);
    else expand_copy_rows<false>(E, w, g, P.ex_G, tid, 64);
  }
  expand_meta_rows(E, b, w, g, P.ex_G, tid, 64, desc_samples(P.desc[b], P.K));
}

template <int ES, bool VEC>
__global__ __launch_bounds__(64) void verify_segsum_kernel(VerifyParams P) {
  if ((int64_t)blockIdx.x >= (int64_t)P.B * P.nseg) {
    chained_expand(P, (int)(blockIdx.x - P.B * P.nseg));
    return;
  }
  const int j = blockIdx.x % P.nseg;
  const int b = blockIdx.x / P.nseg;
  const ReqDesc d = P.desc[b];
  if (!desc_samples(d, P.K)) return;
  const bool res = d.mode == kModeResidual;
  const char* prow = row_ptr<ES>(P, b, d.a);
  const char* qrow = res ? P.draft + d.qoff * ES : prow;
  const WeightCtx w = make_ctx(d);
  double rs, ps;
  if (res) segment_sums<ES, VEC, true>(prow, qrow, w, j * kSeg, P.V, rs, ps);
  else segment_sums<ES, VEC, false>(prow, qrow, w, j * kSeg, P.V, rs, ps);
  if (threadIdx.x == 0) {
    double* seg = P.seg + ((int64_t)b * P.nseg + j) * 2;
    seg[0] = rs;
    seg[1] = ps;
  }
}

// --------------------------------------------------------------------- draw
constexpr int kWGD = kDrawThreads;

template <int ES, bool VEC>
__global__ __launch_bounds__(kWGD) void verify_draw_kernel(VerifyParams P) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int nseg = P.nseg;
  const double* seg = P.seg + (int64_t)b * P.nseg * 2;
  // the last kernel of the verification advances the launch counter (the
  // row pass and the decision of this launch have read it)
  if (b == 0 && tid == 0) *P.epoch = *P.epoch + 1;
  // the decision record and the first block of segment sums are loaded together
  const ReqDesc d = P.desc[b];
  const bool in0 = tid < nseg;
  const double r0 = in0 ? seg[2 * tid + 0] : 0.0;
  const double p0 = in0 ? seg[2 * tid + 1] : 0.0;
  // a chained expansion's window, for the bonus id written at the end: its
  // loads go out with the others instead of after the draw
  ExpandWindow xw{};
  if (P.ex_on && tid == 0) xw = expand_window(P.ex, b);
  if (!desc_samples(d, P.K)) return;  // greedy or invalid: nothing to sample
  __shared__ double sh_base;
  int found = -1, lastpos = -1;
  double base = 0.0, target;
  bool res;
  if (nseg <= 64) {
    // one wave scans both weight kinds and finds the crossing of u' * W; the
    // other waves take the result from LDS
    __shared__ double sh_target;
    __shared__ int sh_found, sh_last, sh_res;
    if (tid < 64) {
      const double ir = wave_scan_d(r0), ip = wave_scan_d(p0);
      const double tr = lane_d(ir, 63), tp = lane_d(ip, 63);
      const bool rs = d.mode == kModeResidual && tr > 0.0;  // else the weights fall back to p
      const double tg = d.u * (rs ? tr : tp);
      const double incl = rs ? ir : ip, v = rs ? r0 : p0;
      const uint64_t m = __ballot(in0 && incl > tg);
      const uint64_t pos = __ballot(v > 0.0);
      const int f = m ? (int)__builtin_ctzll(m) : -1;
      const double ex = wave_shr1_d(incl);          // exclusive prefix of every lane
      const double bf = f >= 0 ? lane_d(ex, f) : 0.0;  // the crossing segment's start (whole wave)
      if (tid == 0) {
        sh_res = rs;
        sh_target = tg;
        sh_found = f;
        sh_last = pos ? 63 - (int)__builtin_clzll(pos) : -1;
        sh_base = bf;
      }
    }
    __syncthreads();
    res = sh_res != 0;
    target = sh_target;
    found = sh_found;
    lastpos = sh_last;
    base = sh_base;
  } else {
    // totals of both weight kinds, a fixed-order batched scan over the segments
    double carry_r = 0.0, carry_p = 0.0;
    for (int j0 = 0; j0 < nseg; j0 += kWGD) {
      const int j = j0 + tid;
      double i1, e1, t1, i2, e2, t2;
      block_scan_d2<kWGD>(j < nseg ? seg[2 * j + 0] : 0.0, j < nseg ? seg[2 * j + 1] : 0.0, i1, e1, t1, i2, e2,
                          t2);
      carry_r += t1;
      carry_p += t2;
    }
    res = d.mode == kModeResidual && carry_r > 0.0;
    const int wsel = res ? 0 : 1;
    target = d.u * (res ? carry_r : carry_p);
    double carry = 0.0;
    for (int j0 = 0; j0 < nseg && found < 0; j0 += kWGD) {
      const int j = j0 + tid;
      const double v = j < nseg ? seg[2 * j + wsel] : 0.0;
      double incl, excl, tot, i2, e2, t2;
      block_scan_d2<kWGD>(v, 0.0, incl, excl, tot, i2, e2, t2);
      const int f = block_first_true<kWGD>(j < nseg && carry + incl > target);
      lastpos = max(lastpos, block_max_int<kWGD>(v > 0.0 ? j : -1));
      if (f >= 0 && tid == f) sh_base = carry + excl;
      __syncthreads();
      if (f >= 0) {
        found = j0 + f;
        base = sh_base;
      }
      carry += tot;
      __syncthreads();
    }
  }
  const bool resmode = d.mode == kModeResidual;
  const char* prow = row_ptr<ES>(P, b, d.a);
  const char* qrow = resmode ? P.draft + d.qoff * ES : prow;
  const WeightCtx w = make_ctx(d);
  int y = -1;  // no positive weight anywhere: only reachable outside the data contract
  if (found >= 0)
    y = draw_in_segment<ES, VEC>(prow, qrow, P.V, w, resmode, res, 1.0, found, base, target, false);
  else if (lastpos >= 0)
    y = draw_in_segment<ES, VEC>(prow, qrow, P.V, w, resmode, res, 1.0, lastpos, 0.0, 0.0, true);
  if (tid == 0) {
    P.out_tokens[(int64_t)b * (P.K + 1) + d.a] = y;
    if (P.ex_on && xw.valid) P.ex.out_ids[xw.o + d.a] = y;  // the chained expansion's bonus id
  }
}

// --------------------------------------------------------------- launch
// Workgroups of the dynamic row pass: K position blocks of (draft rows read:
// 2, else 1) x C1 chunks + a decider slot per request, then the bonus block.
static int64_t dyn_blocks(int64_t B, int64_t K, int64_t C1, bool dstats) {
  return K * B * ((dstats ? 1 : 2) * C1 + 1) + B * (C1 + 1);
}

bool verify_grids_fit(int32_t B, int32_t K, int32_t C1, int32_t nseg, bool dyn, bool dstats, int64_t ex_items) {
  const int64_t kMax = UINT32_MAX;  // work-items of one dispatch
  const int64_t rows = (int64_t)K + 1 + (dstats ? 0 : K);  // rows of the widest row-pass phase
  if (B > 65535 && (int64_t)B * rows * C1 * kWG > kMax) return false;  // the linear row-pass grid
  if (dyn && dyn_blocks(B, K, C1, dstats) * kWG > kMax) return false;
  if (((int64_t)B * nseg + ex_items) * 64 > kMax) return false;  // segment sums (+ a chained expansion)
  return (int64_t)B * kWGD <= kMax;  // the draw (the widest per-request launch)
}

template <int ES, bool VEC>
static hipError_t launch_typed(VerifyParams P, uint64_t phase_starts, hipEvent_t phase_event,
                               hipStream_t stream) {
  const int K = P.K;
  int lo = P.dyn ? K + 1 : 0;
  if (P.dyn) {  // one row pass with its decider slots
    P.ph_lo = 0;
    P.ph_nt = K + 1;
    P.ph_nd = K;
    P.ph_rd = P.dstats ? 0 : K;
    P.ph_check = P.phased = P.last_lo = 0;
    const int64_t g1 = dyn_blocks(P.B, K, P.C1, P.dstats != nullptr);
    hipLaunchKernelGGL((verify_rowstats_dyn_kernel<ES, VEC>), dim3((unsigned)g1), dim3(kWG), 0, stream, P);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  for (int j = 0; lo <= K; ++j) {  // phases [lo, hi), the last one ends past target row K
    int hi = lo + 1;
    while (hi <= K && !((phase_starts >> hi) & 1u)) ++hi;
    P.ph_lo = lo;
    P.ph_nt = hi - lo;
    P.ph_nd = min(hi, K) - lo;
    P.ph_rd = P.dstats ? 0 : P.ph_nd;  // with draft statistics the draft rows are not read here
    P.ph_check = j > 0;
    const int nr = P.ph_nt + P.ph_rd;
    const dim3 g1 = P.B <= 65535 ? dim3((unsigned)P.C1, (unsigned)nr, (unsigned)P.B)
                                 : dim3((unsigned)((int64_t)P.B * nr * P.C1));
    hipLaunchKernelGGL((verify_rowstats_kernel<ES, VEC>), g1, dim3(kWG), 0, stream, P);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (hi <= K) {
      hipLaunchKernelGGL((verify_phase_kernel<ES>), dim3((unsigned)P.B), dim3(kWG), 0, stream, P);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    P.last_lo = lo;
    P.phased = j > 0;
    lo = hi;
  }
  if (phase_event) {
    const hipError_t e = hipEventRecord(phase_event, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((verify_decide_kernel<ES>), dim3((unsigned)P.B), dim3(kWG), 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t g2 = (int64_t)P.B * P.nseg + (P.ex_on ? (int64_t)P.B * P.ex_G : 0);
  hipLaunchKernelGGL((verify_segsum_kernel<ES, VEC>), dim3((unsigned)g2), dim3(64), 0, stream, P);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_draw_kernel<ES, VEC>), dim3((unsigned)P.B), dim3(kWGD), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyParams& P, int dtype, bool vec, uint64_t phase_starts,
                         hipEvent_t phase_event, hipStream_t stream) {
  if (dtype == SPEC_BF16)
    return vec ? launch_typed<2, true>(P, phase_starts, phase_event, stream)
               : launch_typed<2, false>(P, phase_starts, phase_event, stream);
  return vec ? launch_typed<4, true>(P, phase_starts, phase_event, stream)
             : launch_typed<4, false>(P, phase_starts, phase_event, stream);
}

}  // namespace specv
