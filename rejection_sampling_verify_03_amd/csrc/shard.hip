// shard.hip -- verification with the vocabulary split over shards, as a
// tensor-parallel target holds its logits (MineDraft notes: a TP = 4
// verifier), each shard seeing only its slice [v0, v0 + Vs) of every row.
//
// The method is the one of the explainer page (sections "修正拒绝采样" and
// "核心思想"); only its data layout changes.  Every quantity it needs is a sum
// or a maximum over the vocabulary, so each shard reduces its slice and the
// shards exchange the reductions, never the logits:
//
//  shard_stats   per (request, row): the slice's S * 2^M (or max and global
//      argmax) and the logit at the position's draft token when the slice
//      holds it -> one 32-byte record; all shards' records are exchanged.
//  shard_decide  per request, on every shard: merges the G records of each
//      row in shard order, so every shard takes the same accept decisions and
//      writes the same outputs; then sums the residual (and p) weights of its
//      slice of the sampling row(s) per 4096-logit segment -> one (R_g, P_g)
//      pair per request; the pairs are exchanged.
//  shard_phase   (early exit only) between phases, per request on every
//      shard: the phase's accept tests from every shard's records of its
//      rows, leaving the same per-request state on every shard.
//  shard_draw    per request: the totals over shards, in shard order, give
//      u' * W and the shard holding the crossing; that shard alone finds the
//      token in its slice (segment scan, then one segment) and writes it as a
//      global id; the others leave -1 there, so a maximum over the shards'
//      outputs (the third exchange) yields it.
#include <float.h>
#include <limits.h>

#include "decision.hpp"
#include "device_common.hpp"
#include "rowpass.hpp"
#include "sampling.hpp"
#include "verify_kernels.hpp"
#include "verify_layout.hpp"

namespace specv {

// Drafts K_b of request b (ragged counts, else K), loaded unconditionally so
// it can be issued with other loads; -1 for a count outside [0, K].
__device__ __forceinline__ int shard_drafts_of(const ShardParams& P, int b) {
  const int32_t* t = P.num_drafts ? P.num_drafts : reinterpret_cast<const int32_t*>(P.temperature);
  const int v = t[b];
  const int kb = P.num_drafts ? v : P.K;
  return (kb >= 0 && kb <= P.K) ? kb : -1;
}

// The draft row table's entry for position k (clamped into [0, K); 0 without
// a table), loaded unconditionally; and whether it names a row of the buffer.
__device__ __forceinline__ int shard_draft_entry(const ShardParams& P, int b, int k) {
  const int32_t* t = P.dridx ? P.dridx : P.tokens;
  const int v = t[(int64_t)b * P.K + min(max(k, 0), P.K - 1)];
  return P.dridx ? v : 0;
}

__device__ __forceinline__ bool shard_entry_ok(const ShardParams& P, int di) {
  return !P.dridx || (uint32_t)di < (uint32_t)P.draft_rows;
}

// Element offset of draft row k of request b's slice from the draft base.
__device__ __forceinline__ int64_t shard_draft_off(const ShardParams& P, int b, int k, int di) {
  return P.dridx ? (int64_t)di * P.d_row : (int64_t)b * P.d_req + (int64_t)k * P.d_row;
}

// Row r of request b's slice: target rows 0..K, then draft rows K+1..2K.
template <int ES>
__device__ __forceinline__ const char* shard_row(const ShardParams& P, int b, int r, int di = 0) {
  if (r <= P.K) return P.target + ((int64_t)b * P.t_req + (int64_t)r * P.t_row) * ES;
  return P.draft + shard_draft_off(P, b, r - P.K - 1, di) * ES;
}

// Statistics of the rows of one phase (every row in one pass): one
// workgroup per (request, row) reduces this shard's slice of the row.  Rows
// that are not read write no record: draft rows of greedy requests, rows of
// requests that stopped in an earlier phase, rows past a request's drafts,
// and rows of a request whose draft count, token or row entry is out of
// range (such a request is invalid; no record of it is used).
template <int ES, bool VEC>
__global__ __launch_bounds__(kWG) void shard_stats_kernel(ShardParams P) {
  const int nr = P.ph_nt + P.ph_nd;
  const int b = blockIdx.x / nr, lr = blockIdx.x % nr;
  const int r = lr < P.ph_nt ? P.ph_lo + lr : P.K + 1 + P.ph_lo + (lr - P.ph_nt);
  const int k = r <= P.K ? r : r - P.K - 1;
  // independent loads, issued together (the state of a first phase is stale
  // and ignored; position K has no token)
  const float T = P.temperature[b];
  const int st = P.state[b];
  const int xt = P.tokens[(int64_t)b * P.K + min(k, P.K - 1)];
  const int di = shard_draft_entry(P, b, k);
  const int kb = shard_drafts_of(P, b);
  const bool greedy = T == 0.0f;
  const bool bad_t = !temperature_valid(T);
  const bool skip = bad_t | (greedy & (r > P.K)) | ((P.ph_check != 0) & (st != kStateAlive)) |
                    ((k < kb) & ((uint32_t)xt >= (uint32_t)P.V)) | ((r > P.K) & !shard_entry_ok(P, di)) |
                    (kb < 0) | ((r <= P.K) & (k > kb)) | ((r > P.K) & (k >= kb));
  if (skip) return;
  const int x = k < kb ? xt : -1;
  ShardRec rec;
  rec.m = -INFINITY;
  rec.idx = INT_MAX;
  rec.s = 0.0;
  rec.z = 0.f;
  rec.has_z = 0;
  rec.pad = 0;
  const char* row = shard_row<ES>(P, b, r, di);
  if (greedy) {
    const VI v = block_argmax(chunk_argmax<ES, VEC>(row, 0, P.Vs));
    rec.m = v.v;
    rec.idx = v.i + P.v0;
  } else {
    // the logit at the position's draft token, when the slice holds it: loaded
    // before the stream (clamped into the slice) so that nothing waits for it
    // after
    const bool has_x = x >= P.v0 && x - P.v0 < P.Vs;
    const float zx = load_one<ES>(row, min(max(x - P.v0, 0), P.Vs - 1));
    float s_hi, s_lo;
    temperature_scale(T, s_hi, s_lo);
    const MS v = block_merge_ms(chunk_stats<ES, VEC>(row, 0, P.Vs, s_hi, s_lo));
    rec.m = v.m;
    rec.s = v.s;
    if (has_x) {
      rec.z = zx;
      rec.has_z = 1;
    }
  }
  if (threadIdx.x == 0) P.recs[((int64_t)P.g * P.B + b) * P.R + r] = rec;
}

struct ShardShared {
  int64_t qoff[SPEC_MAX_K];     // draft row offsets of the positions
  float m[2 * SPEC_MAX_K + 1];
  double s[2 * SPEC_MAX_K + 1];
  float z[2 * SPEC_MAX_K + 1];  // logit of the row at its position's draft token
  int g[SPEC_MAX_K + 1];
  unsigned char bad[2 * SPEC_MAX_K + 1];  // a merged sampled row without a usable normaliser
  int a;
  int kb;
};

constexpr int kNotAliveShard = -3;  // shard_tests: the request stopped in an earlier phase

// The accept tests of request b over draft positions [lo, hi) from every
// shard's records, in the order of the unsharded decision: merges (in shard
// order) the records of target rows [lo, thi) and, for a sampled request,
// draft rows [lo, min(thi, K)); with known >= 0 no test runs and a = known.
// Returns, in every thread, a in [lo, hi] or -1 for invalid data (every
// draft token, the temperature, the draft count and the row entries are
// checked whatever the range; a row without a usable normaliser counts where
// the request stops, as in stop_position); with check_state, kNotAliveShard
// for a request that stopped earlier.  All threads of the workgroup call it.
__device__ int shard_tests(const ShardParams& P, int b, int lo, int hi, int thi, int known, bool invalid,
                           bool check_state, ShardShared& sh) {
  const int K = P.K;
  const int tid = threadIdx.x;
  const bool test = known < 0;
  const int st = P.state[b];
  const float T = P.temperature[b];
  const int kb_ = shard_drafts_of(P, b);
  const int x = P.tokens[(int64_t)b * K + min(tid, K - 1)];
  const int nt = thi - lo;
  const int nd = min(thi, K) - lo;
  const bool row_thread = tid < nt + nd && !invalid;
  const int r = tid < nt ? lo + tid : K + 1 + lo + (tid - nt);
  const int k = tid < nt ? r : r - K - 1;
  const int dix = shard_draft_entry(P, b, tid);
  const bool greedy = T == 0.0f;
  const int kb = max(kb_, 0);
  bool inbad = invalid || kb_ < 0 || !temperature_valid(T) || (tid < kb && (x < 0 || x >= P.V));
  if (!greedy && tid < kb) {
    inbad |= !shard_entry_ok(P, dix);  // a sampled request reads every draft row
    sh.qoff[tid] = shard_draft_off(P, b, tid, dix);
  }
  const bool row_exists = tid < nt ? k <= kb : k < kb;
  if (row_thread && row_exists && (!greedy || tid < nt) && temperature_valid(T)) {
    const ShardRec* rr = P.recs + (int64_t)b * P.R + r;
    const int64_t stride = (int64_t)P.B * P.R;
    if (greedy) {
      VI best{rr[0].m, rr[0].idx};
      for (int h = 1; h < P.G; ++h) best = vi_pick(best, VI{rr[h * stride].m, rr[h * stride].idx});
      sh.g[r] = best.i;
    } else {
      MS acc{rr[0].m, rr[0].s};
      float z = rr[0].z;
      for (int h = 1; h < P.G; ++h) {
        const ShardRec q = rr[h * stride];
        acc = ms_merge(acc, MS{q.m, q.s});
        if (q.has_z) z = q.z;
      }
      sh.m[r] = acc.m;
      sh.s[r] = acc.s;
      sh.z[r] = z;
      sh.bad[r] = !row_usable(acc.m, acc.s);
    }
  }
  const bool anybad = __syncthreads_or(inbad) != 0;
  if (check_state && st != kStateAlive) return kNotAliveShard;  // its records here were never written
  if (tid < 64) {  // wave 0: one lane per draft position
    const bool merged = !greedy && tid >= lo && tid < thi && tid < kb;
    const bool rowbad = merged && (sh.bad[tid] || sh.bad[K + 1 + tid]);
    const bool bonusbad = !greedy && kb >= lo && kb < thi && sh.bad[kb];
    bool acc = tid < lo;
    if (test && tid >= lo && tid < min(hi, kb) && !anybad && !rowbad) {
      if (greedy) {
        acc = x == sh.g[tid];
      } else {
        float dp, dq;
        acc = accept_test(T, sh.z[tid], sh.m[tid], sh.s[tid], sh.z[K + 1 + tid], sh.m[K + 1 + tid],
                          sh.s[K + 1 + tid], P.seed, (uint32_t)b + P.request_base, (uint32_t)tid, P.step, dp, dq);
      }
    }
    // lanes >= min(hi, K_b) fail: a <= min(hi, K_b)
    const int a = stop_position(test, lo, hi, thi, known, kb, acc, rowbad, bonusbad, anybad);
    if (tid == 0) {
      sh.a = a;
      sh.kb = kb;
    }
  }
  __syncthreads();
  return sh.a;
}

// Between early-exit phases: the accept tests of the phase's positions
// [ph_lo, ph_lo + ph_nd) for every request still alive, from every shard's
// records of the phase; one workgroup per request updates the state (every
// shard computes the same).
template <int ES>
__global__ __launch_bounds__(kWG) void shard_phase_kernel(ShardParams P) {
  __shared__ ShardShared sh;
  const int b = blockIdx.x;
  const int lo = P.ph_lo, hi = P.ph_lo + P.ph_nd;
  const int a = shard_tests(P, b, lo, hi, hi, -1, false, P.ph_check != 0, sh);
  if (a == kNotAliveShard) return;
  if (threadIdx.x == 0) P.state[b] = a < 0 ? kStateInvalid : (a < hi ? a : kStateAlive);
}

// The decision workgroup is 16 waves, so that each of a slice's segments
// (10 at a quarter of a 151936-token vocabulary) gets a wave of its own and
// the sampling row's segment sums take one round of loads.
constexpr int kDecideWG = 1024;
constexpr int kDecideWaves = kDecideWG / 64;

template <int ES, bool VEC>
__global__ __launch_bounds__(kDecideWG) void shard_decide_kernel(ShardParams P) {
  __shared__ ShardShared sh;
  __shared__ ReqDesc D;
  const int b = blockIdx.x, K = P.K, tid = threadIdx.x;
  int lo = 0, known = -1;
  bool invalid = false;
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
  const int a = shard_tests(P, b, lo, K, thi, known, invalid, false, sh);
  const float T = P.temperature[b];
  const bool greedy = T == 0.0f;
  const bool bad = a < 0;
  if (tid < 64) {
    int32_t* out = P.out_tokens + (int64_t)b * (K + 1);
    for (int j = tid; j <= K; j += 64) {  // K <= 63: one pass
      int tok;
      if (bad || j > a) tok = -1;
      else if (j < a) tok = P.tokens[(int64_t)b * K + j];
      else tok = greedy ? sh.g[a] : -1;  // sampled: the owning shard's draw writes it
      out[j] = tok;
    }
    if (tid == 0) {
      P.accepted[b] = a;
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
      P.desc[b] = d;
    }
  }
  __syncthreads();
  double* mass = P.masses + ((int64_t)P.g * P.B + b) * 2;
  if (D.mode == kModeNone) {
    if (tid == 0) mass[0] = mass[1] = 0.0;
    return;
  }
  // the residual and p weights of this shard's slice of the sampling row(s),
  // per segment, in units of 1 / S_p of the whole row
  const bool res = D.mode == kModeResidual;
  const char* prow = shard_row<ES>(P, b, D.a);
  const char* qrow = res ? P.draft + D.qoff * ES : prow;
  WeightCtx w;
  w.s_hi = D.s_hi;
  w.s_lo = D.s_lo;
  w.negMp = -(float)D.mp;
  w.negMq = -(float)D.mq;
  const double c = res ? D.sp / D.sq : 0.0;
  w.c_hi = (float)c;
  w.c_lo = (float)(c - (double)w.c_hi);
  double* seg = P.seg + (int64_t)b * P.nseg * 2;
  // each wave's running masses in segment order, kept in LDS for the total
  __shared__ double wr[kDecideWaves], wp[kDecideWaves];
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar segment bounds
  if (P.nseg <= kDecideWaves) {
    // one segment per wave (every slice up to 16 segments): its sums go to
    // LDS as well, and thread 0 totals them in segment order from there
    if (wave < P.nseg) {
      double rs, ps;
      if (res) segment_sums<ES, VEC, true>(prow, qrow, w, wave * kSeg, P.Vs, rs, ps);
      else segment_sums<ES, VEC, false>(prow, qrow, w, wave * kSeg, P.Vs, rs, ps);
      if (lane == 0) {
        seg[2 * wave] = rs;
        seg[2 * wave + 1] = ps;
        wr[wave] = rs;
        wp[wave] = ps;
      }
    }
    __syncthreads();
    if (tid == 0) {  // the slice's masses, summed in segment order
      double R = 0.0, Pm = 0.0;
      for (int j = 0; j < P.nseg; ++j) {
        R += wr[j];
        Pm += wp[j];
      }
      mass[0] = R;
      mass[1] = Pm;
    }
    return;
  }
  for (int j = wave; j < P.nseg; j += kDecideWaves) {
    double rs, ps;
    if (res) segment_sums<ES, VEC, true>(prow, qrow, w, j * kSeg, P.Vs, rs, ps);
    else segment_sums<ES, VEC, false>(prow, qrow, w, j * kSeg, P.Vs, rs, ps);
    if (lane == 0) {
      seg[2 * j] = rs;
      seg[2 * j + 1] = ps;
    }
  }
  __syncthreads();
  if (tid == 0) {  // the slice's masses, summed in segment order
    double R = 0.0, Pm = 0.0;
    for (int j = 0; j < P.nseg; ++j) {
      R += seg[2 * j];
      Pm += seg[2 * j + 1];
    }
    mass[0] = R;
    mass[1] = Pm;
  }
}

template <int ES, bool VEC>
__global__ __launch_bounds__(kDrawThreads) void shard_draw_kernel(ShardParams P) {
  constexpr int NT = kDrawThreads;
  const int b = blockIdx.x, tid = threadIdx.x;
  const ReqDesc d = P.desc[b];
  if (d.mode == kModeNone || d.a < 0 || d.a > P.K) return;
  // totals over the shards in shard order; the weights fall back to p when
  // the residual has no mass anywhere
  double Rt = 0.0, Pt = 0.0;
  for (int h = 0; h < P.G; ++h) {
    Rt += P.masses[((int64_t)h * P.B + b) * 2];
    Pt += P.masses[((int64_t)h * P.B + b) * 2 + 1];
  }
  const bool res = d.mode == kModeResidual && Rt > 0.0;
  const int wsel = res ? 0 : 1;
  const double target = d.u * (res ? Rt : Pt);
  // the owner: the first shard whose cumulative mass exceeds the target (else
  // the last shard with mass, for its last positive logit)
  int owner = -1, lastpos = -1;
  double base = 0.0, acc = 0.0;
  for (int h = 0; h < P.G; ++h) {
    const double m = P.masses[((int64_t)h * P.B + b) * 2 + wsel];
    if (m > 0.0) lastpos = h;
    if (owner < 0 && acc + m > target) {
      owner = h;
      base = acc;
    }
    acc += m;
  }
  const bool last_positive = owner < 0;
  if (last_positive) owner = lastpos;
  if (owner != P.g) return;
  const double* seg = P.seg + (int64_t)b * P.nseg * 2;
  __shared__ double sh_base;
  int found = -1, lastseg = -1;
  double sbase = base, carry = base;
  if (!last_positive) {
    for (int j0 = 0; j0 < P.nseg && found < 0; j0 += NT) {
      const int j = j0 + tid;
      const double v = j < P.nseg ? seg[2 * j + wsel] : 0.0;
      double incl, excl, tot, i2, e2, t2;
      block_scan_d2<NT>(v, 0.0, incl, excl, tot, i2, e2, t2);
      const int f = block_first_true<NT>(j < P.nseg && carry + incl > target);
      lastseg = max(lastseg, block_max_int<NT>(v > 0.0 ? j : -1));
      if (f >= 0 && tid == f) sh_base = carry + excl;
      __syncthreads();
      if (f >= 0) {
        found = j0 + f;
        sbase = sh_base;
      }
      carry += tot;
      __syncthreads();
    }
  } else {
    for (int j0 = 0; j0 < P.nseg; j0 += NT) {
      const int j = j0 + tid;
      const double v = j < P.nseg ? seg[2 * j + wsel] : 0.0;
      lastseg = max(lastseg, block_max_int<NT>(v > 0.0 ? j : -1));
    }
  }
  const bool resmode = d.mode == kModeResidual;
  const char* prow = shard_row<ES>(P, b, d.a);
  const char* qrow = resmode ? P.draft + d.qoff * ES : prow;
  WeightCtx w;
  w.s_hi = d.s_hi;
  w.s_lo = d.s_lo;
  w.negMp = -(float)d.mp;
  w.negMq = -(float)d.mq;
  const double c = resmode ? d.sp / d.sq : 0.0;
  w.c_hi = (float)c;
  w.c_lo = (float)(c - (double)w.c_hi);
  int y = -1;
  if (found >= 0)
    y = draw_in_segment<ES, VEC>(prow, qrow, P.Vs, w, resmode, res, 1.0, found, sbase, target, false);
  else if (lastseg >= 0)
    y = draw_in_segment<ES, VEC>(prow, qrow, P.Vs, w, resmode, res, 1.0, lastseg, 0.0, 0.0, true);
  if (tid == 0 && y >= 0) P.out_tokens[(int64_t)b * (P.K + 1) + d.a] = y + P.v0;
}

#define SHARD_DISPATCH(KERNEL, GRID, BLOCK)                                                           \
  do {                                                                                                \
    if (dtype == SPEC_BF16) {                                                                         \
      if (vec) hipLaunchKernelGGL((KERNEL<2, true>), dim3(GRID), dim3(BLOCK), 0, stream, P);           \
      else hipLaunchKernelGGL((KERNEL<2, false>), dim3(GRID), dim3(BLOCK), 0, stream, P);              \
    } else {                                                                                          \
      if (vec) hipLaunchKernelGGL((KERNEL<4, true>), dim3(GRID), dim3(BLOCK), 0, stream, P);           \
      else hipLaunchKernelGGL((KERNEL<4, false>), dim3(GRID), dim3(BLOCK), 0, stream, P);              \
    }                                                                                                 \
    return hipGetLastError();                                                                         \
  } while (0)

hipError_t launch_shard_stats(const ShardParams& P, int dtype, bool vec, hipStream_t stream) {
  SHARD_DISPATCH(shard_stats_kernel, (unsigned)(P.B * (P.ph_nt + P.ph_nd)), kWG);
}

hipError_t launch_shard_phase(const ShardParams& P, int dtype, bool vec, hipStream_t stream) {
  (void)vec;
  if (dtype == SPEC_BF16) hipLaunchKernelGGL((shard_phase_kernel<2>), dim3((unsigned)P.B), dim3(kWG), 0, stream, P);
  else hipLaunchKernelGGL((shard_phase_kernel<4>), dim3((unsigned)P.B), dim3(kWG), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_shard_decide(const ShardParams& P, int dtype, bool vec, hipStream_t stream) {
  SHARD_DISPATCH(shard_decide_kernel, (unsigned)P.B, kDecideWG);
}

hipError_t launch_shard_draw(const ShardParams& P, int dtype, bool vec, hipStream_t stream) {
  SHARD_DISPATCH(shard_draw_kernel, (unsigned)P.B, kDrawThreads);
}

}  // namespace specv
