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
//  shard_draw    per request: the totals over shards, in shard order, give
//      u' * W and the shard holding the crossing; that shard alone finds the
//      token in its slice (segment scan, then one segment) and writes it as a
//      global id; the others leave -1 there, so a maximum over the shards'
//      outputs (the third exchange) yields it.
#include <float.h>
#include <limits.h>

#include "device_common.hpp"
#include "rowpass.hpp"
#include "sampling.hpp"
#include "verify_kernels.hpp"
#include "verify_layout.hpp"

namespace specv {

template <int ES>
__device__ __forceinline__ const char* shard_row(const ShardParams& P, int b, int r) {
  if (r <= P.K) return P.target + ((int64_t)b * P.t_req + (int64_t)r * P.t_row) * ES;
  return P.draft + ((int64_t)b * P.d_req + (int64_t)(r - P.K - 1) * P.d_row) * ES;
}

template <int ES, bool VEC>
__global__ __launch_bounds__(kWG) void shard_stats_kernel(ShardParams P) {
  const int b = blockIdx.x / P.R, r = blockIdx.x % P.R;
  const int k = r <= P.K ? r : r - P.K - 1;
  const float T = P.temperature[b];
  const int x = P.tokens[(int64_t)b * P.K + min(k, P.K - 1)];
  const bool greedy = T == 0.0f;
  ShardRec rec;
  rec.m = -INFINITY;
  rec.idx = INT_MAX;
  rec.s = 0.0;
  rec.z = 0.f;
  rec.has_z = 0;
  rec.pad = 0;
  if (temperature_valid(T) && !(greedy && r > P.K)) {  // greedy requests read no draft rows
    const char* row = shard_row<ES>(P, b, r);
    if (greedy) {
      const VI v = block_argmax(chunk_argmax<ES, VEC>(row, 0, P.Vs));
      rec.m = v.v;
      rec.idx = v.i + P.v0;
    } else {
      float s_hi, s_lo;
      temperature_scale(T, s_hi, s_lo);
      const MS v = block_merge_ms(chunk_stats<ES, VEC>(row, 0, P.Vs, s_hi, s_lo));
      rec.m = v.m;
      rec.s = v.s;
      if (k < P.K && x >= P.v0 && x - P.v0 < P.Vs) {
        rec.z = load_one<ES>(row, x - P.v0);
        rec.has_z = 1;
      }
    }
  }
  if (threadIdx.x == 0) P.recs[((int64_t)P.g * P.B + b) * P.R + r] = rec;
}

// The decision workgroup is 16 waves, so that each of a slice's segments
// (10 at a quarter of a 151936-token vocabulary) gets a wave of its own and
// the sampling row's segment sums take one round of loads.
constexpr int kDecideWG = 1024;
constexpr int kDecideWaves = kDecideWG / 64;

template <int ES, bool VEC>
__global__ __launch_bounds__(kDecideWG) void shard_decide_kernel(ShardParams P) {
  __shared__ float sm[2 * SPEC_MAX_K + 1];
  __shared__ double ss[2 * SPEC_MAX_K + 1];
  __shared__ float sz[2 * SPEC_MAX_K + 1];
  __shared__ int sg[SPEC_MAX_K + 1];
  __shared__ ReqDesc D;
  const int b = blockIdx.x, K = P.K, tid = threadIdx.x;
  const float T = P.temperature[b];
  const bool greedy = T == 0.0f;
  const int x = P.tokens[(int64_t)b * K + min(tid, K - 1)];
  bool mybad = !temperature_valid(T) || (tid < K && (x < 0 || x >= P.V));
  const int nrows = greedy ? K + 1 : P.R;
  if (tid < nrows && temperature_valid(T)) {
    // the G records of row tid, merged in shard order
    const ShardRec* rr = P.recs + (int64_t)b * P.R + tid;
    const int64_t stride = (int64_t)P.B * P.R;
    if (greedy) {
      VI best{rr[0].m, rr[0].idx};
      for (int h = 1; h < P.G; ++h) best = vi_pick(best, VI{rr[h * stride].m, rr[h * stride].idx});
      sg[tid] = best.i;
    } else {
      MS acc{rr[0].m, rr[0].s};
      float z = rr[0].z;
      for (int h = 1; h < P.G; ++h) {
        const ShardRec q = rr[h * stride];
        acc = ms_merge(acc, MS{q.m, q.s});
        if (q.has_z) z = q.z;
      }
      sm[tid] = acc.m;
      ss[tid] = acc.s;
      sz[tid] = z;
      mybad |= !(acc.s > 0.0 && acc.s <= DBL_MAX && fabsf(acc.m) <= FLT_MAX);
    }
  }
  const bool bad = __syncthreads_or(mybad) != 0;
  float s_hi = 0.f, s_lo = 0.f;
  if (!greedy && !bad) temperature_scale(T, s_hi, s_lo);
  const uint32_t k0 = (uint32_t)(P.seed & 0xffffffffu), k1 = (uint32_t)(P.seed >> 32);
  const uint32_t req = (uint32_t)b + P.request_base;
  if (tid < 64) {  // wave 0: one lane per draft position
    bool acc = false;
    if (tid < K && !bad) {
      if (greedy) {
        acc = x == sg[tid];
      } else {
        const double s_eff = (double)s_hi + (double)s_lo;
        const double p = exp2((double)sz[tid] * s_eff - (double)sm[tid]) / ss[tid];
        const double q = exp2((double)sz[K + 1 + tid] * s_eff - (double)sm[K + 1 + tid]) / ss[K + 1 + tid];
        const double thr = q > 0.0 ? fmin(1.0, p / q) : (p > 0.0 ? 1.0 : 0.0);
        acc = unit_uniform(philox4x32_10(req, (uint32_t)tid, P.step, 0u, k0, k1).w[0]) < thr;
      }
    }
    const uint64_t mask = __ballot(acc);
    const int a = bad ? -1 : (int)__builtin_ctzll(~mask);
    int32_t* out = P.out_tokens + (int64_t)b * (K + 1);
    for (int j = tid; j <= K; j += 64) {  // K <= 63: one pass
      int tok;
      if (bad || j > a) tok = -1;
      else if (j < a) tok = P.tokens[(int64_t)b * K + j];
      else tok = greedy ? sg[a] : -1;  // sampled: the owning shard's draw writes it
      out[j] = tok;
    }
    if (tid == 0) {
      P.accepted[b] = a;
      ReqDesc d;
      d.a = a;
      d.mode = (bad || greedy) ? kModeNone : (a < K ? kModeResidual : kModeBonus);
      d.s_hi = s_hi;
      d.s_lo = s_lo;
      d.mp = d.sp = d.mq = d.sq = d.u = 0.0;
      d.qoff = 0;
      if (d.mode != kModeNone) {
        d.mp = (double)sm[a];
        d.sp = ss[a];
        if (a < K) {
          d.mq = (double)sm[K + 1 + a];
          d.sq = ss[K + 1 + a];
        }
        d.u = unit_uniform(philox4x32_10(req, (uint32_t)a, P.step, 0u, k0, k1).w[1]);
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
  const char* qrow = res ? shard_row<ES>(P, b, K + 1 + D.a) : prow;
  WeightCtx w;
  w.s_hi = D.s_hi;
  w.s_lo = D.s_lo;
  w.negMp = -(float)D.mp;
  w.negMq = -(float)D.mq;
  const double c = res ? D.sp / D.sq : 0.0;
  w.c_hi = (float)c;
  w.c_lo = (float)(c - (double)w.c_hi);
  double* seg = P.seg + (int64_t)b * P.nseg * 2;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar segment bounds
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
  const char* qrow = resmode ? shard_row<ES>(P, b, P.K + 1 + d.a) : prow;
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
  SHARD_DISPATCH(shard_stats_kernel, (unsigned)(P.B * P.R), kWG);
}

hipError_t launch_shard_decide(const ShardParams& P, int dtype, bool vec, hipStream_t stream) {
  SHARD_DISPATCH(shard_decide_kernel, (unsigned)P.B, kDecideWG);
}

hipError_t launch_shard_draw(const ShardParams& P, int dtype, bool vec, hipStream_t stream) {
  SHARD_DISPATCH(shard_draw_kernel, (unsigned)P.B, kDrawThreads);
}

}  // namespace specv
