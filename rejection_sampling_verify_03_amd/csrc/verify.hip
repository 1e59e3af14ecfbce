// verify.hip -- batched modified-rejection-sampling verification on gfx950.
//
// The method (explainer page on speculative decoding, sections "修正拒绝采样"
// and "核心思想"): draft token x_k is accepted with probability
// min(1, p_k(x_k) / q_k(x_k)); at the first rejection a token is resampled from
// normalize(max(0, p - q)); if all K drafts are accepted a bonus token is
// sampled from p_K.  Temperature 0 is the greedy limit (accept iff x_k is the
// target argmax, emit the target argmax where the request stops).
//
// Three kernels in stream order, no host round trip, and no communication
// between workgroups of one kernel (kernel boundaries make each kernel's
// writes visible to the next, so no atomics and no cache-maintenance fences):
//
//  verify_rowstats  one workgroup per (request, row, chunk of ~32K logits)
//      streams every row the parallel formulation needs exactly once (target
//      rows 0..K and, for sampled requests, draft rows 0..K-1) with 16-byte
//      loads, and reduces the chunk to S * 2^M = sum_v 2^(x_v * s - M)
//      (s = log2(e) / T, M an integer-valued reference raised by exact
//      power-of-two rescaling) or, for greedy requests, to (max, lowest
//      argmax).
//
//  verify_decide    one workgroup per (request, chunk): merges the request's
//      chunk partials in order, evaluates the K accept tests in parallel (one
//      lane per position, Philox uniforms, double-precision p(x), q(x)) and
//      finds a_b as the count of trailing ones of a wavefront ballot -- every
//      workgroup of the request derives the same decision; the chunk-0
//      workgroup writes the outputs -- then re-reads its chunk of the sampling
//      row(s) (p_a and q_a, or p_K for the bonus) and writes sums of the
//      residual weights max(0, p - q) and of p over 512-element segments.
//
//  verify_sample    one workgroup per sampled request scans the segment sums
//      for the inverse-CDF crossing of u' * R, recomputes the weights of that
//      one segment and finds the token with a wavefront scan.
#include <float.h>
#include <limits.h>

#include "device_common.hpp"
#include "verify_kernels.hpp"
#include "verify_layout.hpp"

namespace specv {

// log2(e) / T split as s_hi + s_lo with s_hi rounded toward zero and
// s_lo >= FLT_MIN (keeps -inf * s = -inf in both fma terms).
__device__ __forceinline__ void temperature_scale(float T, float& s_hi, float& s_lo) {
  const double s = 1.4426950408889634074 / (double)T;
  s_hi = __double2float_rz(s);
  s_lo = fmaxf(__double2float_rn(s - (double)s_hi), FLT_MIN);
}

__device__ __forceinline__ bool temperature_valid(float T) { return T >= 0.0f && T <= FLT_MAX; }

template <int ES>
__device__ __forceinline__ const char* row_ptr(const VerifyParams& P, int b, int r) {
  if (r <= P.K) return P.target + ((int64_t)b * P.t_req + (int64_t)r * P.t_row) * ES;
  return P.draft + ((int64_t)b * P.d_req + (int64_t)(r - P.K - 1) * P.d_row) * ES;
}

// Raise the reference exponent of a lane's running (M, S) to cover a new
// group maximum gm (the rescale is an exact power of two).
__device__ __forceinline__ void raise_ref(float& M, double& S, float gm, float s_hi) {
  const float gM = ceilf(gm * s_hi);
  if (gM > M) {
    S = ldexp(S, (int)fmaxf(M - gM, -2000.f));
    M = gM;
  }
}

__device__ __forceinline__ float sum8_exp(const float x[8], float s_hi, float s_lo, float negM) {
  float e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = scaled_exp2(x[i], s_hi, s_lo, negM);
  return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
}

// ------------------------------------------------------------ chunk passes
// Each thread takes groups tid, tid + 256, ...; the main loop issues U
// unconditional 16-byte loads per lane before using any of them, the
// remainder loop takes one group at a time, and the (< 8) trailing logits of a
// row whose length is not a multiple of 8 go to thread 0.
template <int ES, bool VEC>
__device__ __forceinline__ MS chunk_stats(const char* __restrict__ row, int e0, int e1, float s_hi,
                                          float s_lo) {
  constexpr int U = (ES == 2) ? 4 : 2;  // 64 bytes in flight per lane per iteration
  const int nfull = (e1 - e0) >> 3;
  float M = -INFINITY;
  double S = 0.0;
  int g = threadIdx.x;
  for (; g + (U - 1) * kWG < nfull; g += kWG * U) {
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) load_group<ES, VEC>(row, (int64_t)e0 + 8 * (int64_t)(g + u * kWG), x[u]);
    float gm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) gm = fmaxf(gm, x[u][i]);
    raise_ref(M, S, gm, s_hi);
    const float negM = -fmaxf(M, -1e30f);
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) acc += sum8_exp(x[u], s_hi, s_lo, negM);
    S += (double)acc;
  }
  for (; g < nfull; g += kWG) {
    float x[8];
    load_group<ES, VEC>(row, (int64_t)e0 + 8 * (int64_t)g, x);
    float gm = x[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) gm = fmaxf(gm, x[i]);
    raise_ref(M, S, gm, s_hi);
    S += (double)sum8_exp(x, s_hi, s_lo, -fmaxf(M, -1e30f));
  }
  const int t0 = e0 + 8 * nfull;
  if (t0 < e1 && threadIdx.x == 0) {
    for (int e = t0; e < e1; ++e) {
      const float x = load_one<ES>(row, e);
      raise_ref(M, S, x, s_hi);
      S += (double)scaled_exp2(x, s_hi, s_lo, -fmaxf(M, -1e30f));
    }
  }
  return MS{M, S};
}

template <int ES, bool VEC>
__device__ __forceinline__ VI chunk_argmax(const char* __restrict__ row, int e0, int e1) {
  constexpr int U = (ES == 2) ? 4 : 2;
  const int nfull = (e1 - e0) >> 3;
  VI best{-INFINITY, INT_MAX};
  int g = threadIdx.x;
  for (; g + (U - 1) * kWG < nfull; g += kWG * U) {
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) load_group<ES, VEC>(row, (int64_t)e0 + 8 * (int64_t)(g + u * kWG), x[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 8; ++i) best = vi_pick(best, VI{x[u][i], e0 + 8 * (g + u * kWG) + i});
  }
  for (; g < nfull; g += kWG) {
    float x[8];
    load_group<ES, VEC>(row, (int64_t)e0 + 8 * (int64_t)g, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) best = vi_pick(best, VI{x[i], e0 + 8 * g + i});
  }
  const int t0 = e0 + 8 * nfull;
  if (t0 < e1 && threadIdx.x == 0)
    for (int e = t0; e < e1; ++e) best = vi_pick(best, VI{load_one<ES>(row, e), e});
  return best;
}

__device__ __forceinline__ MS block_merge_ms(MS v) {
  __shared__ float sm[kWaves];
  __shared__ double ss[kWaves];
  v = wave_merge_ms(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[w] = v.m;
    ss[w] = v.s;
  }
  __syncthreads();
  MS r{sm[0], ss[0]};
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = ms_merge(r, MS{sm[i], ss[i]});
  return r;
}

__device__ __forceinline__ VI block_argmax(VI v) {
  __shared__ float sv[kWaves];
  __shared__ int si[kWaves];
  v = wave_argmax(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sv[w] = v.v;
    si[w] = v.i;
  }
  __syncthreads();
  VI r{sv[0], si[0]};
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = vi_pick(r, VI{sv[i], si[i]});
  return r;
}

// ------------------------------------------------------------- decision
struct Decision {
  int a;     // accepted drafts, -1 for invalid request data
  int mode;  // kModeNone / kModeResidual / kModeBonus
  float s_hi, s_lo;
  double mp, sp, mq, sq, u;
};

// The decision of request b, computed by the whole workgroup into `D`
// (shared).  With `write`, the outputs of the request are written too.
template <int ES>
__device__ void decide(const VerifyParams& P, int b, bool write, Decision& D) {
  __shared__ float sh_m[2 * SPEC_MAX_K + 1];
  __shared__ double sh_s[2 * SPEC_MAX_K + 1];
  __shared__ int sh_g[SPEC_MAX_K + 1];
  __shared__ int sh_bad;
  const int K = P.K;
  const int tid = threadIdx.x;
  const float T = P.temperature[b];
  const bool greedy = (T == 0.0f);
  if (tid == 0) sh_bad = temperature_valid(T) ? 0 : 1;
  __syncthreads();
  int x = 0;
  if (tid < K) {
    x = P.tokens[(int64_t)b * K + tid];
    if (x < 0 || x >= P.V) atomicOr(&sh_bad, 1);
  }
  const int nrows = greedy ? K + 1 : P.R;
  if (tid < nrows) {
    const RowPartial* rp = P.rowp + ((int64_t)b * P.R + tid) * P.C;
    if (greedy) {
      VI best{rp[0].m, rp[0].idx};
      for (int c = 1; c < P.C; ++c) best = vi_pick(best, VI{rp[c].m, rp[c].idx});
      sh_g[tid] = best.i;
    } else {
      MS acc{rp[0].m, rp[0].s};
      for (int c = 1; c < P.C; ++c) acc = ms_merge(acc, MS{rp[c].m, rp[c].s});
      sh_m[tid] = acc.m;
      sh_s[tid] = acc.s;
      if (!(acc.s > 0.0 && acc.s <= DBL_MAX && fabsf(acc.m) <= FLT_MAX)) atomicOr(&sh_bad, 1);
    }
  }
  __syncthreads();
  const bool bad = sh_bad != 0;
  float s_hi = 0.f, s_lo = 0.f;
  if (!greedy && !bad) temperature_scale(T, s_hi, s_lo);
  const uint32_t k0 = (uint32_t)(P.seed & 0xffffffffu), k1 = (uint32_t)(P.seed >> 32);
  const uint32_t req = (uint32_t)b + P.request_base;

  if (tid < 64) {  // wave 0: one lane per draft position
    bool acc = false;
    float dp = 0.f, dq = 0.f;
    if (tid < K && !bad) {
      if (greedy) {
        acc = (x == sh_g[tid]);
      } else {
        const double s_eff = (double)s_hi + (double)s_lo;
        const double zt = (double)load_one<ES>(row_ptr<ES>(P, b, tid), x);
        const double zq = (double)load_one<ES>(row_ptr<ES>(P, b, K + 1 + tid), x);
        const double p = exp2(zt * s_eff - (double)sh_m[tid]) / sh_s[tid];
        const double q = exp2(zq * s_eff - (double)sh_m[K + 1 + tid]) / sh_s[K + 1 + tid];
        const double thr = q > 0.0 ? fmin(1.0, p / q) : (p > 0.0 ? 1.0 : 0.0);
        const Philox4 r = philox4x32_10(req, (uint32_t)tid, P.step, 0u, k0, k1);
        acc = unit_uniform(r.w[0]) < thr;
        dp = (float)p;
        dq = (float)q;
      }
    }
    const uint64_t mask = __ballot(acc);
    const int a = bad ? -1 : (int)__builtin_ctzll(~mask);  // lanes >= K never accept, so a <= K
    if (write) {
      if (P.debug && tid < K) {
        P.debug[((int64_t)b * K + tid) * 2 + 0] = dp;
        P.debug[((int64_t)b * K + tid) * 2 + 1] = dq;
      }
      int32_t* out = P.out_tokens + (int64_t)b * (K + 1);
      for (int j = tid; j <= K; j += 64) {  // K <= 63: one pass
        int tok;
        if (bad || j > a) tok = -1;
        else if (j < a) tok = P.tokens[(int64_t)b * K + j];
        else tok = greedy ? sh_g[a] : -1;  // sampled: written by the sampling kernel
        if (!(j == a && !greedy && !bad)) out[j] = tok;
      }
      if (tid == 0) P.accepted[b] = a;
    }
    if (tid == 0) {
      D.a = a;
      D.mode = (bad || greedy) ? kModeNone : (a < K ? kModeResidual : kModeBonus);
      D.s_hi = s_hi;
      D.s_lo = s_lo;
      D.mp = D.sp = D.mq = D.sq = D.u = 0.0;
      if (D.mode != kModeNone) {
        D.mp = (double)sh_m[a];
        D.sp = sh_s[a];
        if (a < K) {
          D.mq = (double)sh_m[K + 1 + a];
          D.sq = sh_s[K + 1 + a];
        }
        D.u = unit_uniform(philox4x32_10(req, (uint32_t)a, P.step, 0u, k0, k1).w[1]);
      }
      if (write) {
        ReqDesc d;
        d.mode = D.mode;
        d.a = D.a;
        d.s_hi = D.s_hi;
        d.s_lo = D.s_lo;
        d.mp = D.mp;
        d.sp = D.sp;
        d.mq = D.mq;
        d.sq = D.sq;
        d.u = D.u;
        d.pad = 0.0;
        P.desc[b] = d;
      }
    }
  }
  __syncthreads();
}

template <int ES, bool VEC>
__global__ __launch_bounds__(kWG) void verify_rowstats_kernel(VerifyParams P) {
  const int c = blockIdx.x % P.C;
  const int r = (blockIdx.x / P.C) % P.R;
  const int b = blockIdx.x / (P.C * P.R);
  const float T = P.temperature[b];
  const bool greedy = (T == 0.0f);
  if (greedy && r > P.K) return;  // greedy requests read no draft rows
  const char* row = row_ptr<ES>(P, b, r);
  const int e0 = c * P.chunk;
  const int e1 = min(P.V, e0 + P.chunk);
  RowPartial part;
  if (greedy) {
    const VI v = block_argmax(chunk_argmax<ES, VEC>(row, e0, e1));
    part.m = v.v;
    part.idx = v.i;
    part.s = 0.0;
  } else {
    float s_hi, s_lo;
    temperature_scale(T, s_hi, s_lo);
    const MS v = block_merge_ms(chunk_stats<ES, VEC>(row, e0, e1, s_hi, s_lo));
    part.m = v.m;
    part.idx = 0;
    part.s = v.s;
  }
  if (threadIdx.x == 0) P.rowp[((int64_t)b * P.R + r) * P.C + c] = part;
}

// ------------------------------------------------------- sampling pass
// Sampling weight of one logit pair: p(v) (bonus) or max(0, p(v) - q(v)).
struct WeightCtx {
  float s_hi, s_lo, negMp, negMq;
  double ip, iq;
};

__device__ __forceinline__ void pair_weights(const WeightCtx& w, float xp, float xq, bool res, double& r,
                                             double& pv) {
  pv = (double)scaled_exp2(xp, w.s_hi, w.s_lo, w.negMp) * w.ip;
  if (res) {
    const double qv = (double)scaled_exp2(xq, w.s_hi, w.s_lo, w.negMq) * w.iq;
    r = fmax(pv - qv, 0.0);
  } else {
    r = pv;
  }
}

__device__ __forceinline__ WeightCtx make_ctx(const ReqDesc& d) {
  WeightCtx w;
  w.s_hi = d.s_hi;
  w.s_lo = d.s_lo;
  w.negMp = -(float)d.mp;
  w.negMq = -(float)d.mq;
  w.ip = 1.0 / d.sp;
  w.iq = d.mode == kModeResidual ? 1.0 / d.sq : 0.0;
  return w;
}

// 8 consecutive logits from e0 on, -inf past the row end e1.
template <int ES, bool VEC>
__device__ __forceinline__ void load_group_bounded(const char* row, int e0, int e1, float x[8]) {
  if (e0 + 8 <= e1) {
    load_group<ES, VEC>(row, e0, x);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (e0 + i < e1) ? load_one<ES>(row, e0 + i) : -INFINITY;
  }
}

// Sums of the sampling weights over one tile (256 groups = 4 segments of 512
// logits, one per wave) -> the segment sums of the residual and of p.
template <int U>
__device__ __forceinline__ void tile_segment_sums(const WeightCtx& w, bool res, const float (&xp)[U][8],
                                                  const float (&xq)[U][8], int seg0, int e1,
                                                  double* __restrict__ seg) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    double rs = 0.0, ps = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      double r, pv;
      pair_weights(w, xp[u][i], xq[u][i], res, r, pv);
      rs += r;
      ps += pv;
    }
    rs = wave_sum_d(rs);
    ps = wave_sum_d(ps);
    const int s_idx = seg0 + u * kWaves + wave;
    if (lane == 0 && s_idx * kSeg < e1) {
      seg[2 * s_idx + 0] = rs;
      seg[2 * s_idx + 1] = ps;
    }
  }
}

template <int ES, bool VEC, bool RES>
__device__ __forceinline__ void residual_chunk(const VerifyParams& P, int b, int c, const ReqDesc& d,
                                               double* __restrict__ seg) {
  constexpr int U = (ES == 2) ? 2 : 1;
  const char* prow = row_ptr<ES>(P, b, d.a);
  const char* qrow = RES ? row_ptr<ES>(P, b, P.K + 1 + d.a) : prow;
  const WeightCtx w = make_ctx(d);
  const int e0 = c * P.chunk;
  const int e1 = min(P.V, e0 + P.chunk);
  const int nfull = (e1 - e0) >> 3;
  const int ngroups = (e1 - e0 + 7) >> 3;
  const int tid = threadIdx.x;
  int tile = 0;
  for (; (tile + U) * kWG <= nfull; tile += U) {  // tiles of full groups only
    float xp[U][8], xq[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gg = (tile + u) * kWG + tid;
      load_group<ES, VEC>(prow, (int64_t)e0 + 8 * gg, xp[u]);
      if (RES) load_group<ES, VEC>(qrow, (int64_t)e0 + 8 * gg, xq[u]);
      else {
#pragma unroll
        for (int i = 0; i < 8; ++i) xq[u][i] = 0.f;
      }
    }
    tile_segment_sums<U>(w, RES, xp, xq, e0 / kSeg + tile * kWaves, e1, seg);
  }
  for (; tile * kWG < ngroups; ++tile) {  // the last, partly filled tiles
    float xp[1][8], xq[1][8];
    const int gg = tile * kWG + tid;
    if (gg < ngroups) {
      load_group_bounded<ES, VEC>(prow, e0 + 8 * gg, e1, xp[0]);
      if (RES) load_group_bounded<ES, VEC>(qrow, e0 + 8 * gg, e1, xq[0]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) xp[0][i] = -INFINITY;
    }
    if (!RES || gg >= ngroups) {
#pragma unroll
      for (int i = 0; i < 8; ++i) xq[0][i] = RES ? -INFINITY : 0.f;
    }
    tile_segment_sums<1>(w, RES, xp, xq, e0 / kSeg + tile * kWaves, e1, seg);
  }
}

// Inclusive / exclusive scan of one double per thread over the workgroup, in
// a fixed order; `total` is the workgroup sum.  All threads must call it.
__device__ __forceinline__ void block_scan_d(double v, double& incl, double& excl, double& total) {
  __shared__ double wt[kWaves];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  double xe = __shfl_up(x, 1, 64);
  if (lane == 0) xe = 0.0;
  if (lane == 63) wt[w] = x;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) base += wt[i];
    tot += wt[i];
  }
  incl = base + x;
  excl = base + xe;
  total = tot;
  __syncthreads();
}

// Lowest thread index whose predicate holds, or -1.  All threads must call it.
__device__ __forceinline__ int block_first_true(bool pred) {
  __shared__ int first[kWaves];
  const uint64_t m = __ballot(pred);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) first[w] = m ? (int)__builtin_ctzll(m) + 64 * w : -1;
  __syncthreads();
  int r = -1;
#pragma unroll
  for (int i = kWaves - 1; i >= 0; --i)
    if (first[i] >= 0) r = first[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ int block_max_int(int v) {
  __shared__ int mx[kWaves];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) mx[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = mx[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = max(r, mx[i]);
  __syncthreads();
  return r;
}

// Within segment j (run by wave 0): the first element whose cumulative weight
// (starting from `base`) exceeds `target`, or with `last_positive`, the last
// element of positive weight.
template <int ES, bool VEC>
__device__ int search_segment(const VerifyParams& P, int b, const ReqDesc& d, bool res, int j,
                              double base, double target, bool last_positive) {
  const int lane = threadIdx.x & 63;
  const char* prow = row_ptr<ES>(P, b, d.a);
  const char* qrow = d.mode == kModeResidual ? row_ptr<ES>(P, b, P.K + 1 + d.a) : prow;
  const WeightCtx w = make_ctx(d);
  const int e0 = j * kSeg + 8 * lane;
  const int e1 = P.V;
  float xp[8], xq[8];
  if (e0 < e1) {
    load_group_bounded<ES, VEC>(prow, e0, e1, xp);
    load_group_bounded<ES, VEC>(qrow, e0, e1, xq);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) xp[i] = xq[i] = -INFINITY;
  }
  double wt[8];
  double ls = 0.0;
  int lastpos = -1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    double r, pv;
    pair_weights(w, xp[i], xq[i], d.mode == kModeResidual, r, pv);
    wt[i] = res ? r : pv;
    ls += wt[i];
    if (wt[i] > 0.0) lastpos = e0 + i;
  }
  // inclusive / exclusive wave scan of the lane sums
  double x = ls;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  double xe = __shfl_up(x, 1, 64);
  if (lane == 0) xe = 0.0;
  int pick = -1;
  if (!last_positive) {
    const uint64_t m = __ballot(base + x > target);
    if (m) {
      const int L = (int)__builtin_ctzll(m);
      if (lane == L) {
        double run = base + xe;
        for (int i = 0; i < 8; ++i) {
          run += wt[i];
          if (wt[i] > 0.0 && target < run) {
            pick = e0 + i;
            break;
          }
        }
        if (pick < 0) pick = lastpos;  // cumulative rounding: stay inside this lane
      }
      for (int off = 32; off >= 1; off >>= 1) pick = max(pick, __shfl_xor(pick, off, 64));
      return pick;
    }
  }
  // the last element of positive weight in the segment
  pick = lastpos;
  for (int off = 32; off >= 1; off >>= 1) pick = max(pick, __shfl_xor(pick, off, 64));
  return pick;
}

template <int ES, bool VEC>
__device__ void sample(const VerifyParams& P, int b, const ReqDesc& d, const double* __restrict__ seg) {
  __shared__ int sh_pick;
  __shared__ double sh_base;
  const int tid = threadIdx.x;
  const int nseg = P.nseg;
  // totals of both weight kinds, as a fixed-order batched scan over segments
  double carry_r = 0.0, carry_p = 0.0;
  for (int j0 = 0; j0 < nseg; j0 += kWG) {
    const int j = j0 + tid;
    const double vr = j < nseg ? seg[2 * j + 0] : 0.0;
    const double vp = j < nseg ? seg[2 * j + 1] : 0.0;
    double i1, e1, t1, i2, e2, t2;
    block_scan_d(vr, i1, e1, t1);
    block_scan_d(vp, i2, e2, t2);
    carry_r += t1;
    carry_p += t2;
  }
  const bool res = d.mode == kModeResidual && carry_r > 0.0;
  const int wsel = res ? 0 : 1;
  const double W = res ? carry_r : carry_p;
  const double target = d.u * W;
  // first segment whose cumulative weight exceeds target
  double carry = 0.0;
  int found = -1, lastpos = -1;
  double base = 0.0;
  for (int j0 = 0; j0 < nseg && found < 0; j0 += kWG) {
    const int j = j0 + tid;
    const double v = j < nseg ? seg[2 * j + wsel] : 0.0;
    double incl, excl, tot;
    block_scan_d(v, incl, excl, tot);
    const int f = block_first_true(j < nseg && carry + incl > target);
    lastpos = max(lastpos, block_max_int(v > 0.0 ? j : -1));
    if (f >= 0 && tid == f) sh_base = carry + excl;
    __syncthreads();
    if (f >= 0) {
      found = j0 + f;
      base = sh_base;
    }
    carry += tot;
    __syncthreads();
  }
  if (tid < 64) {
    int y = -1;  // no positive weight anywhere: only reachable outside the data contract
    if (found >= 0) y = search_segment<ES, VEC>(P, b, d, res, found, base, target, false);
    else if (lastpos >= 0) y = search_segment<ES, VEC>(P, b, d, res, lastpos, 0.0, 0.0, true);
    if (tid == 0) sh_pick = y;
  }
  __syncthreads();
  if (tid == 0) P.out_tokens[(int64_t)b * (P.K + 1) + d.a] = sh_pick;
}

template <int ES, bool VEC>
__global__ __launch_bounds__(kWG) void verify_decide_kernel(VerifyParams P) {
  const int c = blockIdx.x % P.C;
  const int b = blockIdx.x / P.C;
  __shared__ Decision D;
  decide<ES>(P, b, c == 0, D);
  if (D.mode == kModeNone) return;
  ReqDesc d;
  d.mode = D.mode;
  d.a = D.a;
  d.s_hi = D.s_hi;
  d.s_lo = D.s_lo;
  d.mp = D.mp;
  d.sp = D.sp;
  d.mq = D.mq;
  d.sq = D.sq;
  d.u = D.u;
  double* seg = P.seg + (int64_t)b * P.nseg * 2;
  if (D.mode == kModeResidual) residual_chunk<ES, VEC, true>(P, b, c, d, seg);
  else residual_chunk<ES, VEC, false>(P, b, c, d, seg);
}

template <int ES, bool VEC>
__global__ __launch_bounds__(kWG) void verify_sample_kernel(VerifyParams P) {
  const int b = blockIdx.x;
  const ReqDesc d = P.desc[b];
  if (d.mode == kModeResidual) {
    if (d.a < 0 || d.a >= P.K) return;
  } else if (d.mode == kModeBonus) {
    if (d.a != P.K) return;
  } else {
    return;  // greedy or invalid: nothing to sample
  }
  sample<ES, VEC>(P, b, d, P.seg + (int64_t)b * P.nseg * 2);
}

// --------------------------------------------------------------- launch
template <int ES, bool VEC>
static hipError_t launch_typed(const VerifyParams& P, hipEvent_t phase_event, hipStream_t stream) {
  const int64_t g1 = (int64_t)P.B * P.R * P.C;
  const int64_t g2 = (int64_t)P.B * P.C;
  hipLaunchKernelGGL((verify_rowstats_kernel<ES, VEC>), dim3((unsigned)g1), dim3(kWG), 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (phase_event) {
    e = hipEventRecord(phase_event, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((verify_decide_kernel<ES, VEC>), dim3((unsigned)g2), dim3(kWG), 0, stream, P);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((verify_sample_kernel<ES, VEC>), dim3((unsigned)P.B), dim3(kWG), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_verify(const VerifyParams& P, int dtype, bool vec, hipEvent_t phase_event,
                         hipStream_t stream) {
  if (dtype == SPEC_BF16)
    return vec ? launch_typed<2, true>(P, phase_event, stream) : launch_typed<2, false>(P, phase_event, stream);
  return vec ? launch_typed<4, true>(P, phase_event, stream) : launch_typed<4, false>(P, phase_event, stream);
}

}  // namespace specv
