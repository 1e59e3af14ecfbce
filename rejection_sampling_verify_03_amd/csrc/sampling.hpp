// sampling.hpp -- device pieces shared by the samplers (the verification's
// draw and segment sums, their vocab-sharded forms, and the draft-token
// statistics pass's bounded loads): the per-logit sampling weights, bounded
// group loads, workgroup scans and searches, and the search for the
// inverse-CDF crossing inside one 4096-logit segment.
#pragma once

#include "device_common.hpp"
#include "verify_layout.hpp"

namespace specv {

constexpr int kDrawThreads = 512;  // draw workgroup: 8 waves, one 512-logit block each
static_assert(kDrawThreads / 64 * 512 == kSeg, "a draw wave per 512-logit block of a segment");

// The draw samples from r = max(0, p - q) (or from p for the bonus).  With
// e_p = 2^(x_p s - M_p), e_q = 2^(x_q s - M_q) and the normalisers S_p, S_q,
// r = max(0, e_p - e_q * c) / S_p with c = S_p / S_q.  The weights are kept in
// units of 1 / S_p (a common factor that cancels in the inverse CDF) and
// computed in fp32 with c split as c_hi + c_lo: each fma rounds once,
// relative to the result, so the residual keeps ~1e-7 relative accuracy even
// where p and q nearly cancel.
struct WeightCtx {
  float s_hi, s_lo, negMp, negMq, c_hi, c_lo;
};

// Weight of one logit pair: residual (res) or p, in units of 1 / S_p.
__device__ __forceinline__ float pair_weight(const WeightCtx& w, float xp, float xq, bool res, float& ep) {
  ep = scaled_exp2(xp, w.s_hi, w.s_lo, w.negMp);
  if (!res) return ep;
  const float eq = scaled_exp2(xq, w.s_hi, w.s_lo, w.negMq);
  const float t = __builtin_fmaf(-eq, w.c_lo, __builtin_fmaf(-eq, w.c_hi, ep));
  return fmaxf(t, 0.0f);
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

// A group of 8 logits from e0 on, -inf past the row end V (scalar loads for a
// group that straddles the end).
template <int ES, bool VEC>
__device__ __forceinline__ RawGroup<ES, VEC> load_raw_bounded(const char* row, int e0, int V) {
  if (e0 + 8 <= V) return load_raw<ES, VEC>(row, e0);
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (e0 + i < V) ? load_one<ES>(row, e0 + i) : -INFINITY;
  RawGroup<ES, VEC> r;
  if constexpr (!VEC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) r.x[i] = x[i];
  } else if constexpr (ES == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (__float_as_uint(x[2 * i]) >> 16) | (__float_as_uint(x[2 * i + 1]) & 0xffff0000u);
    r.v = u32x4{w[0], w[1], w[2], w[3]};
  } else {
    r.a = f32x4{x[0], x[1], x[2], x[3]};
    r.b = f32x4{x[4], x[5], x[6], x[7]};
  }
  return r;
}

template <int NT>
__device__ __forceinline__ int block_first_true(bool pred) {
  constexpr int W = NT / 64;
  __shared__ int first[W];
  const uint64_t m = __ballot(pred);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) first[w] = m ? (int)__builtin_ctzll(m) + 64 * w : -1;
  __syncthreads();
  int r = -1;
#pragma unroll
  for (int i = W - 1; i >= 0; --i)
    if (first[i] >= 0) r = first[i];
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ int block_max_int(int v) {
  constexpr int W = NT / 64;
  __shared__ int mx[W];
  v = wave_max_i(v);
  if ((threadIdx.x & 63) == 0) mx[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = mx[0];
#pragma unroll
  for (int i = 1; i < W; ++i) r = max(r, mx[i]);
  __syncthreads();
  return r;
}

// Inside segment j of a row of V logits (q's row read only with resmode): the
// first logit whose cumulative weight (from `base`) exceeds `target`, or with
// `last_positive` the last logit of positive weight.  The weights are
// pair_weight's residual (res) or p, times `scale` (an exact power of two
// that brings them to the units of base and target).  Wave w recomputes the
// weights of block w (512 logits); the crossing block is found from the block
// totals in order, then the crossing lane and logit.  All kDrawThreads
// threads of the workgroup call it.
template <int ES, bool VEC>
__device__ int draw_in_segment(const char* prow, const char* qrow, int V, const WeightCtx& w, bool resmode,
                               bool res, double scale, int j, double base, double target, bool last_positive) {
  constexpr int W = kDrawThreads / 64;
  __shared__ double blk_tot[W];
  __shared__ int blk_last[W];
  __shared__ int sh_w, sh_mode;
  __shared__ double sh_base;
  __shared__ int sh_pick;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = j * kSeg + wave * 512 + 8 * lane;
  float xp[8], xq[8];
  if (e0 < V) {
    load_group_bounded<ES, VEC>(prow, e0, V, xp);
    if (resmode) load_group_bounded<ES, VEC>(qrow, e0, V, xq);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) xp[i] = -INFINITY;
  }
  if (!resmode || e0 >= V) {
#pragma unroll
    for (int i = 0; i < 8; ++i) xq[i] = resmode ? -INFINITY : 0.f;
  }
  double wt[8];
  double ls = 0.0;
  int lastpos = -1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float ep;
    const float r = pair_weight(w, xp[i], xq[i], resmode, ep);
    wt[i] = (double)(res ? r : ep) * scale;
    ls += wt[i];
    if (wt[i] > 0.0) lastpos = e0 + i;
  }
  const double x = wave_scan_d(ls);  // DPP: fixed order, no LDS round trips
  const double xe = wave_shr1_d(x);
  const double wtotal = lane_d(x, 63);
  const int wl = wave_max_i(lastpos);
  if (lane == 0) {
    blk_tot[wave] = wtotal;
    blk_last[wave] = wl;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int wsel = -1, mode = 1;  // 0: search the block, 1: its last positive logit
    double acc = base;
    if (!last_positive) {
      for (int i = 0; i < W; ++i) {
        if (acc + blk_tot[i] > target) {
          wsel = i;
          mode = 0;
          break;
        }
        acc += blk_tot[i];
      }
    }
    if (wsel < 0)
      for (int i = 0; i < W; ++i)
        if (blk_last[i] >= 0) wsel = i;
    sh_w = wsel;
    sh_mode = mode;
    sh_base = acc;
    sh_pick = -1;
  }
  __syncthreads();
  if (wave == sh_w) {
    int pick = -1;
    if (sh_mode == 0) {
      const uint64_t m = __ballot(sh_base + x > target);
      const int L = m ? (int)__builtin_ctzll(m) : 63;
      if (lane == L) {
        double run = sh_base + xe;
        for (int i = 0; i < 8; ++i) {
          run += wt[i];
          if (wt[i] > 0.0 && target < run) {
            pick = e0 + i;
            break;
          }
        }
        if (pick < 0) pick = lastpos;  // cumulative rounding: stay inside this lane
      }
      pick = lane_i(pick, L);
      if (pick < 0) pick = blk_last[wave];
    } else {
      pick = blk_last[wave];
    }
    if (lane == 0) sh_pick = pick;
  }
  __syncthreads();
  return sh_pick;
}

// Inclusive and exclusive scans of two doubles per thread over the workgroup in
// one pass (fixed order); totals of both.  All threads must call it.
template <int NT>
__device__ __forceinline__ void block_scan_d2(double v0, double v1, double& incl0, double& excl0, double& tot0,
                                              double& incl1, double& excl1, double& tot1) {
  constexpr int W = NT / 64;
  __shared__ double wt[2][W];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double x0 = wave_scan_d(v0), x1 = wave_scan_d(v1);  // DPP, fixed order
  const double e0 = wave_shr1_d(x0), e1 = wave_shr1_d(x1);
  if (lane == 63) {
    wt[0][w] = x0;
    wt[1][w] = x1;
  }
  __syncthreads();
  double b0 = 0.0, b1 = 0.0, t0 = 0.0, t1 = 0.0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    if (i < w) {
      b0 += wt[0][i];
      b1 += wt[1][i];
    }
    t0 += wt[0][i];
    t1 += wt[1][i];
  }
  incl0 = b0 + x0;
  excl0 = b0 + e0;
  tot0 = t0;
  incl1 = b1 + x1;
  excl1 = b1 + e1;
  tot1 = t1;
  __syncthreads();
}

// One wave sums the weights of segment [s0, s0 + kSeg) (clipped to V): lane l
// takes groups l, l+64, ... so that every load of the wave is one contiguous
// kilobyte, and a whole part of the segment (both rows) is loaded before any
// of it is used.  Returns (residual sum, p sum) in every lane.
template <int ES, bool VEC, bool RES>
__device__ __forceinline__ void segment_sums(const char* prow, const char* qrow, const WeightCtx& w, int s0,
                                             int V, double& rsum, double& psum) {
  constexpr int H = (ES == 2 && VEC) ? kSegGroups : kSegGroups / 2;  // groups per part
  constexpr int NH = kSegGroups / H;
  const int lane = threadIdx.x & 63;
  const bool full = s0 + kSeg <= V;
  rsum = 0.0;
  psum = 0.0;
#pragma unroll 1
  for (int h = 0; h < NH; ++h) {
    RawGroup<ES, VEC> rp[H], rq[H];
#pragma unroll
    for (int g = 0; g < H; ++g) {
      const int e = s0 + ((h * H + g) * 64 + lane) * 8;
      if (full) {
        rp[g] = load_raw<ES, VEC>(prow, e);
        if (RES) rq[g] = load_raw<ES, VEC>(qrow, e);
      } else if (e < V) {
        rp[g] = load_raw_bounded<ES, VEC>(prow, e, V);
        if (RES) rq[g] = load_raw_bounded<ES, VEC>(qrow, e, V);
      } else {
        rp[g] = neg_inf_group<ES, VEC>();
        if (RES) rq[g] = neg_inf_group<ES, VEC>();
      }
    }
#pragma unroll
    for (int g = 0; g < H; ++g) {
      float xp[8], xq[8];
      unpack_group<ES, VEC>(rp[g], xp);
      if (RES) unpack_group<ES, VEC>(rq[g], xq);
      float r8 = 0.f, p8 = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float ep;
        r8 += pair_weight(w, xp[i], RES ? xq[i] : 0.f, RES, ep);
        p8 += ep;
      }
      rsum += (double)r8;
      psum += (double)p8;
    }
  }
  rsum = wave_total_d(rsum);  // DPP, fixed order
  psum = wave_total_d(psum);
}

}  // namespace specv
