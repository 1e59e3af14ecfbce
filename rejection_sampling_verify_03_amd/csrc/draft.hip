// draft.hip -- the next draft tokens, sampled from the drafter's logits at the
// new-token indices of an expanded P-EAGLE batch, on gfx950.
//
// "P-EAGLE: parallel speculative decoding in vLLM" page, section "Triton
// Kernel": the expansion emits the new-token indices, the drafter rows at
// which the draft tokens are sampled (one drafter pass predicts all K,
// section "核心方法").  Token k of request b is drawn from
// q = softmax(logits[row_index[b, k]] / T_b), the distribution the next
// verification checks it against (explainer page, section "修正拒绝采样"),
// by the inverse CDF in vocabulary order with one Philox4x32-10 uniform,
// counter {b + request_base, k, step, 1} (a stream apart from the
// verification's), word 0; temperature 0 takes the lowest-index argmax.
//
// Two kernels, one read of each row plus one 4096-logit segment:
//
//  draft_segstats  one 256-thread workgroup per (row, 8 segments): each wave
//      takes a segment (lane l loads groups l, l+64, ...: one contiguous
//      kilobyte per wave load) and reduces it to S_j * 2^(M_j) =
//      sum 2^(x * s - M_j) with its own integer-valued reference M_j (the
//      segment maximum, rounded up, in units of the scale s = log2(e) / T),
//      or to (max, lowest argmax) at temperature 0.
//
//  draft_draw      one 512-thread workgroup per (request, position): brings
//      the segment sums to the row's largest reference M* by exact
//      power-of-two scaling, scans them in order for the crossing of u * W,
//      and finds the token inside that one segment, recomputing its weights
//      scaled by the same power of two.
#include <limits.h>

#include "device_common.hpp"
#include "sampling.hpp"
#include "verify_kernels.hpp"
#include "verify_layout.hpp"

namespace specv {

__device__ __forceinline__ bool draft_row_valid(const DraftParams& P, int row, float T) {
  return row >= 0 && row < P.N && temperature_valid(T);
}

template <int ES, bool VEC>
__global__ __launch_bounds__(kWG) void draft_segstats_kernel(DraftParams P) {
  const int c = blockIdx.x % P.C;
  const int i = blockIdx.x / P.C;  // (request, position)
  const int b = i / P.K;
  const int row = P.row_index[i];
  const float T = P.temperature[b];
  if (!draft_row_valid(P, row, T)) return;  // the draw reports -1
  const char* lg = P.logits + (int64_t)row * P.row_stride * ES;
  const bool greedy = T == 0.0f;
  float s_hi = 0.f, s_lo = 0.f;
  if (!greedy) temperature_scale(T, s_hi, s_lo);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j1 = min(P.nseg, (c + 1) * kDraftChunkSegs);
  for (int j = c * kDraftChunkSegs + wave; j < j1; j += kWaves) {
    const int s0 = j * kSeg;
    const bool full = s0 + kSeg <= P.V;
    RawGroup<ES, VEC> rg[kSegGroups];
#pragma unroll
    for (int g = 0; g < kSegGroups; ++g) {
      const int e = s0 + (g * 64 + lane) * 8;
      if (full) rg[g] = load_raw<ES, VEC>(lg, e);
      else if (e < P.V) rg[g] = load_raw_bounded<ES, VEC>(lg, e, P.V);
      else rg[g] = neg_inf_group<ES, VEC>();
    }
    RowPartial part;
    if (greedy) {
      VI best{-INFINITY, INT_MAX};
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g) {
        float x[8];
        unpack_group<ES, VEC>(rg[g], x);
        const int e = s0 + (g * 64 + lane) * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (e + q < P.V) best = vi_pick(best, VI{x[q], e + q});
      }
      best = wave_argmax(best);
      part.m = best.v;
      part.idx = best.i;
      part.s = 0.0;
    } else {
      float gm = -INFINITY;
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g) {
        float x[8];
        unpack_group<ES, VEC>(rg[g], x);
#pragma unroll
        for (int q = 0; q < 8; ++q) gm = fmaxf(gm, x[q]);
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) gm = fmaxf(gm, __shfl_xor(gm, off, 64));
      const float M = ceilf(gm * s_hi);  // -inf for a segment without a finite logit
      const float negM = -fmaxf(M, -1e30f);
      double S = 0.0;
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g) {
        float x[8];
        unpack_group<ES, VEC>(rg[g], x);
        S += (double)sum8_exp(x, s_hi, s_lo, negM);
      }
      part.m = M;
      part.idx = 0;
      part.s = wave_sum_d(S);
    }
    if (lane == 0) P.segp[(int64_t)i * P.nseg + j] = part;
  }
}

template <int NT>
__device__ __forceinline__ float block_max_f(float v) {
  constexpr int W = NT / 64;
  __shared__ float mx[W];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  if ((threadIdx.x & 63) == 0) mx[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = mx[0];
#pragma unroll
  for (int i = 1; i < W; ++i) r = fmaxf(r, mx[i]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ VI block_argmax_vi(VI v) {
  constexpr int W = NT / 64;
  __shared__ float sv[W];
  __shared__ int si[W];
  v = wave_argmax(v);
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = v.v;
    si[threadIdx.x >> 6] = v.i;
  }
  __syncthreads();
  VI r{sv[0], si[0]};
#pragma unroll
  for (int i = 1; i < W; ++i) r = vi_pick(r, VI{sv[i], si[i]});
  __syncthreads();
  return r;
}

// Segment j's sum in units of 2^M* (exact power-of-two scaling).
__device__ __forceinline__ double scaled_seg(const RowPartial& p, float Mstar) {
  return ldexp(p.s, (int)fmaxf(p.m - Mstar, -2000.f));
}

template <int ES, bool VEC>
__global__ __launch_bounds__(kDrawThreads) void draft_draw_kernel(DraftParams P) {
  constexpr int NT = kDrawThreads;
  const int i = blockIdx.x;
  const int b = i / P.K, k = i % P.K;
  const int tid = threadIdx.x;
  const int row = P.row_index[i];
  const float T = P.temperature[b];
  if (!draft_row_valid(P, row, T)) {
    if (tid == 0) P.tokens[i] = -1;
    return;
  }
  const RowPartial* sp = P.segp + (int64_t)i * P.nseg;
  const int nseg = P.nseg;
  if (T == 0.0f) {
    VI best{-INFINITY, INT_MAX};
    for (int j = tid; j < nseg; j += NT) best = vi_pick(best, VI{sp[j].m, sp[j].idx});
    best = block_argmax_vi<NT>(best);
    if (tid == 0) P.tokens[i] = best.i;
    return;
  }
  float mloc = -INFINITY;
  for (int j = tid; j < nseg; j += NT) mloc = fmaxf(mloc, sp[j].m);
  const float Mstar = block_max_f<NT>(mloc);
  if (!(fabsf(Mstar) <= FLT_MAX)) {  // no finite logit in the row
    if (tid == 0) P.tokens[i] = -1;
    return;
  }
  const uint32_t k0 = (uint32_t)(P.seed & 0xffffffffu), k1 = (uint32_t)(P.seed >> 32);
  const double u = unit_uniform(philox4x32_10((uint32_t)b + P.request_base, (uint32_t)k, P.step, 1u, k0, k1).w[0]);
  // totals, then the crossing of u * W in a fixed-order scan over the segments
  __shared__ double sh_base;
  double W = 0.0;
  for (int j0 = 0; j0 < nseg; j0 += NT) {
    const int j = j0 + tid;
    double incl, excl, tot, i2, e2, t2;
    block_scan_d2<NT>(j < nseg ? scaled_seg(sp[j], Mstar) : 0.0, 0.0, incl, excl, tot, i2, e2, t2);
    W += tot;
  }
  const double target = u * W;
  int found = -1, lastpos = -1;
  double base = 0.0, carry = 0.0;
  for (int j0 = 0; j0 < nseg && found < 0; j0 += NT) {
    const int j = j0 + tid;
    const double v = j < nseg ? scaled_seg(sp[j], Mstar) : 0.0;
    double incl, excl, tot, i2, e2, t2;
    block_scan_d2<NT>(v, 0.0, incl, excl, tot, i2, e2, t2);
    const int f = block_first_true<NT>(j < nseg && carry + incl > target);
    lastpos = max(lastpos, block_max_int<NT>(v > 0.0 ? j : -1));
    if (f >= 0 && tid == f) sh_base = carry + excl;
    __syncthreads();
    if (f >= 0) {
      found = j0 + f;
      base = sh_base;
    }
    carry += tot;
    __syncthreads();
  }
  const int js = found >= 0 ? found : lastpos;
  int y = -1;  // no positive weight anywhere: only reachable outside the data contract
  if (js >= 0) {
    const float mj = sp[js].m;
    WeightCtx w;
    w.s_hi = 0.f;
    w.s_lo = 0.f;
    temperature_scale(T, w.s_hi, w.s_lo);
    w.negMp = -mj;
    w.negMq = 0.f;
    w.c_hi = w.c_lo = 0.f;
    const double scale = ldexp(1.0, (int)fmaxf(mj - Mstar, -2000.f));
    const char* lg = P.logits + (int64_t)row * P.row_stride * ES;
    y = draw_in_segment<ES, VEC>(lg, lg, P.V, w, false, false, scale, js, found >= 0 ? base : 0.0,
                                 found >= 0 ? target : 0.0, found < 0);
  }
  if (tid == 0) P.tokens[i] = y;
}

template <int ES, bool VEC>
static hipError_t launch_draft_typed(const DraftParams& P, hipStream_t stream) {
  const int64_t g1 = (int64_t)P.B * P.K * P.C;
  hipLaunchKernelGGL((draft_segstats_kernel<ES, VEC>), dim3((unsigned)g1), dim3(kWG), 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((draft_draw_kernel<ES, VEC>), dim3((unsigned)(P.B * P.K)), dim3(kDrawThreads), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_draft(const DraftParams& P, int dtype, bool vec, hipStream_t stream) {
  if (dtype == SPEC_BF16)
    return vec ? launch_draft_typed<2, true>(P, stream) : launch_draft_typed<2, false>(P, stream);
  return vec ? launch_draft_typed<4, true>(P, stream) : launch_draft_typed<4, false>(P, stream);
}

}  // namespace specv
