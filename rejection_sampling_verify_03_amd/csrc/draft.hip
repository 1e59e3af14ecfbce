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
//  draft_draw      one wave64 workgroup per (request, position): brings the
//      segment sums to the row's largest reference M* by exact power-of-two
//      scaling, scans them in order for the crossing of u * W, and finds the
//      token inside that one segment, recomputing its weights scaled by the
//      same power of two (groups of 8 logits scanned 64 at a time, one per
//      lane, in vocabulary order).  The wave is one chain of dependent
//      steps, so the segment records load with the row index, the segment's
//      64 logits per lane load together, and lanes exchange values through
//      DPP moves and readlane rather than LDS permutes.  On request it also
//      writes the row's normaliser W * 2^M* and the drawn token's logit: the
//      statistics the next verification takes instead of reading the row.
#include <limits.h>

#include "device_common.hpp"
#include "sampling.hpp"
#include "verify_kernels.hpp"
#include "verify_layout.hpp"

namespace specv {

__device__ __forceinline__ bool draft_row_valid(const DraftParams& P, int row, float T) {
  return row >= 0 && row < P.N && temperature_valid(T);
}

// The segments j = j0, j0 + kWaves, ... below j1 of one row, one wave each:
// lane l loads groups l, l+64, ... (one contiguous kilobyte per wave load)
// and the wave writes the segment's record.  GREEDY: (max, lowest argmax);
// else S * 2^M in one pass -- each lane sums its 64 logits against its own
// reference ceil(lane max * s) and the wave merges the (M, S) pairs by exact
// powers of two, so M is ceil(segment max * s) (-inf for a segment without a
// finite logit).  The two kinds are separate loops so that each keeps its
// own register set.
template <int ES, bool VEC, bool GREEDY>
__device__ __forceinline__ void segment_records(const DraftParams& P, const char* lg, RowPartial* out, int j0,
                                                int j1, int lane, float s_hi, float s_lo) {
  for (int j = j0; j < j1; j += kWaves) {
    const int s0 = j * kSeg;
    RawGroup<ES, VEC> rg[kSegGroups];
    if (s0 + kSeg <= P.V) {  // a full segment: eight loads in a row, none under a branch
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g) rg[g] = load_raw<ES, VEC>(lg, s0 + (g * 64 + lane) * 8);
    } else {
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g) {
        const int e = s0 + (g * 64 + lane) * 8;
        rg[g] = e < P.V ? load_raw_bounded<ES, VEC>(lg, e, P.V) : neg_inf_group<ES, VEC>();
      }
    }
    RowPartial part;
    if constexpr (GREEDY) {
      VI best{-INFINITY, INT_MAX};
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g) {
        opaque_group<ES, VEC>(rg[g]);  // widened one group at a time
        float x[8];
        unpack_group<ES, VEC>(rg[g], x);
        const int e = s0 + (g * 64 + lane) * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (e + q < P.V) best = vi_pick(best, VI{x[q], e + q});
      }
      best = wave_argmax(vi_floor(best, s0));
      part.m = best.v;
      part.idx = best.i;
      part.s = 0.0;
    } else {
      float x[kSegGroups][8];
      float gm = -INFINITY;
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g) {
        unpack_group<ES, VEC>(rg[g], x[g]);
#pragma unroll
        for (int q = 0; q < 8; ++q) gm = fmaxf(gm, x[g][q]);
      }
      const float Ml = ceilf(gm * s_hi);
      const float negM = -fmaxf(Ml, -1e30f);
      double S = 0.0;
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g) S += (double)sum8_exp(x[g], s_hi, s_lo, negM);
      const MS ms = wave_merge_ms(MS{Ml, S});
      part.m = ms.m;
      part.idx = 0;
      part.s = ms.s;
    }
    if (lane == 0) out[j] = part;
  }
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
  // the wave index through readfirstlane, so that the segment bounds and the
  // full-segment test are scalar (uniform branches around the loads)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j0 = c * kDraftChunkSegs + wave;
  const int j1 = min(P.nseg, (c + 1) * kDraftChunkSegs);
  RowPartial* out = P.segp + (int64_t)i * P.nseg;
  if (T == 0.0f) {
    segment_records<ES, VEC, true>(P, lg, out, j0, j1, lane, 0.f, 0.f);
  } else {
    float s_hi, s_lo;
    temperature_scale(T, s_hi, s_lo);
    segment_records<ES, VEC, false>(P, lg, out, j0, j1, lane, s_hi, s_lo);
  }
}

// Segment j's sum in units of 2^M* (exact power-of-two scaling).
__device__ __forceinline__ double scaled_seg(const RowPartial& p, float Mstar) {
  return ldexp(p.s, (int)fmaxf(p.m - Mstar, -2000.f));
}

// One wave per (request, position): the crossing segment from a scan of the
// segment sums, then the token inside it -- lane l takes the groups of 8
// logits l, l + 64, ... of the segment, so that each round of 64 groups is one
// contiguous wave load; the rounds are scanned in vocabulary order and the
// crossing lane walks its own 8 logits.  The whole search is one chain of
// dependent steps per wave, so every load of a step is issued before any of
// its results is used, and lanes exchange values through DPP and readlane.
template <int ES, bool VEC>
__global__ __launch_bounds__(64) void draft_draw_kernel(DraftParams P) {
  const int i = blockIdx.x;
  const int b = i / P.K, k = i % P.K;
  const int lane = threadIdx.x;
  const int row = P.row_index[i];
  const float T = P.temperature[b];
  // the records of segments 0..63 stay in registers, one per lane; loaded
  // together with the row index (an invalid row's records are never used)
  const RowPartial* sp = P.segp + (int64_t)i * P.nseg;
  const int nseg = P.nseg;
  RowPartial r0{-INFINITY, INT_MAX, 0.0};
  if (lane < nseg) r0 = sp[lane];
  const RowPartial none{0.f, 0, 0.0};  // the statistics record of a position drawn at T = 0 or given -1
  if (!draft_row_valid(P, row, T)) {
    if (lane == 0) {
      P.tokens[i] = -1;
      if (P.stats) P.stats[i] = none;
    }
    return;
  }
  if (T == 0.0f) {
    VI best{r0.m, r0.idx};
    for (int j = lane + 64; j < nseg; j += 64) best = vi_pick(best, VI{sp[j].m, sp[j].idx});
    best = wave_argmax(best);
    if (lane == 0) {
      P.tokens[i] = best.i;
      if (P.stats) P.stats[i] = none;
    }
    return;
  }
  float Mstar = r0.m;
  for (int j = lane + 64; j < nseg; j += 64) Mstar = fmaxf(Mstar, sp[j].m);
  Mstar = wave_max_f(Mstar);
  if (!(fabsf(Mstar) <= kMaxRef)) {  // no finite logit in the row, or its scaled maximum out of range
    if (lane == 0) {
      P.tokens[i] = -1;
      if (P.stats) P.stats[i] = none;
    }
    return;
  }
  const uint32_t k0 = (uint32_t)(P.seed & 0xffffffffu), k1 = (uint32_t)(P.seed >> 32);
  const double u = unit_uniform(philox4x32_10((uint32_t)b + P.request_base, (uint32_t)k, P.step, 1u, k0, k1).w[0]);
  // total W, then the crossing of u * W, in one fixed-order scan over the
  // segments (64 at a time)
  const double v0 = lane < nseg ? scaled_seg(r0, Mstar) : 0.0;
  const double x0 = wave_scan_d(v0);
  double W = lane_d(x0, 63);
  for (int j0 = 64; j0 < nseg; j0 += 64) {
    const int j = j0 + lane;
    W += lane_d(wave_scan_d(j < nseg ? scaled_seg(sp[j], Mstar) : 0.0), 63);
  }
  if (!(W > 0.0 && W <= DBL_MAX)) {  // a row without a finite normaliser (a NaN logit): as a bad row
    if (lane == 0) {
      P.tokens[i] = -1;
      if (P.stats) P.stats[i] = none;
    }
    return;
  }
  const double target = u * W;
  int found = -1, lastseg = -1;
  double base = 0.0, carry = 0.0;
  for (int j0 = 0; j0 < nseg && found < 0; j0 += 64) {
    const int j = j0 + lane;
    double v = v0, x = x0;
    if (j0 > 0) {
      v = j < nseg ? scaled_seg(sp[j], Mstar) : 0.0;
      x = wave_scan_d(v);
    }
    const uint64_t m = __ballot(j < nseg && carry + x > target);
    const uint64_t pos = __ballot(v > 0.0);
    if (pos) lastseg = j0 + 63 - __builtin_clzll(pos);
    if (m) {
      const int f = __builtin_ctzll(m);
      found = j0 + f;
      base = carry + lane_d(x - v, f);
    }
    carry += lane_d(x, 63);
  }
  const bool last_positive = found < 0;
  const int js = last_positive ? lastseg : found;
  int y = -1;  // no positive weight anywhere: only reachable outside the data contract
  if (js >= 0) {
    const char* lg = P.logits + (int64_t)row * P.row_stride * ES;
    const int s0 = js * kSeg;
    // all 64 logits of the lane in flight at once; a segment cut by the row
    // end reads clamped addresses and masks them
    float xs[kSegGroups][8];
    if (s0 + kSeg <= P.V) {
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g) load_group<ES, VEC>(lg, s0 + (g * 64 + lane) * 8, xs[g]);
    } else {
#pragma unroll
      for (int g = 0; g < kSegGroups; ++g)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int e = s0 + (g * 64 + lane) * 8 + q;
          const float v = load_one<ES>(lg, min(e, P.V - 1));
          xs[g][q] = e < P.V ? v : -INFINITY;
        }
    }
    float s_hi, s_lo;
    temperature_scale(T, s_hi, s_lo);
    const float mj = js < 64 ? lane_f(r0.m, js) : sp[js].m;
    const float negM = -mj;
    const double scale = ldexp(1.0, (int)fmaxf(mj - Mstar, -2000.f));
    // groups in vocabulary order: 64 per round (one per lane), scanned in order
    double carry = base;
    int pick = -1, lpos = -1;
#pragma unroll
    for (int g = 0; g < kSegGroups; ++g) {
      const int e = s0 + (g * 64 + lane) * 8;
      double w[8], wg = 0.0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        w[q] = (double)scaled_exp2(xs[g][q], s_hi, s_lo, negM) * scale;
        wg += w[q];
        if (w[q] > 0.0) lpos = e + q;
      }
      const double x = wave_scan_d(wg);
      const double tot = lane_d(x, 63);
      if (!last_positive && pick < 0 && carry + tot > target) {
        const uint64_t m = __ballot(carry + x > target);
        const int L = m ? __builtin_ctzll(m) : 63;
        double run = carry + (x - wg);
        int pl = -1;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          run += w[q];
          if (pl < 0 && w[q] > 0.0 && target < run) pl = e + q;
        }
        if (pl < 0) pl = lpos >= e ? lpos : -1;  // cumulative rounding: stay inside this group
        pick = lane_i(pl, L);
      }
      carry += tot;
    }
    if (pick < 0) {  // the last positive logit of the segment
      pick = wave_max_i(lpos);
    }
    y = pick;
  }
  if (lane == 0) {
    P.tokens[i] = y;
    // the row's normaliser W * 2^M* and the drawn logit, for a verification
    // of this token against this row (the draft row statistics it takes)
    if (P.stats) {
      RowPartial rec = none;
      if (y >= 0) {
        rec.m = Mstar;
        rec.idx = (int32_t)load_bits<ES>(P.logits + (int64_t)row * P.row_stride * ES, y);
        rec.s = W;
      }
      P.stats[i] = rec;
    }
  }
}

template <int ES, bool VEC>
static hipError_t launch_draft_typed(const DraftParams& P, hipStream_t stream) {
  const int64_t g1 = (int64_t)P.B * P.K * P.C;
  hipLaunchKernelGGL((draft_segstats_kernel<ES, VEC>), dim3((unsigned)g1), dim3(kWG), 0, stream, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((draft_draw_kernel<ES, VEC>), dim3((unsigned)(P.B * P.K)), dim3(64), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_draft(const DraftParams& P, int dtype, bool vec, hipStream_t stream) {
  if (dtype == SPEC_BF16)
    return vec ? launch_draft_typed<2, true>(P, stream) : launch_draft_typed<2, false>(P, stream);
  return vec ? launch_draft_typed<4, true>(P, stream) : launch_draft_typed<4, false>(P, stream);
}

}  // namespace specv
