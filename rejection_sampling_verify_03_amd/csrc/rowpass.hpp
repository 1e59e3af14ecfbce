// rowpass.hpp -- device pieces of the row-statistics pass shared by the
// verification and its vocab-sharded form: one workgroup reduces a run of
// logits of one row to S * 2^M = sum 2^(x * s - M) (integer-valued M) or to
// (max, lowest argmax).
#pragma once

#include <limits.h>

#include "device_common.hpp"

namespace specv {

// Raise the reference exponent of a lane's running (M, S) to cover a new
// group maximum gm (the rescale is an exact power of two).
__device__ __forceinline__ void raise_ref(float& M, double& S, float gm, float s_hi) {
  const float gM = ceilf(gm * s_hi);
  if (gM > M) {
    S = ldexp(S, (int)fmaxf(M - gM, -2000.f));
    M = gM;
  }
}

// ------------------------------------------------------------ chunk passes
// Each thread takes groups tid, tid + 256, ...: U of them per batch (U
// 16-byte loads per lane in flight before any is used).  The last batch of a
// chunk that is not a multiple of U * 256 groups loads clamped addresses (a
// lane's first group again) and masks what lies past the chunk, so that its
// loads are still issued together; the (< 8) trailing logits of a row whose
// length is not a multiple of 8 go to thread 0.
template <int ES>
constexpr int batch_groups() { return ES == 2 ? 8 : 4; }  // 128 bytes per lane

// The U groups g, g + 256, ... of a batch; with MASKED, groups from nfull on
// read group g and come back as -inf.
template <int ES, bool VEC, bool MASKED>
__device__ __forceinline__ void load_batch(const char* __restrict__ row, int e0, int g, int nfull,
                                           float x[batch_groups<ES>()][8]) {
  constexpr int U = batch_groups<ES>();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int gu = g + u * kWG;
    const int gl = (!MASKED || gu < nfull) ? gu : g;
    load_group<ES, VEC>(row, (int64_t)e0 + 8 * (int64_t)gl, x[u]);
    if (MASKED) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = gu < nfull ? x[u][i] : -INFINITY;
    }
  }
}

template <int ES>
__device__ __forceinline__ void stats_batch(const float x[batch_groups<ES>()][8], float s_hi, float s_lo, float& M,
                                            double& S) {
  constexpr int U = batch_groups<ES>();
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

template <int ES, bool VEC>
__device__ __forceinline__ MS chunk_stats(const char* __restrict__ row, int e0, int e1, float s_hi,
                                          float s_lo) {
  constexpr int U = batch_groups<ES>();
  const int nfull = (e1 - e0) >> 3;
  float M = -INFINITY;
  double S = 0.0;
  int g = threadIdx.x;
  for (; g + (U - 1) * kWG < nfull; g += kWG * U) {
    float x[U][8];
    load_batch<ES, VEC, false>(row, e0, g, nfull, x);
    stats_batch<ES>(x, s_hi, s_lo, M, S);
  }
  if (g < nfull) {
    float x[U][8];
    load_batch<ES, VEC, true>(row, e0, g, nfull, x);
    stats_batch<ES>(x, s_hi, s_lo, M, S);
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

// The groups past the chunk of a masked batch repeat the lane's first group
// (same values, same indices), which cannot change the lowest-index argmax.
template <int ES, bool VEC>
__device__ __forceinline__ VI chunk_argmax(const char* __restrict__ row, int e0, int e1) {
  constexpr int U = batch_groups<ES>();
  const int nfull = (e1 - e0) >> 3;
  VI best{-INFINITY, INT_MAX};
  int g = threadIdx.x;
  for (; g < nfull; g += kWG * U) {
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gu = g + u * kWG;
      const int gl = gu < nfull ? gu : g;
      load_group<ES, VEC>(row, (int64_t)e0 + 8 * (int64_t)gl, x[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gu = g + u * kWG;
      const int gl = gu < nfull ? gu : g;
#pragma unroll
      for (int i = 0; i < 8; ++i) best = vi_pick(best, VI{x[u][i], e0 + 8 * gl + i});
    }
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

}  // namespace specv
