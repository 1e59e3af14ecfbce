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
// Each thread takes groups tid, tid + 256, ...; the main loop issues U
// unconditional 16-byte loads per lane before using any of them, the
// remainder loop takes one group at a time, and the (< 8) trailing logits of a
// row whose length is not a multiple of 8 go to thread 0.
template <int ES, bool VEC>
__device__ __forceinline__ MS chunk_stats(const char* __restrict__ row, int e0, int e1, float s_hi,
                                          float s_lo) {
  constexpr int U = (ES == 2) ? 8 : 4;  // 128 bytes in flight per lane per iteration
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
  constexpr int U = (ES == 2) ? 8 : 4;
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

}  // namespace specv
