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
// 16-byte loads per lane in flight before any is used).  One loop body serves
// every batch: groups past the chunk (in its last batch) load the lane's
// first group again and are left out of the reduction, so a short last batch
// still issues its loads together and the loop keeps one register set; the
// arithmetic of groups that no lane of the wave needs is skipped (a
// wave-uniform branch), which in a pass bound by its own arithmetic as much
// as by memory is what a short last batch costs.  The
// (< 8) trailing logits of a row whose length is not a multiple of 8 go to
// thread 0.
template <int ES>
constexpr int batch_groups() { return ES == 2 ? 8 : 4; }  // 128 bytes per lane

template <int ES, bool VEC>
__device__ __forceinline__ MS chunk_stats(const char* __restrict__ row, int e0, int e1, float s_hi,
                                          float s_lo) {
  constexpr int U = batch_groups<ES>();
  const int nfull = (e1 - e0) >> 3;
  float M = -INFINITY;
  double S = 0.0;
  for (int g = threadIdx.x; g < nfull; g += kWG * U) {
    // groups u < nu are needed by some lane of the wave (its first active lane
    // holds the lowest group): the rest are skipped with a wave-uniform branch
    const int g0 = __builtin_amdgcn_readfirstlane(g);
    const int nu = (nfull - g0 + kWG - 1) / kWG;
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gu = g + u * kWG;
      load_group<ES, VEC>(row, (int64_t)e0 + 8 * (int64_t)(gu < nfull ? gu : g), x[u]);
    }
    float gm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < nu) {
        float m = x[u][0];
#pragma unroll
        for (int i = 1; i < 8; ++i) m = fmaxf(m, x[u][i]);
        if (g + u * kWG < nfull) gm = fmaxf(gm, m);
      }
    }
    raise_ref(M, S, gm, s_hi);
    const float negM = -fmaxf(M, -1e30f);
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < nu) {
        const float e = sum8_exp(x[u], s_hi, s_lo, negM);
        acc += g + u * kWG < nfull ? e : 0.f;
      }
    }
    S += (double)acc;
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

// Full batches of U groups, then the remaining groups as one masked batch.
template <int ES, bool VEC>
__device__ __forceinline__ VI chunk_argmax(const char* __restrict__ row, int e0, int e1) {
  constexpr int U = batch_groups<ES>();
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
  if (g < nfull) {
    // the remaining groups as one batch: a group past the chunk reads the
    // lane's first group again and counts as -inf at its own (larger) index,
    // which never wins against the lane's lower indices
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gu = g + u * kWG;
      load_group<ES, VEC>(row, (int64_t)e0 + 8 * (int64_t)(gu < nfull ? gu : g), x[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gu = g + u * kWG;
#pragma unroll
      for (int i = 0; i < 8; ++i) best = vi_pick(best, VI{gu < nfull ? x[u][i] : -INFINITY, e0 + 8 * gu + i});
    }
  }
  const int t0 = e0 + 8 * nfull;
  if (t0 < e1 && threadIdx.x == 0)
    for (int e = t0; e < e1; ++e) best = vi_pick(best, VI{load_one<ES>(row, e), e});
  return vi_floor(best, e0);
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
