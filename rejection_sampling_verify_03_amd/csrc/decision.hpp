// decision.hpp -- the accept test of one draft position and the stopping
// position of a request, shared by every form of the verification (one pass,
// early-exit phases, decisions inside the row pass, vocab shards).
#pragma once

#include <float.h>

#include "device_common.hpp"

namespace specv {

// A row's statistics are usable when its normaliser is positive and finite
// (its maximum was finite) and its reference m = ceil(max * s) is an exact
// fp32 integer: beyond 2^24 the scaled logits near the maximum are no longer
// held to within one unit of the reference, so the row is refused rather
// than computed inexactly.
__device__ __forceinline__ bool row_usable(float m, double s) {
  return s > 0.0 && s <= DBL_MAX && fabsf(m) <= kMaxRef;
}

// The accept test at draft position k of request `req` (explainer page on
// speculative decoding, section "修正拒绝采样"): p = p_k(x_k) and q = q_k(x_k)
// from each row's reference M, normaliser S and the logit z at the draft
// token, p = 2^(z s - M) / S in double; accept iff u_k < min(1, p / q) (q = 0:
// accept iff p > 0), u_k from word 0 of Philox4x32-10 at {req, k, step, 0}.
__device__ __forceinline__ bool accept_test(float T, float zp, float mp, double sp, float zq, float mq,
                                            double sq, uint64_t seed, uint32_t req, uint32_t k, uint32_t step,
                                            float& dp, float& dq) {
  float s_hi, s_lo;
  temperature_scale(T, s_hi, s_lo);
  const double s_eff = (double)s_hi + (double)s_lo;
  const double p = exp2((double)zp * s_eff - (double)mp) / sp;
  const double q = exp2((double)zq * s_eff - (double)mq) / sq;
  const double thr = q > 0.0 ? fmin(1.0, p / q) : (p > 0.0 ? 1.0 : 0.0);
  const uint32_t k0 = (uint32_t)(seed & 0xffffffffu), k1 = (uint32_t)(seed >> 32);
  dp = (float)p;
  dq = (float)q;
  return unit_uniform(philox4x32_10(req, k, step, 0u, k0, k1).w[0]) < thr;
}

// Where a request stops, from its tests over positions [lo, min(hi, K_b))
// (same page, section "核心思想": the positions are taken in order and the
// first rejection ends the request).  Called by every lane of one wave, lane
// k standing for position k: `acc` true when position k passed (always for
// k < lo), `rowbad` when a row of position k that was read has no usable
// normaliser.  With test false no test ran and the request stops at `known`.
// Returns a in [lo, min(hi, K_b)] (min(hi, K_b): every test in range passed),
// or -1 when the data is invalid: `inbad` (the inputs: tokens, temperature,
// counts, row entries), a row without a usable normaliser at the position
// where the request stops, or (a = K_b with the bonus row read here, K_b <
// thi) `bonusbad` for that row.  Rows past the stop do not count.
__device__ __forceinline__ int stop_position(bool test, int lo, int hi, int thi, int known, int kb, bool acc,
                                             bool rowbad, bool bonusbad, bool inbad) {
  const uint64_t pass = __ballot(acc);
  const uint64_t badm = __ballot(rowbad);
  const int a = test ? (int)__builtin_ctzll(~pass) : known;
  const bool at_test = test ? a < min(hi, kb) : known < kb;
  const bool stopbad = at_test ? ((badm >> a) & 1u) != 0 : (a == kb && kb < thi && bonusbad);
  return (inbad || stopbad) ? -1 : a;
}

}  // namespace specv
