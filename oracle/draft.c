/*
 * draft.c -- CPU oracle for sampling the next draft tokens from the drafter's
 * logits at the new-token indices of an expanded P-EAGLE batch.
 *
 * TEST INFRASTRUCTURE ONLY (see spec_oracle.h).
 *
 * Source: "P-EAGLE: parallel speculative decoding in vLLM" page, section
 * "Triton Kernel": the expansion emits new-token indices, the rows of the
 * drafter batch at which the draft tokens are sampled (one forward pass of the
 * drafter predicts all K of them, section "核心方法").  The sampled tokens and
 * the drafter's distributions q at those rows are what the next verification
 * checks (explainer page, section "修正拒绝采样": x ~ q, accepted with
 * probability min(1, p(x)/q(x))).
 *
 * Readings of points the pages leave open (listed in the design notes): the
 * draft token of position k of request b is drawn from q = softmax(logits[row]
 * / T_b), row = row_index[b, k], with the same temperature as the
 * verification; the draw is the inverse CDF in ascending vocabulary order with
 * one uniform, Philox4x32-10 counter {b + request_base, k, step, 1}, word 0 (a
 * stream apart from the verification's, which uses counter word 3 = 0);
 * temperature 0 takes the lowest-index argmax.  Everything in double,
 * sequentially.
 */
#include "spec_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>

void oracle_draft_uniform(uint64_t seed, uint32_t step, uint32_t request, uint32_t position, double* u) {
  uint32_t ctr[4] = {request, position, step, 1u /* stream of the drafting step */};
  uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  *u = oracle_uniform(out[0]);
}

void oracle_draft_uniforms_many(uint64_t seed, uint32_t step, const uint32_t* requests,
                                const uint32_t* positions, int64_t n, double* u) {
  for (int64_t i = 0; i < n; ++i) oracle_draft_uniform(seed, step, requests[i], positions[i], &u[i]);
}

int oracle_draft_sample(const oracle_draft_args* a) {
  if (!a || a->B < 0 || a->K < 1 || a->V < 1 || a->N < 0 || (a->dtype != 0 && a->dtype != 1)) return -1;
  if (a->B > 0 && (!a->logits || !a->row_index || !a->temperature || !a->tokens)) return -1;
  if (a->row_stride < a->V) return -1;
  int bad = 0;
  double* p = (double*)malloc(sizeof(double) * (size_t)a->V);
  if (!p) return -1;
  for (int b = 0; b < a->B; ++b) {
    const double T = (double)a->temperature[b];
    for (int k = 0; k < a->K; ++k) {
      const int64_t i = (int64_t)b * a->K + k;
      const int32_t row = a->row_index[i];
      a->tokens[i] = -1;
      if (a->trace) a->trace[i] = NAN;
      if (row < 0 || row >= a->N || !(T >= 0.0) || isinf(T) || (T > 0.0 && T < FLT_MIN)) {
        ++bad;
        continue;
      }
      const void* logits = (const char*)a->logits + (int64_t)row * a->row_stride * (a->dtype == 0 ? 4 : 2);
      if (T == 0.0) {
        a->tokens[i] = oracle_argmax(logits, a->dtype, a->V);
        continue;
      }
      /* mutation 1 plants the mistake of ignoring the temperature */
      if (!oracle_scaled_max_in_range(logits, a->dtype, a->V, a->temperature[b]) ||
          oracle_softmax(logits, a->dtype, a->V, a->mutation == 1 ? 1.0 : T, p) != 0) {
        ++bad;
        continue;
      }
      double W = 0.0;
      for (int v = 0; v < a->V; ++v) W += p[v];
      double u;
      oracle_draft_uniform(a->seed, a->step, (uint32_t)b + a->request_base, (uint32_t)k, &u);
      if (a->trace) a->trace[i] = u;
      a->tokens[i] = oracle_invcdf(p, a->V, W, u);
    }
  }
  free(p);
  return bad;
}
