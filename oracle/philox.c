/*
 * philox.c -- Philox4x32-10 counter-based generator for the CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY (see spec_oracle.h).
 *
 * Written from the definition in Salmon, Moraes, Dror and Shaw, "Parallel
 * Random Numbers: As Easy as 1, 2, 3" (SC'11), section on the Philox family:
 * each round multiplies counter words 0 and 2 by two fixed odd constants,
 * takes the 64-bit products apart into high and low halves, and recombines
 * them with the other two counter words and the round key by XOR, while the
 * key is bumped by the Weyl constants (golden ratio and sqrt(3) - 1) between
 * rounds.  The random draws of the verification step (the explainer page,
 * section "修正拒绝采样", uses one uniform per accept test and one per
 * resample) are taken from this stream.
 */
#include "spec_oracle.h"

#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; ++round) {
    if (round > 0) {
      k0 += PHILOX_W0;
      k1 += PHILOX_W1;
    }
    uint64_t prod0 = (uint64_t)PHILOX_M0 * (uint64_t)x0;
    uint64_t prod1 = (uint64_t)PHILOX_M1 * (uint64_t)x2;
    uint32_t hi0 = (uint32_t)(prod0 >> 32), lo0 = (uint32_t)prod0;
    uint32_t hi1 = (uint32_t)(prod1 >> 32), lo1 = (uint32_t)prod1;
    uint32_t y0 = hi1 ^ x1 ^ k0;
    uint32_t y1 = lo1;
    uint32_t y2 = hi0 ^ x3 ^ k1;
    uint32_t y3 = lo0;
    x0 = y0; x1 = y1; x2 = y2; x3 = y3;
  }
  out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

double oracle_uniform(uint32_t w) {
  /* 24 high bits as an integer times 2^-24: every value is exact in double and
   * lies in [0, 1). */
  return (double)(w >> 8) * (1.0 / 16777216.0);
}

void oracle_verify_uniforms(uint64_t seed, uint32_t step, uint32_t request, uint32_t row,
                            double* u_accept, double* u_sample) {
  uint32_t ctr[4] = {request, row, step, 0u /* stream of the verification step */};
  uint32_t key[2] = {(uint32_t)(seed & 0xffffffffu), (uint32_t)(seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  if (u_accept) *u_accept = oracle_uniform(out[0]);
  if (u_sample) *u_sample = oracle_uniform(out[1]);
}

void oracle_verify_uniforms_many(uint64_t seed, uint32_t step, const uint32_t* requests, const uint32_t* rows,
                                 int64_t n, double* u_accept, double* u_sample) {
  for (int64_t i = 0; i < n; ++i)
    oracle_verify_uniforms(seed, step, requests[i], rows[i], &u_accept[i], &u_sample[i]);
}
