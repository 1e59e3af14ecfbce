/*
 * spec_oracle.h -- plain, slow, scalar-C CPU oracle for speculative-decoding
 * verification and P-EAGLE batch expansion.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes or
 * calls this code; only the test-suite, the package smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no header, kernel, helper
 * or constant with the HIP implementation.
 *
 * Sources it follows (cited by page title and section):
 *  - "大模型生成慢..." explainer page, section "修正拒绝采样" (modified rejection
 *    sampling): accept draft token x with probability min(1, p(x)/q(x)); on
 *    rejection resample from normalize(max(0, p - q)); theorem that the output
 *    law is p.
 *  - same page, section "核心思想" flowchart: K drafts verified together, stop at
 *    the first rejection, all accepted => K+1 tokens.
 *  - same page, section "一轮能赚多少": expected tokens per round
 *    (1 - b^(g+1)) / (1 - b).
 *  - "P-EAGLE: parallel speculative decoding in vLLM" page, sections
 *    "并行草稿生成的挑战", "Triton Kernel" and "Hidden State 管理": the expanded
 *    drafter batch (shifted copy, bonus insert, MASK slots, masks, new-token
 *    indices, hidden-state mapping), the two-statement hidden-state fill and
 *    the KV-cache slot mapping; the draft tokens sampled at the new-token
 *    indices.
 *
 * Floating point is IEEE double throughout (logits are widened exactly from
 * fp32 / bf16).  Uniforms come from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), written here from the
 * paper's definition.
 */
#ifndef SPEC_ORACLE_H
#define SPEC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- Philox -- */
/* Philox4x32 with 10 rounds: counter ctr[4], key key[2] -> out[4]. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
/* Map a 32-bit word to a uniform in [0,1): (w >> 8) * 2^-24 (exact in double). */
double oracle_uniform(uint32_t w);
/* The two uniforms drawn for (request r, row k, step): word 0 drives the accept
 * test at row k, word 1 the sampling draw at row k.  Counter
 * {r, k, step, 0}, key {seed lo 32, seed hi 32}. */
void oracle_verify_uniforms(uint64_t seed, uint32_t step, uint32_t request, uint32_t row,
                            double* u_accept, double* u_sample);
/* The same for n (request, row) pairs: oracle_verify_uniforms(seed, step,
 * requests[i], rows[i], &u_accept[i], &u_sample[i]) for each i. */
void oracle_verify_uniforms_many(uint64_t seed, uint32_t step, const uint32_t* requests, const uint32_t* rows,
                                 int64_t n, double* u_accept, double* u_sample);

/* ------------------------------------------------------ decision primitives */
/* Accept rule: u < min(1, p_x / q_x); q_x == 0 => accept iff p_x > 0. */
int oracle_accept(double p_x, double q_x, double u);
/* Inverse CDF over non-negative weights w[0..V) with normaliser W:
 * the smallest v with w[v] > 0 and u*W < sum_{i<=v} w[i]; if none, the last v
 * with w[v] > 0; -1 if every weight is zero. */
int oracle_invcdf(const double* w, int V, double W, double u);
/* Residual weights w = max(0, p - q) with W = sum(w).  If W == 0 the weights
 * fall back to p (W = sum(p)); returns 1 in that case, else 0. */
int oracle_residual(const double* p, const double* q, int V, double* w, double* W);
/* softmax(logits / T) in double, max-subtracted; dtype 0 = fp32, 1 = bf16 bits.
 * Returns 0, or -1 if the row has no finite maximum or T is not > 0. */
int oracle_softmax(const void* row, int dtype, int V, double T, double* out);
/* 1 if the row's largest logit m is finite and its scaled reference
 * ceil(m * s) -- s = log2(e) / T rounded toward zero to fp32, the product
 * rounded to nearest in fp32 -- is an exact fp32 integer, |ref| <= 2^24;
 * else 0.  The kernels hold a row's softmax as S * 2^ref with that fp32
 * reference, exact only in this range; a sampled row outside it (|m| / T
 * above about 1.16e7: a temperature tiny against the logits) counts as a row
 * without a usable normaliser, on both sides. */
int oracle_scaled_max_in_range(const void* row, int dtype, int V, float T);
/* Lowest index of the maximum logit (exact float compare), a NaN logit
 * counting as -inf: a row with nothing above -inf gives 0. */
int oracle_argmax(const void* row, int dtype, int V);

/* Vectorised forms of the primitives for exhaustive enumeration tests:
 * out[i] = oracle_accept(p_x, q_x, oracle_uniform(words[i])) and
 * out[i] = oracle_invcdf(w, V, W, oracle_uniform(words[i])). */
void oracle_accept_many(double p_x, double q_x, const uint32_t* words, int64_t n, uint8_t* out);
void oracle_invcdf_many(const double* w, int V, double W, const uint32_t* words, int64_t n,
                        int32_t* out);

/* ---------------------------------------------------------------- verify -- */
typedef struct {
  int32_t B, K, V;
  int32_t dtype;                     /* 0 = fp32, 1 = bf16 (uint16 bits) */
  const void* target;                /* [B, K+1, V] logits */
  int64_t t_req_stride, t_row_stride;/* in elements; req stride 0 => shared rows */
  const void* draft;                 /* [B, >=K, V] logits (row K never read) */
  int64_t d_req_stride, d_row_stride;
  const int32_t* draft_tokens;       /* [B, K] */
  const float* temperature;          /* [B]; 0 => greedy */
  uint64_t seed;
  uint32_t step;
  uint32_t request_base;             /* request r of this call uses counter r + base */
  const double* uniforms;            /* nullable [B, K+1, 2] override of the Philox draws */
  int32_t* accepted;                 /* out [B]: number of accepted drafts, -1 on bad data */
  int32_t* out_tokens;               /* out [B, K+1]: drafts, then the sampled token, then -1 */
  float* debug_probs;                /* nullable out [B, K, 2]: p_k(x_k), q_k(x_k) */
  double* trace;                     /* nullable out [B, K+1, 3]: u_accept, threshold, u_sample */
  int32_t mutation;                  /* 0 = the method; 1, 2 = planted mistakes for test power */
  int32_t nthreads;                  /* OpenMP threads over requests (<=0: library default) */
  const int32_t* num_drafts;         /* nullable [B]: drafts K_b <= K of request b (ragged K);
                                        positions k >= K_b do not exist, the bonus is at row K_b */
} oracle_verify_args;

/* Returns the number of requests rejected as invalid data (bad token id,
 * temperature < 0 / NaN / inf or below the smallest normal fp32 value but
 * not 0, K_b outside [0, K], a row reached without a finite maximum or with
 * its scaled maximum out of range); their outputs are accepted = -1 and
 * out_tokens all -1.  Returns -1 on bad arguments. */
int oracle_verify(const oracle_verify_args* a);

/* The sampling weights of request b at row j (j < K: residual or its p
 * fallback; j == K: p) and their normaliser, as oracle_verify uses them. */
int oracle_sampling_weights(const oracle_verify_args* a, int b, int j, double* w, double* W);

/* ---------------------------------------------------------------- expand -- */
typedef struct {
  int32_t B, K, H, N_in;
  const int32_t* in_token_ids;       /* [N_in] */
  const int64_t* in_positions;       /* [N_in] */
  const int32_t* in_start;           /* [B+1], in_start[0] = 0, in_start[B] = N_in */
  const int32_t* accepted;           /* [B], 0 <= a_b <= n_b - 1 */
  const int32_t* bonus;              /* [B] */
  int32_t mask_id;
  const uint16_t* target_hidden;     /* nullable [N_in, H] bf16 bits, row stride below */
  int64_t hidden_row_stride;
  const uint16_t* mask_hidden;       /* [H] */
  int32_t* out_token_ids;            /* [N_out] */
  int64_t* out_positions;            /* [N_out] */
  uint8_t* rejected_mask;            /* [N_out] */
  uint8_t* masked_mask;              /* [N_out] */
  int32_t* new_token_indices;        /* [B, K] */
  int32_t* hidden_map;               /* [N_in] */
  int32_t* out_start;                /* [B+1] */
  uint16_t* out_hidden;              /* nullable [N_out, H] */
  /* KV-cache slot mapping (nullable slot_mapping skips it): paged cache of
   * block_size slots per block, block_table[b, i] = physical block of the
   * request's logical block i (i < max_blocks; row stride bt_row_stride) */
  const int32_t* block_table;
  int64_t bt_row_stride;
  int32_t max_blocks;
  int32_t block_size;
  int64_t* slot_mapping;             /* nullable [N_out] */
} oracle_expand_args;

/* Slot mapping ("P-EAGLE" page, section "Hidden State 管理": valid tokens get
 * their normal KV-cache slot, rejected ones PADDING_SLOT_ID = -1 so that
 * nothing is written to the cache for them): an output slot at position pos of
 * request b maps to block_table[b, pos / block_size] * block_size +
 * pos % block_size, or -1 when it is rejected or its position has no block
 * (pos < 0, pos / block_size >= max_blocks, or a negative table entry).
 *
 * Returns the number of requests with invalid data (n_b < 1, a window
 * outside [0, N_in], accepted out of range); such a request writes only its
 * new-token indices, all -1.  If in_start[0] != 0 or in_start[B] != N_in every
 * request is invalid in that way and out_start is not written.  -1 on bad
 * arguments.  A decreasing in_start is outside the contract. */
int oracle_expand(const oracle_expand_args* a);

/* ------------------------------------------------------ draft sampling -- */
/* The uniform of the draft draw at (request, position, step): Philox4x32-10
 * counter {request, position, step, 1}, key {seed lo 32, seed hi 32}, word 0. */
void oracle_draft_uniform(uint64_t seed, uint32_t step, uint32_t request, uint32_t position, double* u);
/* The same for n (request, position) pairs. */
void oracle_draft_uniforms_many(uint64_t seed, uint32_t step, const uint32_t* requests,
                                const uint32_t* positions, int64_t n, double* u);

typedef struct {
  int32_t B, K, V, N;
  int32_t dtype;                     /* 0 = fp32, 1 = bf16 (uint16 bits) */
  const void* logits;                /* [N, V] drafter logits with the row stride below */
  int64_t row_stride;                /* elements, >= V */
  const int32_t* row_index;          /* [B, K]: row of position k of request b (new-token indices) */
  const float* temperature;          /* [B]; 0 => greedy */
  uint64_t seed;
  uint32_t step;
  uint32_t request_base;
  int32_t* tokens;                   /* out [B, K] */
  double* trace;                     /* nullable out [B, K]: the uniform of each draw */
  int32_t mutation;                  /* 0 = the method; 1 = planted mistake for test power */
} oracle_draft_args;

/* Draft token k of request b: x ~ softmax(logits[row_index[b, k]] / T_b) by the
 * inverse CDF with the uniform above (weights p, normaliser their sum); T = 0:
 * lowest-index argmax.  A row index outside [0, N), a temperature < 0 / NaN /
 * inf or below the smallest normal fp32 value but not 0, or (T > 0) a row
 * without a finite maximum or with its scaled maximum out of range gives
 * token -1.  Returns the number of such positions, or -1 on bad arguments. */
int oracle_draft_sample(const oracle_draft_args* a);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_ORACLE_H */
