/*
 * verify.c -- CPU oracle for batched speculative-decoding verification.
 *
 * TEST INFRASTRUCTURE ONLY (see spec_oracle.h).
 *
 * The method, in the order the explainer page ("大模型生成慢...", sections
 * "核心思想" and "修正拒绝采样") gives it, for each request independently:
 *   for draft position k = 0 .. K-1:
 *     p = softmax(target_k / T), q = softmax(draft_k / T), x = draft token k;
 *     draw u; accept x iff u < min(1, p(x) / q(x));
 *     on rejection draw u' and emit a token from normalize(max(0, p - q))
 *     (the flowchart's "丢弃它之后的候选 / 从修正分布重采样"), then stop;
 *   if all K drafts were accepted, emit one more token sampled from
 *     p = softmax(target_K / T) (the flowchart's "全部接受：产出 K+1 个 token").
 * Temperature 0 is greedy decoding (same page, the greedy remarks in
 * "核心思想" and "边界与代价"): accept iff x equals the target argmax; the
 * emitted token at the stopping row is the target argmax.
 *
 * Readings of points the pages leave open (each one is listed in the design
 * notes): uniforms come from Philox4x32-10 keyed on (seed, request, row,
 * step); word 0 of row k drives the accept test at k and word 1 the sampling
 * draw at k; the accept comparison is strict "<" as printed; q(x) = 0 accepts
 * iff p(x) > 0; the same temperature divides both logits; argmax ties go to
 * the lowest index and a NaN logit counts as -inf there; a residual that
 * sums to exactly zero falls back to p; the inverse CDF runs in ascending
 * vocabulary order over the weights with their own sum as normaliser; a
 * sampled request whose rows at a position it reaches (target and draft row
 * of a tested position, the target row of the bonus) lack a finite maximum,
 * or whose scaled maximum lies beyond the fp32 range the kernels hold it in
 * (oracle_scaled_max_in_range), is invalid, and rows after its stop are
 * never looked at; a temperature between 0 and the smallest normal fp32
 * value is invalid too.
 *
 * Everything is computed in double, sequentially, with no blocking or
 * reordering beyond the definitions above.
 */
#include "spec_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double load_logit(const void* row, int dtype, int v) {
  if (dtype == 0) return (double)((const float*)row)[v];
  uint32_t bits = (uint32_t)((const uint16_t*)row)[v] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

int oracle_softmax(const void* row, int dtype, int V, double T, double* out) {
  if (!(T > 0.0) || !isfinite(T)) return -1;
  double m = -INFINITY;
  for (int v = 0; v < V; ++v) {
    double z = load_logit(row, dtype, v) / T;
    out[v] = z;
    if (z > m) m = z;
  }
  if (!isfinite(m)) return -1;
  double S = 0.0;
  for (int v = 0; v < V; ++v) {
    double e = exp(out[v] - m);
    out[v] = e;
    S += e;
  }
  for (int v = 0; v < V; ++v) out[v] /= S;
  return 0;
}

/* Lowest index of the largest logit, a NaN logit counting as -inf (the
 * pages define the greedy token for numbers only; a NaN carries no
 * preference), so a row with nothing above -inf gives index 0. */
int oracle_argmax(const void* row, int dtype, int V) {
  int best = 0;
  double bv = -INFINITY;
  for (int v = 0; v < V; ++v) {
    double x = load_logit(row, dtype, v);
    if (isnan(x)) x = -INFINITY;
    if (x > bv) {
      bv = x;
      best = v;
    }
  }
  return best;
}

static double accept_threshold(double p_x, double q_x) {
  if (q_x > 0.0) {
    double t = p_x / q_x;
    return t < 1.0 ? t : 1.0;
  }
  return p_x > 0.0 ? 1.0 : 0.0;
}

int oracle_accept(double p_x, double q_x, double u) { return u < accept_threshold(p_x, q_x); }

int oracle_residual(const double* p, const double* q, int V, double* w, double* W) {
  double R = 0.0;
  for (int v = 0; v < V; ++v) {
    double d = p[v] - q[v];
    w[v] = d > 0.0 ? d : 0.0;
    R += w[v];
  }
  if (R == 0.0) {
    double S = 0.0;
    for (int v = 0; v < V; ++v) {
      w[v] = p[v];
      S += p[v];
    }
    *W = S;
    return 1;
  }
  *W = R;
  return 0;
}

int oracle_invcdf(const double* w, int V, double W, double u) {
  double target = u * W;
  double c = 0.0;
  int last = -1;
  for (int v = 0; v < V; ++v) {
    c += w[v];
    if (w[v] > 0.0) {
      last = v;
      if (target < c) return v;
    }
  }
  return last;
}

void oracle_accept_many(double p_x, double q_x, const uint32_t* words, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)oracle_accept(p_x, q_x, oracle_uniform(words[i]));
}

void oracle_invcdf_many(const double* w, int V, double W, const uint32_t* words, int64_t n,
                        int32_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_invcdf(w, V, W, oracle_uniform(words[i]));
}

/* ------------------------------------------------------------------------ */

static const void* row_ptr(const void* base, int dtype, int64_t req_stride, int64_t row_stride,
                           int b, int k) {
  size_t es = dtype == 0 ? 4 : 2;
  return (const char*)base + ((int64_t)b * req_stride + (int64_t)k * row_stride) * (int64_t)es;
}

static const void* trow(const oracle_verify_args* a, int b, int k) {
  return row_ptr(a->target, a->dtype, a->t_req_stride, a->t_row_stride, b, k);
}

static const void* drow(const oracle_verify_args* a, int b, int k) {
  return row_ptr(a->draft, a->dtype, a->d_req_stride, a->d_row_stride, b, k);
}

static void uniforms_for(const oracle_verify_args* a, int b, int k, double* ua, double* us) {
  if (a->uniforms) {
    const double* u = a->uniforms + ((int64_t)b * (a->K + 1) + k) * 2;
    *ua = u[0];
    *us = u[1];
  } else {
    oracle_verify_uniforms(a->seed, a->step, (uint32_t)b + a->request_base, (uint32_t)k, ua, us);
  }
}

static int row_has_finite_max(const void* row, int dtype, int V) {
  for (int v = 0; v < V; ++v) {
    double x = load_logit(row, dtype, v);
    if (isnan(x) || x == INFINITY) return 0;
  }
  for (int v = 0; v < V; ++v)
    if (isfinite(load_logit(row, dtype, v))) return 1;
  return 0;
}

int oracle_scaled_max_in_range(const void* row, int dtype, int V, float T) {
  double m = -INFINITY;
  for (int v = 0; v < V; ++v) {
    double x = load_logit(row, dtype, v);
    if (x > m) m = x;
  }
  if (!isfinite(m)) return 0;
  /* log2(e) / T rounded toward zero to fp32, then max * that in fp32
   * (round to nearest), rounded up to an integer */
  const double s = 1.4426950408889634074 / (double)T;
  float s32 = (float)s;
  if ((double)s32 > s) s32 = nextafterf(s32, 0.0f);
  const float ref = ceilf((float)m * s32);
  return fabsf(ref) <= 0x1p24f;
}

/* A row whose softmax at temperature T the method can use: a finite maximum,
 * no NaN or +inf logit, and a scaled maximum in the fp32 range above. */
static int row_usable_at(const void* row, int dtype, int V, float T) {
  return row_has_finite_max(row, dtype, V) && oracle_scaled_max_in_range(row, dtype, V, T);
}

/* Drafts of request b: K, or its entry of the ragged table. */
static int drafts_of(const oracle_verify_args* a, int b) { return a->num_drafts ? a->num_drafts[b] : a->K; }

/* Data checks made before any decision, on the inputs alone: a draft count
 * in [0, K], every token id in range and a usable temperature.  The rows are
 * checked as the method reaches them (rows_usable). */
static int request_valid(const oracle_verify_args* a, int b) {
  const int Kb = drafts_of(a, b);
  if (Kb < 0 || Kb > a->K) return 0;
  const int32_t* x = a->draft_tokens + (int64_t)b * a->K;
  for (int k = 0; k < Kb; ++k)
    if (x[k] < 0 || x[k] >= a->V) return 0;
  float T = a->temperature[b];
  if (!(T >= 0.0f) || isinf(T) || (T > 0.0f && T < FLT_MIN)) return 0;
  return 1;
}

/* The rows a sampled request reads at position k (explainer page, section
 * "核心思想": the verification walks the positions in order and stops at the
 * first rejection, so a row after the stop is never read): target row k, and
 * draft row k when k < K_b (k = K_b is the bonus row, target only).  Each
 * needs a finite maximum for its softmax to exist. */
static int rows_usable(const oracle_verify_args* a, int b, int k, int Kb) {
  const float T = a->temperature[b];
  if (!row_usable_at(trow(a, b, k), a->dtype, a->V, T)) return 0;
  return k == Kb || row_usable_at(drow(a, b, k), a->dtype, a->V, T);
}

static void sampling_weights(const oracle_verify_args* a, int b, int j, double* p, double* q,
                             double* w, double* W) {
  double T = (double)a->temperature[b];
  oracle_softmax(trow(a, b, j), a->dtype, a->V, T, p);
  if (j == drafts_of(a, b) || a->mutation == 1) {
    /* the bonus row samples from p itself (mutation 1 plants the mistake of
     * resampling from p instead of the residual) */
    double S = 0.0;
    for (int v = 0; v < a->V; ++v) {
      w[v] = p[v];
      S += p[v];
    }
    *W = S;
    return;
  }
  oracle_softmax(drow(a, b, j), a->dtype, a->V, T, q);
  oracle_residual(p, q, a->V, w, W);
}

/* Request b's data is invalid: accepted = -1, every output token -1, debug 0. */
static int invalid_request(const oracle_verify_args* a, int b) {
  int32_t* out = a->out_tokens + (int64_t)b * (a->K + 1);
  for (int k = 0; k <= a->K; ++k) out[k] = -1;
  if (a->debug_probs)
    for (int i = 0; i < 2 * a->K; ++i) a->debug_probs[(int64_t)b * a->K * 2 + i] = 0.0f;
  if (a->trace)
    for (int i = 0; i < (a->K + 1) * 3; ++i) a->trace[(int64_t)b * (a->K + 1) * 3 + i] = NAN;
  a->accepted[b] = -1;
  return 1;
}

static int verify_one(const oracle_verify_args* a, int b, double* p, double* q, double* w) {
  int K = a->K;
  const int V = a->V;
  const int32_t* x = a->draft_tokens + (int64_t)b * K;
  int32_t* out = a->out_tokens + (int64_t)b * (K + 1);
  double* tr = a->trace ? a->trace + (int64_t)b * (K + 1) * 3 : NULL;
  for (int k = 0; k <= K; ++k) out[k] = -1;
  if (tr)
    for (int i = 0; i < (K + 1) * 3; ++i) tr[i] = NAN;
  if (a->debug_probs)
    for (int i = 0; i < 2 * K; ++i) a->debug_probs[(int64_t)b * K * 2 + i] = 0.0f;

  if (!request_valid(a, b)) return invalid_request(a, b);
  const double T = (double)a->temperature[b];
  K = drafts_of(a, b); /* positions k >= K_b do not exist; the bonus row is K_b */

  if (T == 0.0) { /* greedy */
    for (int k = 0; k < K; ++k) {
      int g = oracle_argmax(trow(a, b, k), a->dtype, V);
      if (x[k] != g) {
        out[k] = g;
        a->accepted[b] = k;
        return 0;
      }
      out[k] = x[k];
    }
    out[K] = oracle_argmax(trow(a, b, K), a->dtype, V);
    a->accepted[b] = K;
    return 0;
  }

  if (a->debug_probs) {
    /* every position's p_k(x_k), q_k(x_k), the parallel formulation's view
     * (0 where a row has no finite maximum) */
    for (int k = 0; k < K; ++k) {
      if (!rows_usable(a, b, k, K)) continue;
      oracle_softmax(trow(a, b, k), a->dtype, V, T, p);
      oracle_softmax(drow(a, b, k), a->dtype, V, T, q);
      a->debug_probs[((int64_t)b * a->K + k) * 2 + 0] = (float)p[x[k]];
      a->debug_probs[((int64_t)b * a->K + k) * 2 + 1] = (float)q[x[k]];
    }
  }

  for (int k = 0; k < K; ++k) {
    if (!rows_usable(a, b, k, K)) return invalid_request(a, b);
    oracle_softmax(trow(a, b, k), a->dtype, V, T, p);
    oracle_softmax(drow(a, b, k), a->dtype, V, T, q);
    double ua, us;
    uniforms_for(a, b, k, &ua, &us);
    double px = p[x[k]], qx = q[x[k]];
    int acc;
    if (a->mutation == 2) /* planted mistake: acceptance ignores q */
      acc = ua < px;
    else
      acc = oracle_accept(px, qx, ua);
    if (tr) {
      tr[k * 3 + 0] = ua;
      tr[k * 3 + 1] = a->mutation == 2 ? px : accept_threshold(px, qx);
    }
    if (acc) {
      out[k] = x[k];
      continue;
    }
    double W;
    if (a->mutation == 1) {
      W = 0.0;
      for (int v = 0; v < V; ++v) {
        w[v] = p[v];
        W += p[v];
      }
    } else {
      oracle_residual(p, q, V, w, &W);
    }
    if (tr) tr[k * 3 + 2] = us;
    out[k] = oracle_invcdf(w, V, W, us);
    a->accepted[b] = k;
    return 0;
  }

  /* all K drafts accepted: the bonus token is sampled from p at row K */
  if (!rows_usable(a, b, K, K)) return invalid_request(a, b);
  oracle_softmax(trow(a, b, K), a->dtype, V, T, p);
  double ua, us, W = 0.0;
  uniforms_for(a, b, K, &ua, &us);
  for (int v = 0; v < V; ++v) W += p[v];
  if (tr) tr[K * 3 + 2] = us;
  out[K] = oracle_invcdf(p, V, W, us);
  a->accepted[b] = K;
  return 0;
}

static int args_ok(const oracle_verify_args* a) {
  if (!a || a->B < 0 || a->K < 1 || a->V < 1) return 0;
  if (a->dtype != 0 && a->dtype != 1) return 0;
  if (a->B > 0 && (!a->target || !a->draft || !a->draft_tokens || !a->temperature ||
                   !a->accepted || !a->out_tokens))
    return 0;
  return 1;
}

int oracle_verify(const oracle_verify_args* a) {
  if (!args_ok(a)) return -1;
  int bad = 0;
  int nt = a->nthreads;
#ifdef _OPENMP
  if (nt <= 0) nt = omp_get_max_threads();
#pragma omp parallel num_threads(nt) reduction(+ : bad)
#endif
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)a->V);
    double* q = (double*)malloc(sizeof(double) * (size_t)a->V);
    double* w = (double*)malloc(sizeof(double) * (size_t)a->V);
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
    for (int b = 0; b < a->B; ++b) bad += verify_one(a, b, p, q, w);
    free(p);
    free(q);
    free(w);
  }
  (void)nt;
  return bad;
}

int oracle_sampling_weights(const oracle_verify_args* a, int b, int j, double* w, double* W) {
  /* inputs only: this call writes no verification outputs */
  if (!a || a->B < 1 || a->K < 1 || a->V < 1 || (a->dtype != 0 && a->dtype != 1)) return -1;
  if (!a->target || !a->draft || !a->draft_tokens || !a->temperature || !w || !W) return -1;
  if (b < 0 || b >= a->B || j < 0 || j > a->K) return -1;
  if (!request_valid(a, b) || !(a->temperature[b] > 0.0f) || j > drafts_of(a, b)) return -1;
  if (!rows_usable(a, b, j, drafts_of(a, b))) return -1;
  double* p = (double*)malloc(sizeof(double) * (size_t)a->V);
  double* q = (double*)malloc(sizeof(double) * (size_t)a->V);
  sampling_weights(a, b, j, p, q, w, W);
  free(p);
  free(q);
  return 0;
}
