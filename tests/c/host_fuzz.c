/* The library's host-side code driven over many inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py;
 * no GPU needed): workspace sizing across shapes, the boundary price, the
 * phase planner on pseudo-random acceptance curves (each plan checked against
 * enumeration of every cut for small K), and the argument checks of every
 * entry point on arguments that must be refused before anything is enqueued.
 * Prints "ok <count>" and exits 0, or the first mismatch and exits 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "spec_verify.h"

static uint64_t lcg = 0x9E3779B97F4A7C15ull;
static double unif(void) {
  lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg >> 11) * 0x1p-53;
}

/* expected rows read under a cut (the planner's model), for enumeration */
static double cut_cost(int K, uint64_t mask, const double* s, double f, double cost) {
  double total = 0.0;
  int lo = 0, phases = 0;
  while (lo <= K) {
    int hi = lo + 1;
    while (hi <= K && !((mask >> hi) & 1u)) ++hi;
    total += s[lo] * ((double)(hi - lo) + f * (double)((hi < K ? hi : K) - lo));
    ++phases;
    lo = hi;
  }
  return total + cost * (double)(phases - 1);
}

static int fail(const char* what, long a, long b) {
  printf("mismatch %s %ld %ld\n", what, a, b);
  return 1;
}

int main(void) {
  long checks = 0;
  /* workspace sizing: zero for invalid shapes, growing with every dimension */
  const int32_t Bs[] = {-1, 0, 1, 7, 256, 1024, 65536};
  const int32_t Ks[] = {-1, 0, 1, 5, 8, 63, 64};
  const int32_t Vs[] = {-5, 0, 1, 9, 4096, 151936, 201088, SPEC_MAX_V};
  for (size_t i = 0; i < sizeof Bs / sizeof *Bs; ++i)
    for (size_t j = 0; j < sizeof Ks / sizeof *Ks; ++j)
      for (size_t k = 0; k < sizeof Vs / sizeof *Vs; ++k) {
        const int32_t B = Bs[i], K = Ks[j], V = Vs[k];
        const int valid = B >= 0 && K >= 1 && K <= SPEC_MAX_K && V >= 1 && V <= SPEC_MAX_V;
        const size_t w = spec_verify_workspace_bytes(B, K, V);
        if (!valid && w != 0) return fail("verify_workspace", B, K);
        if (valid && w == 0) return fail("verify_workspace_zero", B, K);
        if (valid && B > 0 && w < spec_verify_workspace_bytes(B - 1, K, V))
          return fail("verify_workspace_monotone", B, K);
        (void)spec_draft_workspace_bytes(B, K, V);
        (void)spec_shard_workspace_bytes(B, K, V);
        const double c = spec_verify_phase_cost(B, K, V, SPEC_BF16);
        if ((!valid || B == 0) != (c == -1.0)) return fail("phase_cost", B, K);
        if (c != -1.0 && !(c > 0.0 && isfinite(c))) return fail("phase_cost_range", B, K);
        checks += 4;
      }
  /* the planner: random non-increasing curves, checked against every cut */
  double s[SPEC_MAX_K + 2];
  for (int trial = 0; trial < 4000; ++trial) {
    const int K = 1 + (int)(unif() * (trial % 4 == 0 ? SPEC_MAX_K : 10));
    s[0] = 1.0;
    for (int k = 1; k <= K; ++k) s[k] = s[k - 1] * (trial % 7 == 0 ? 1.0 : unif());
    const double f = unif(), cost = trial % 5 == 0 ? 0.0 : 3.0 * unif();
    const uint64_t m = spec_verify_plan_phases(K, s, f, cost);
    if (m & 1u) return fail("plan_bit0", trial, (long)m);
    if (K < 63 && (m >> (K + 1)) != 0) return fail("plan_range", trial, (long)m);
    if (K <= 12) {
      const double got = cut_cost(K, m, s, f, cost);
      for (uint64_t c = 0; c < ((uint64_t)1 << K); ++c)
        if (cut_cost(K, c << 1, s, f, cost) < got - 1e-9) return fail("plan_not_optimal", trial, (long)c);
    }
    ++checks;
  }
  const double bad_costs[] = {-1.0, NAN, INFINITY, 1e300};
  for (int i = 0; i < 4; ++i)
    if (spec_verify_plan_phases(8, s, 0.5, bad_costs[i]) != 0) return fail("plan_bad_cost", i, 0);
  s[3] = 1.5;
  if (spec_verify_plan_phases(8, s, 0.5, 1.0) != 0) return fail("plan_bad_survival", 0, 0);
  checks += 5;

  /* argument errors: every call below must be refused before any HIP call */
  char fake[64];
  void* dev = (void*)(fake + 16 - ((uintptr_t)fake & 15u));  /* never dereferenced */
  spec_verify_args v;
  memset(&v, 0, sizeof v);
  v.B = 4; v.K = 3; v.V = 1000; v.dtype = SPEC_BF16;
  v.target_logits = v.draft_logits = dev;
  v.t_row_stride = v.d_row_stride = 1000;
  v.t_req_stride = 4 * 1000; v.d_req_stride = 3 * 1000;
  v.draft_tokens = (const int32_t*)dev; v.temperature = (const float*)dev;
  v.accepted_counts = (int32_t*)dev; v.output_tokens = (int32_t*)dev;
  v.workspace = dev; v.workspace_bytes = 16;  /* too small */
  if (spec_verify_launch(&v, NULL) != SPEC_EWORKSPACE) return fail("verify_ws", 0, 0);
  spec_verify_args w = v;
  w.workspace = (char*)dev + 4;
  w.workspace_bytes = (size_t)1 << 40;
  if (spec_verify_launch(&w, NULL) != SPEC_EALIGN) return fail("verify_align", 0, 0);
  w = v; w.dtype = 9;
  if (spec_verify_launch(&w, NULL) != SPEC_EDTYPE) return fail("verify_dtype", 0, 0);
  w = v; w.phase_starts = 3; /* bit 0 (the dynamic exit) with a cut */
  w.workspace_bytes = (size_t)1 << 40;
  if (spec_verify_launch(&w, NULL) != SPEC_EINVAL) return fail("verify_phase_bit0", 0, 0);
  w.phase_starts = (uint64_t)1 << 5;
  if (spec_verify_launch(&w, NULL) != SPEC_EINVAL) return fail("verify_phase_range", 0, 0);
  w = v; w.t_row_stride = 999;
  if (spec_verify_launch(&w, NULL) != SPEC_EINVAL) return fail("verify_stride", 0, 0);
  w = v; w.t_req_stride = 3999;
  if (spec_verify_launch(&w, NULL) != SPEC_EINVAL) return fail("verify_req_stride", 0, 0);
  w = v; w.temperature = NULL;
  if (spec_verify_launch(&w, NULL) != SPEC_EINVAL) return fail("verify_null", 0, 0);
  w = v; w.B = 4096; w.K = 8; w.V = 201088; w.t_row_stride = w.d_row_stride = 201088;
  w.t_req_stride = 9 * 201088; w.d_req_stride = 8 * 201088;
  if (spec_verify_launch_noalloc(&w, NULL) != SPEC_EWORKSPACE) return fail("noalloc_ws", 0, 0);
  w.K = 64;
  if (spec_verify_launch_noalloc(&w, NULL) != SPEC_EINVAL) return fail("noalloc_k", 0, 0);
  checks += 10;

  spec_expand_args e;
  memset(&e, 0, sizeof e);
  e.B = 2; e.K = 3; e.H = 8; e.N_in = 8;
  e.in_token_ids = (const int32_t*)dev; e.in_positions = (const int64_t*)dev; e.in_start = (const int32_t*)dev;
  e.accepted_counts = (const int32_t*)dev;
  e.out_token_ids = (int32_t*)dev; e.out_positions = (int64_t*)dev; e.rejected_mask = (uint8_t*)dev;
  e.masked_mask = (uint8_t*)dev; e.new_token_indices = (int32_t*)dev; e.hidden_map = (int32_t*)dev;
  e.out_start = (int32_t*)dev;
  if (spec_expand_launch(&e, NULL) != SPEC_EINVAL) return fail("expand_no_bonus", 0, 0);  /* no bonus source */
  spec_expand_args x = e;
  x.bonus_tokens = (const int32_t*)dev; x.verify_output_tokens = (const int32_t*)dev;
  if (spec_expand_launch(&x, NULL) != SPEC_EINVAL) return fail("expand_two_bonus", 0, 0);
  x = e; x.bonus_tokens = (const int32_t*)dev; x.out_hidden = (uint16_t*)dev; x.hidden_row_stride = 4;
  x.mask_hidden = (const uint16_t*)dev; x.target_hidden = (const uint16_t*)dev;
  if (spec_expand_launch(&x, NULL) != SPEC_EINVAL) return fail("expand_stride", 0, 0);
  x = e; x.bonus_tokens = (const int32_t*)dev; x.slot_mapping = (int64_t*)dev; x.block_size = 0;
  if (spec_expand_launch(&x, NULL) != SPEC_EINVAL) return fail("expand_block", 0, 0);
  x = e; x.bonus_tokens = (const int32_t*)dev; x.N_in = INT32_MAX;
  if (spec_expand_launch(&x, NULL) != SPEC_EINVAL) return fail("expand_overflow", 0, 0);
  if (spec_expand_hidden_launch(&x, NULL) != SPEC_EINVAL) return fail("expand_hidden_overflow", 0, 0);
  x = e; x.bonus_tokens = (const int32_t*)dev; x.B = 3;
  if (spec_verify_expand_launch(&v, &x, NULL) != SPEC_EWORKSPACE) return fail("chained", 0, 0);
  checks += 7;

  spec_draft_args d;
  memset(&d, 0, sizeof d);
  d.B = 2; d.K = 3; d.V = 100; d.N = 4; d.dtype = SPEC_F32; d.logits = dev; d.row_stride = 99;
  d.row_index = (const int32_t*)dev; d.temperature = (const float*)dev; d.tokens = (int32_t*)dev;
  d.workspace = dev; d.workspace_bytes = (size_t)1 << 30;
  if (spec_draft_sample_launch(&d, NULL) != SPEC_EINVAL) return fail("draft_stride", 0, 0);
  d.row_stride = 100; d.workspace_bytes = 1;
  if (spec_draft_sample_launch(&d, NULL) != SPEC_EWORKSPACE) return fail("draft_ws", 0, 0);
  checks += 2;

  spec_shard_args h;
  memset(&h, 0, sizeof h);
  h.B = 2; h.K = 3; h.V = 100; h.dtype = SPEC_BF16; h.G = 2; h.g = 1; h.v0 = 50; h.Vs = 51;  /* past V */
  if (spec_shard_stats_launch(&h, NULL) != SPEC_EINVAL) return fail("shard_slice", 0, 0);
  h.Vs = 50; h.g = 2;
  if (spec_shard_decide_launch(&h, NULL) != SPEC_EINVAL) return fail("shard_g", 0, 0);
  h.g = 1;
  if (spec_shard_draw_launch(&h, NULL) != SPEC_EINVAL) return fail("shard_null", 0, 0);
  checks += 3;

  for (int st = -10; st <= 3; ++st)
    if (spec_status_string(st) == NULL || strlen(spec_status_string(st)) == 0) return fail("status", st, 0);
  printf("ok %ld\n", checks);
  return 0;
}
