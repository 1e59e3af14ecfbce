/* A C99 caller of the library's host-side entry points (no GPU needed):
 * compiled against include/spec_verify.h and linked to the built library by
 * tests/test_c_header.py.  Prints one "name value" line per call. */
#include <stdio.h>

#include "spec_verify.h"

int main(void) {
  const double survival[9] = {1.0, 0.8145, 0.7026, 0.6206, 0.5498, 0.501, 0.4668, 0.4395, 0.3989};
  spec_verify_args v = {0};
  spec_expand_args e = {0};
  spec_draft_args d = {0};
  spec_shard_args s = {0};
  printf("verify_workspace %zu\n", spec_verify_workspace_bytes(256, 8, 151936));
  printf("verify_workspace_bad %zu\n", spec_verify_workspace_bytes(4, SPEC_MAX_K + 1, 10));
  printf("draft_workspace %zu\n", spec_draft_workspace_bytes(256, 8, 151936));
  printf("shard_workspace %zu\n", spec_shard_workspace_bytes(256, 8, 37984));
  printf("plan %llu\n", (unsigned long long)spec_verify_plan_phases(8, survival, 2.0 / 3.0, 1.05));
  printf("plan_null %llu\n", (unsigned long long)spec_verify_plan_phases(8, NULL, 0.5, 1.0));
  printf("phase_cost %.17g\n", spec_verify_phase_cost(256, 8, 151936, SPEC_BF16));
  printf("phase_cost_bad %.17g\n", spec_verify_phase_cost(0, 8, 151936, SPEC_BF16));
  printf("verify_null %d\n", spec_verify_launch(NULL, NULL));
  v.K = 0; /* invalid: rejected before anything is enqueued */
  printf("verify_bad %d\n", spec_verify_launch(&v, NULL));
  e.K = 0;
  printf("expand_bad %d\n", spec_expand_launch(&e, NULL));
  printf("chained_bad %d\n", spec_verify_expand_launch(&v, &e, NULL));
  d.K = 0;
  printf("draft_bad %d\n", spec_draft_sample_launch(&d, NULL));
  s.G = 0;
  printf("shard_bad %d\n", spec_shard_stats_launch(&s, NULL));
  printf("status %s\n", spec_status_string(SPEC_EWORKSPACE));
  return 0;
}
