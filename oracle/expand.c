/*
 * expand.c -- CPU oracle for the P-EAGLE parallel-drafting batch expansion
 * and the hidden-state fill.
 *
 * TEST INFRASTRUCTURE ONLY (see spec_oracle.h).
 *
 * Sources: "P-EAGLE: parallel speculative decoding in vLLM" page.
 *  - "并行草稿生成的挑战": the drafter batch appends MASK placeholders
 *    ([token, MASK, MASK, ...]); token ids, hidden states and positions are
 *    expanded to make room for them, positions are advanced per request and
 *    the per-request start indices are recomputed.
 *  - "Triton Kernel": one pass copies the old token ids and positions into
 *    their new slots, inserts the per-request bonus token sampled by the
 *    target, fills the extra slots with the MASK id, and emits the
 *    rejected-token mask, the masked-token mask, the new-token indices used to
 *    sample draft tokens, and the hidden-state mapping.
 *  - "Hidden State 管理": the hidden rows are filled in two steps, the
 *    target rows scattered to their mapped slots, then the masked rows take
 *    the learned placeholder; valid tokens get their normal KV-cache slot and rejected
 *    tokens the padding slot -1, so that no cache entry is written for them.
 *  - "核心方法" step 2: the drafter input at a position pairs the token of the
 *    next position with the hidden state of this one (inputs shifted by one).
 *
 * Readings of points the page leaves open (listed in the design notes):
 * request b owns a fixed window of n_b + K - 1 output slots starting at
 * in_start[b] + b*(K-1); slot j < n_b pairs input hidden row j with the token
 * of the following position (the bonus at j = a_b, the input token j + 1
 * otherwise, clamped at the last input token), at position in_positions[j]+1;
 * slots j > a_b are the rejected ones; the K - 1 MASK slots follow at
 * positions in_positions[a_b] + 1 + m, m = 1..K-1; new-token indices are the
 * bonus slot then the MASK slots.  The "normal" slot is the paged-cache one:
 * logical block pos / block_size of the request through its block table, at
 * offset pos % block_size; a position without a block maps to -1 as well.
 */
#include "spec_oracle.h"

#include <string.h>

static int expand_args_ok(const oracle_expand_args* a) {
  if (!a || a->B < 0 || a->K < 1 || a->N_in < 0 || a->H < 0) return 0;
  if (!a->in_start || !a->accepted || !a->bonus || !a->out_start) return 0;
  if (a->B > 0 && (!a->in_token_ids || !a->in_positions || !a->out_token_ids ||
                   !a->out_positions || !a->rejected_mask || !a->masked_mask ||
                   !a->new_token_indices || !a->hidden_map))
    return 0;
  if (a->out_hidden && (!a->target_hidden || !a->mask_hidden || a->hidden_row_stride < a->H))
    return 0;
  if (a->slot_mapping && ((!a->block_table && a->max_blocks > 0) || a->block_size < 1 || a->max_blocks < 0 ||
                          a->bt_row_stride < a->max_blocks))
    return 0;
  return 1;
}

/* KV-cache slot of an output slot at position pos of request b. */
static int64_t cache_slot(const oracle_expand_args* a, int b, int64_t pos, int rejected) {
  if (rejected || pos < 0) return -1; /* PADDING_SLOT_ID */
  const int64_t block = pos / a->block_size;
  if (block >= a->max_blocks) return -1;
  const int32_t phys = a->block_table[(int64_t)b * a->bt_row_stride + block];
  if (phys < 0) return -1;
  return (int64_t)phys * a->block_size + pos % a->block_size;
}

static void mark_invalid(const oracle_expand_args* a, int b) {
  for (int m = 0; m < a->K; ++m) a->new_token_indices[(int64_t)b * a->K + m] = -1;
}

int oracle_expand(const oracle_expand_args* a) {
  if (!expand_args_ok(a)) return -1;
  const int B = a->B, K = a->K;
  if (B == 0) return 0; /* nothing to expand, nothing written */
  if (a->in_start[0] != 0 || a->in_start[B] != a->N_in) {
    /* the start indices do not describe the N_in input rows: every request is
     * invalid and only its new-token indices are written (all -1) */
    for (int b = 0; b < B; ++b) mark_invalid(a, b);
    return B;
  }

  for (int b = 0; b <= B; ++b) a->out_start[b] = a->in_start[b] + b * (K - 1);

  int bad = 0;
  for (int b = 0; b < B; ++b) {
    const int s = a->in_start[b];
    const int n = a->in_start[b + 1] - s;
    const int acc = a->accepted[b];
    const int o = a->out_start[b];
    if (n < 1 || s < 0 || a->in_start[b + 1] > a->N_in || acc < 0 || acc > n - 1) {
      mark_invalid(a, b);
      ++bad;
      continue;
    }
    for (int j = 0; j < n; ++j) {
      const int src_tok = j + 1 < n ? j + 1 : n - 1;
      a->hidden_map[s + j] = o + j;
      a->out_token_ids[o + j] = (j == acc) ? a->bonus[b] : a->in_token_ids[s + src_tok];
      a->out_positions[o + j] = a->in_positions[s + j] + 1;
      a->rejected_mask[o + j] = (uint8_t)(j > acc);
      a->masked_mask[o + j] = 0;
      if (a->slot_mapping) a->slot_mapping[o + j] = cache_slot(a, b, a->out_positions[o + j], j > acc);
    }
    for (int m = 1; m <= K - 1; ++m) {
      const int slot = o + n - 1 + m;
      a->out_token_ids[slot] = a->mask_id;
      a->out_positions[slot] = a->in_positions[s + acc] + 1 + m;
      a->rejected_mask[slot] = 0;
      a->masked_mask[slot] = 1;
      if (a->slot_mapping) a->slot_mapping[slot] = cache_slot(a, b, a->out_positions[slot], 0);
    }
    a->new_token_indices[(int64_t)b * K + 0] = o + acc;
    for (int m = 1; m <= K - 1; ++m) a->new_token_indices[(int64_t)b * K + m] = o + n - 1 + m;
  }

  if (a->out_hidden) {
    const int64_t H = a->H;
    /* statement 1: hidden[mapping] = target_hidden (rows of valid requests) */
    for (int b = 0; b < B; ++b) {
      const int s = a->in_start[b];
      const int n = a->in_start[b + 1] - s;
      const int acc = a->accepted[b];
      if (n < 1 || s < 0 || a->in_start[b + 1] > a->N_in || acc < 0 || acc > n - 1) continue;
      for (int i = s; i < s + n; ++i)
        memcpy(a->out_hidden + (int64_t)a->hidden_map[i] * H,
               a->target_hidden + (int64_t)i * a->hidden_row_stride, (size_t)H * 2);
    }
    /* statement 2: where(masked, placeholder, hidden) over the output rows of
     * valid requests */
    for (int b = 0; b < B; ++b) {
      const int s = a->in_start[b];
      const int n = a->in_start[b + 1] - s;
      const int acc = a->accepted[b];
      if (n < 1 || s < 0 || a->in_start[b + 1] > a->N_in || acc < 0 || acc > n - 1) continue;
      const int o = a->out_start[b];
      for (int slot = o; slot < o + n + K - 1; ++slot)
        if (a->masked_mask[slot]) memcpy(a->out_hidden + (int64_t)slot * H, a->mask_hidden, (size_t)H * 2);
    }
  }
  return bad;
}
