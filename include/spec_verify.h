/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) speculative-decoding hot path:
 * batched modified-rejection-sampling verification and the P-EAGLE
 * parallel-drafting batch expansion with its hidden-state gather.
 *
 * Conventions for every entry point
 *  - Pointers marked "device" are HIP device pointers; the library never
 *    dereferences them on the host.  Pointers to the argument structs are host
 *    pointers, read only during the call.
 *  - The caller owns all memory and keeps it alive until the stream has passed
 *    the launch.  The library allocates nothing, keeps no per-call state and
 *    performs no host-device synchronisation inside *_launch; work is enqueued
 *    asynchronously on `stream` (a hipStream_t; 0 = the null stream).
 *  - Argument errors are returned synchronously as a negative spec_status
 *    before anything is enqueued.  Data errors only the device can see are
 *    reported per request in the outputs (documented per call).
 *  - Strides are in elements.  Vectorised 16-byte loads are used when the
 *    logits/hidden base pointers and row strides are 16-byte aligned; other
 *    layouts take a scalar path with identical results.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

typedef enum {
  SPEC_OK = 0,
  SPEC_EINVAL = -1,     /* null pointer, size or stride out of range (also a batch whose kernel
                           grids would exceed one dispatch's 2^32 work-items) */
  SPEC_EDTYPE = -2,     /* unknown logits dtype */
  SPEC_EALIGN = -3,     /* workspace (or a statistics record array) not 16-byte aligned */
  SPEC_EWORKSPACE = -4, /* workspace smaller than spec_verify_workspace_bytes() */
  SPEC_ELAUNCH = -5     /* the HIP runtime refused a launch */
} spec_status;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* spec_verify_args.phase_starts value selecting the dynamic early exit (the
 * row pass takes the decisions as it goes; see "Early exit" below). */
#define SPEC_PHASES_DYNAMIC 1ull

/* Largest number of drafts per request (one 64-lane wavefront ballot). */
#define SPEC_MAX_K 63

/* Largest vocabulary (2^31 - 2^16): every index into a row, padded to whole
 * 4096-logit segments, stays within 32 bits.  Larger V is SPEC_EINVAL. */
#define SPEC_MAX_V 2147418112

/* ------------------------------------------------------------- verification
 *
 * Defined by the explainer page on speculative decoding, section "修正拒绝采样"
 * (accept draft token x with probability min(1, p(x)/q(x)); on rejection
 * resample from normalize(max(0, p - q)); the emitted law is p) and section
 * "核心思想" (the target scores K+1 positions at once; stop at the first
 * rejection; all K accepted yields K+1 tokens, the last sampled from p), with
 * the greedy limit of the same page: temperature 0 accepts iff the draft is
 * the target argmax and emits the target argmax where it stops.
 *
 * For request b with temperature T_b > 0, p_k = softmax(target[b,k,:] / T_b)
 * and q_k = softmax(draft[b,k,:] / T_b).  Uniforms: Philox4x32-10 with counter
 * {b + request_base, k, step, 0} and key {seed & 0xffffffff, seed >> 32};
 * word 0 -> u_k for the accept test at row k, word 1 -> u'_k for the sampling
 * draw at row k; a word w maps to (w >> 8) * 2^-24.  Accept iff
 * u_k < min(1, p_k(x_k) / q_k(x_k)) (q_k(x_k) = 0: accept iff p_k(x_k) > 0).
 * a_b = number of leading accepts.  If a_b < K the emitted token is the
 * smallest v with r(v) > 0 and u'_{a} * R < sum_{i<=v} r(i), r = max(0, p_a -
 * q_a), R = sum r (if R == 0, r = p_a); if a_b == K it is drawn the same way
 * from r = p_K.  Argmax ties (T = 0) go to the lowest index.
 *
 * Layouts: target [B, K+1, V] and draft [B, >=K, V] with the given request and
 * row strides (request stride 0 shares one set of rows across all requests);
 * draft row K is never read, and draft rows are not read at all for T_b = 0.
 *
 * Data checked as the request reaches its rows (the target and draft row of
 * a position it tests, or its bonus row): a row of a sampled request must
 * have a finite maximum, no NaN or +inf logit, and its largest logit m must
 * satisfy |ceil(m * s)| <= 2^24 with s = log2(e) / T_b (|m| / T_b up to about
 * 1.16e7); a row that does not is a data error.  A greedy row may hold NaN
 * (counted as -inf) and +inf logits.
 */
typedef struct {
  int32_t B;                   /* requests, >= 0 */
  int32_t K;                   /* drafts per request, 1..SPEC_MAX_K */
  int32_t V;                   /* vocabulary size, 1..SPEC_MAX_V */
  int32_t dtype;               /* spec_dtype of both logits tensors */
  const void* target_logits;   /* device [B, K+1, V] */
  int64_t t_req_stride;        /* elements between requests (0 = shared), else >= (K+1)*t_row_stride */
  int64_t t_row_stride;        /* elements between rows, >= V */
  const void* draft_logits;    /* device [B, >=K, V] */
  int64_t d_req_stride;        /* 0 = shared, else >= K*d_row_stride */
  int64_t d_row_stride;        /* >= V */
  const int32_t* draft_tokens; /* device [B, K], the K draft tokens of each request */
  const float* temperature;    /* device [B]; 0 = greedy */
  uint64_t seed;               /* Philox key */
  uint32_t step;               /* Philox counter word 2 (decode step) */
  uint32_t request_base;       /* added to the request index in the counter */
  int32_t* accepted_counts;    /* device out [B]: a_b in 0..K; -1 = invalid request data */
  int32_t* output_tokens;      /* device out [B, K+1]: x_0..x_{a-1}, the emitted token, then -1 */
  float* debug_probs;          /* device out [B, K, 2] or NULL: p_k(x_k), q_k(x_k) (0 for T = 0) */
  void* workspace;             /* device scratch, >= spec_verify_workspace_bytes(B, K, V) bytes, 16-B aligned */
  size_t workspace_bytes;
  void* phase_event;           /* hipEvent_t or NULL: recorded on `stream` right after the
                                  row-statistics stage (to time it apart from the rest) */
  uint64_t phase_starts;       /* early exit: bit k (1 <= k <= K) starts a new phase at draft
                                  position k; 0 = one pass over every row;
                                  SPEC_PHASES_DYNAMIC = decisions inside the row pass (see below) */
  const int32_t* draft_row_index; /* device [B, K] or NULL: draft row k of request b is row
                                  draft_row_index[b*K + k] of a [draft_rows, V] buffer at
                                  draft_logits (row stride d_row_stride; d_req_stride unused),
                                  e.g. the drafter's logits at the new-token indices */
  int32_t draft_rows;          /* rows of that buffer; an entry outside [0, draft_rows) makes a
                                  sampled request invalid */
  const int32_t* num_drafts;   /* device [B] or NULL: ragged draft counts K_b in [0, K]; positions
                                  k >= K_b do not exist (their tokens and rows are never read), a
                                  request that accepts all K_b drafts takes the bonus from target
                                  row K_b; a count outside [0, K] makes the request invalid */
  const void* draft_stats;     /* device [B, K] records of 16 bytes (16-byte aligned), or NULL: the statistics of the
                                  draft rows as spec_draft_sample_launch wrote them (stats_out) when
                                  it drew draft_tokens from these rows at these temperatures; the
                                  row statistics then read no draft row (see below) */
} spec_verify_args;

/* Early exit (same explainer page, section "核心思想": a request stops at
 * its first rejection, so the rows after it are never needed).  With
 * phase_starts != 0 the positions 0..K are cut into phases at the set bits;
 * the rows of a phase (target rows k and, for sampled requests, draft rows k
 * of its positions) are read only for requests whose drafts before the phase
 * were all accepted, and a small kernel between phases runs the phase's
 * accept tests.  With phase_starts == SPEC_PHASES_DYNAMIC there is one row
 * pass, ordered by position, and workgroups inside it run the accept tests
 * of each request as the records of its rows come in, so that the rows of a
 * request past its stop are mostly never read; no plan is needed, and how
 * many rows are skipped depends on timing, not the outputs: the final
 * decision recomputes every test from the rows read, and a request's rows up
 * to its stop are always read.  In every mode accepted_counts and
 * output_tokens are identical to the one-pass result (a row without a finite
 * normaliser counts only at or before the position where the request stops,
 * in every mode).  debug_probs: positions in phases after the one where a
 * request stopped are 0 (their rows are never read); with the dynamic exit
 * every position past the stop is 0. */

/* Draft statistics (same explainer page, section "修正拒绝采样": the
 * accept test needs q only at the drafted token, and its normaliser).  In
 * the P-EAGLE round the draft tokens are drawn from the drafter's rows by
 * spec_draft_sample_launch, which reduces every such row to its normaliser
 * on the way; with draft_stats those records stand in for the row pass over
 * the draft rows, so the row statistics read the target rows only.  A
 * sampled request's q row is still read where the request stops (the
 * residual's weights).  The outputs follow the same method and uniforms;
 * they can differ from reading the rows only where a decision sits within
 * rounding of its threshold (the two reductions round differently).  A
 * record without a finite normaliser makes a sampled request invalid.
 * Records of greedy requests are not read.  Preconditions: record [b, k]
 * was written for token draft_tokens[b, k] of draft row k of request b at
 * temperature[b]. */

/* A phase plan for phase_starts: minimises the expected rows read plus
 * phase_cost per extra phase, over every way of cutting 0..K into phases,
 * when a request reaches position k (all drafts before k accepted) with
 * probability survival[k] (host array [K+1], survival[0] = 1; e.g. measured
 * on recent steps).  Rows are counted per request: one target row per
 * position 0..K plus sampled_fraction draft rows per position 0..K-1; phase_cost
 * is the time of one phase boundary in units of the time to read one row for
 * every request.  Returns 0 (one pass) when that is best or an argument is out
 * of range (K outside 1..SPEC_MAX_K, NULL survival, negative or non-finite
 * inputs). */
uint64_t spec_verify_plan_phases(int32_t K, const double* survival, double sampled_fraction, double phase_cost);

/* The price of one phase boundary on MI355X for a batch of this shape, in the
 * unit spec_verify_plan_phases takes (the time to read one row of every
 * request, B * V logits of `dtype`, at the row pass's streaming rate of
 * 6.8 TB/s).  A boundary costs its decision kernel, two launch gaps and the
 * ramp-up and tail of one more row-pass kernel: 12 us measured at B = 256
 * and B = 1024, plus up to 7.7 us more when one row of every request is less
 * than one dispatch round of the row pass (B * chunks per row below the
 * 1280 workgroups 256 compute units hold at once), fitted to B = 64
 * (V = 201088) where a boundary costs ~17 us.  Returns -1 for an invalid
 * shape (which spec_verify_plan_phases turns into the one-pass plan). */
double spec_verify_phase_cost(int32_t B, int32_t K, int32_t V, int32_t dtype);

/* Bytes of device workspace a verification of this shape needs (0 for an
 * invalid shape).  The workspace needs no initialisation and may be reused
 * for any shape it is large enough for; calls that overlap on one workspace
 * race.  What it carries from one call to the next: the invalid-request count
 * that spec_workspace_error reads, and a launch counter with per-request
 * words of the dynamic early exit, which tag what a launch wrote so that it
 * is told apart from anything older and from memory never written (zero bytes
 * never carry a tag).  Leftover bytes can only make that mode read more
 * rows, never change an output (a request's rows up to its stop are read
 * unless leftover words match this launch's tags by chance: its 56-bit tag
 * in a state word, or its 48-bit tags in all eight words of a record, which
 * repeat only after 2^94 launches, and in any one word only after 2^47, so
 * that a record caught half-written is told apart too; the final decision
 * reports a request invalid if that happened). */
size_t spec_verify_workspace_bytes(int32_t B, int32_t K, int32_t V);

/* Enqueue one verification step.  A request whose data is invalid (a draft
 * token outside [0, V), a temperature that is negative, NaN, infinite or
 * positive below FLT_MIN, a draft row table entry of a sampled request
 * outside [0, draft_rows), a draft count outside [0, K], or, at a position the
 * request reaches, a row of a sampled request without a finite normaliser or
 * whose largest logit m has |ceil(m * log2(e) / T)| above 2^24, the range in
 * which the kernels hold a row's scaled maximum exactly in fp32: |m| / T up
 * to about 1.16e7) gets accepted_counts = -1, output_tokens all -1 and
 * debug_probs 0.  A batch whose kernel grids would
 * exceed one dispatch (2^32 work-items per launch) returns SPEC_EINVAL before
 * anything is enqueued: the draw needs B * 512 < 2^32, the segment sums
 * B * ceil(V / 4096) * 64 < 2^32, and above B = 65535 the row pass needs
 * B * (2K + 1) * ceil(V / 32768) * 256 < 2^32 (about B = 197K at K = 8,
 * V = 151936); split larger batches over calls with request_base. */
int spec_verify_launch(const spec_verify_args* args, hipStream_t stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the same
 * verification as spec_verify_launch (same checks, kernels and outputs),
 * with args->workspace and args->workspace_bytes ignored.  Its workspace is a
 * SPEC_NOALLOC_SCRATCH_BYTES array of device memory inside the library, one
 * per GPU, held from the first call on that GPU until the process ends; the
 * call allocates nothing.  The stream must belong to the current device
 * (else SPEC_EINVAL).  A shape whose spec_verify_workspace_bytes exceeds
 * SPEC_NOALLOC_SCRATCH_BYTES returns SPEC_EWORKSPACE before anything is
 * enqueued (16 MiB holds B = 1024, K = 8, V = 201088: 10.2 MiB).
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * that GPU (other streams, or graphs replayed concurrently) race and must be
 * ordered by the caller.  Invalid requests are reported in the outputs
 * (accepted_counts = -1); their count is not readable through
 * spec_workspace_error. */
#define SPEC_NOALLOC_SCRATCH_BYTES (16u << 20)
int spec_verify_launch_noalloc(const spec_verify_args* args, hipStream_t stream);

/* The data errors of the last verification enqueued on this workspace: waits
 * for `stream` (so it is not for graph capture or a tight loop), then returns
 * the number of requests that verification found invalid (the ones with
 * accepted_counts = -1; 0 when every request was valid).  The count lives in
 * the first 4 bytes of the workspace and is cleared by each verification with
 * B >= 1.  Returns SPEC_EINVAL for a NULL workspace and SPEC_ELAUNCH if the
 * stream reports an error or the copy fails. */
int spec_workspace_error(const void* workspace, hipStream_t stream);

/* ---------------------------------------------------------------- expansion
 *
 * Defined by the "P-EAGLE: parallel speculative decoding in vLLM" page:
 * section "并行草稿生成的挑战" (the drafter batch appends K-1 MASK slots per
 * request, [token, MASK, ...]; ids, hidden states and positions are expanded,
 * positions advance per request, start indices are recomputed), section
 * "Triton Kernel" (one pass copies the old ids and positions into shifted
 * slots, inserts each request's bonus token, fills the MASK slots and emits
 * the rejected-token mask, the masked-token mask, the new-token indices and
 * the hidden-state mapping), section "Hidden State 管理" (target hidden rows go
 * to their mapped slots, MASK slots take the learned placeholder row) and
 * section "核心方法" step 2 (a drafter input pairs the hidden state of a
 * position with the token of the next position).
 *
 * Layout (per request b, n_b = in_start[b+1] - in_start[b], a = a_b):
 *   out_start[b] = o_b = in_start[b] + b*(K-1); request b owns slots
 *   [o_b, o_b + n_b + K - 1); N_out = N_in + B*(K-1).
 *   slot o_b+j, j < n_b: hidden row in_start[b]+j (hidden_map), token = the
 *     bonus if j == a else in_token_ids[in_start[b] + min(j+1, n_b-1)],
 *     position in_positions[in_start[b]+j] + 1, rejected iff j > a;
 *   slot o_b+n_b-1+m, m = 1..K-1: MASK id, position
 *     in_positions[in_start[b]+a] + 1 + m, masked, hidden = mask_hidden;
 *   new_token_indices[b] = {o_b + a, o_b + n_b, ..., o_b + n_b + K - 2}.
 * KV-cache slot mapping (same page, section "Hidden State 管理": valid tokens
 * get their normal slot, rejected tokens PADDING_SLOT_ID = -1 so that nothing
 * is written to the cache for them): slot o_b+j at position pos maps to
 *   block_table[b, pos / block_size] * block_size + pos % block_size,
 * or -1 when the slot is rejected or pos has no block (pos < 0,
 * pos / block_size >= max_blocks, or a negative table entry).  MASK slots are
 * drafter positions and get their slot.
 * A request with n_b < 1, a window outside [0, N_in] or a outside
 * [0, n_b - 1] (or above K when the bonus comes from verify_output_tokens)
 * writes only new_token_indices[b, :] = -1.  If in_start[0] != 0
 * or in_start[B] != N_in every request does so and out_start is not written.
 * A decreasing in_start is outside the contract (results unspecified, all
 * accesses stay in bounds).
 */
typedef struct {
  int32_t B;                      /* requests, >= 0 */
  int32_t K;                      /* drafts per request, >= 1 */
  int32_t H;                      /* hidden width (bf16 elements), >= 0 */
  int32_t N_in;                   /* input slots, = in_start[B] */
  const int32_t* in_token_ids;    /* device [N_in] */
  const int64_t* in_positions;    /* device [N_in] */
  const int32_t* in_start;        /* device [B+1] */
  const int32_t* accepted_counts; /* device [B] */
  const int32_t* bonus_tokens;    /* device [B], or NULL when verify_output_tokens is given */
  const int32_t* verify_output_tokens; /* device [B, K+1] or NULL: output_tokens of a verification
                                  with the same B and K; the bonus of request b is then
                                  verify_output_tokens[b*(K+1) + a_b], which needs a_b <= K */
  int32_t mask_token_id;
  const uint16_t* target_hidden;  /* device bf16 bits [N_in, H] with row stride below */
  int64_t hidden_row_stride;      /* elements, >= H */
  const uint16_t* mask_hidden;    /* device bf16 bits [H] */
  int32_t* out_token_ids;         /* device out [N_out] */
  int64_t* out_positions;         /* device out [N_out] */
  uint8_t* rejected_mask;         /* device out [N_out] */
  uint8_t* masked_mask;           /* device out [N_out] */
  int32_t* new_token_indices;     /* device out [B, K] */
  int32_t* hidden_map;            /* device out [N_in] */
  int32_t* out_start;             /* device out [B+1] */
  uint16_t* out_hidden;           /* device out bf16 bits [N_out, H], or NULL to skip the gather */
  /* KV-cache slot mapping (all four inputs ignored when slot_mapping is NULL) */
  const int32_t* block_table;     /* device [B, >= max_blocks] physical block ids (< 0: none) */
  int64_t bt_row_stride;          /* elements between requests' rows, >= max_blocks */
  int32_t max_blocks;             /* logical blocks per request in the table, >= 0 */
  int32_t block_size;             /* cache slots per block, >= 1 */
  int64_t* slot_mapping;          /* device out [N_out], or NULL */
} spec_expand_args;

/* Enqueue one expansion (metadata and, if out_hidden != NULL, the hidden-row
 * gather) as a single kernel. */
int spec_expand_launch(const spec_expand_args* args, hipStream_t stream);

/* Enqueue only the hidden-row gather of an expansion.  The hidden rows depend
 * on in_start, target_hidden and mask_hidden alone -- not on the accepted
 * counts -- so this may run on another stream while the verification that
 * produces the counts is still running; spec_expand_launch with
 * out_hidden = NULL then writes the metadata.  Reads in_start, target_hidden,
 * hidden_row_stride, mask_hidden, B, K, H, N_in; writes out_hidden for every
 * request whose window is valid (n_b >= 1 inside [0, N_in], in_start[0] = 0,
 * in_start[B] = N_in), whatever its accepted count. */
int spec_expand_hidden_launch(const spec_expand_args* args, hipStream_t stream);

/* One verification step and the expansion of its outputs, enqueued as one
 * chained call: `v` as for spec_verify_launch and `e` as for
 * spec_expand_launch, with e->accepted_counts == v->accepted_counts and
 * e->verify_output_tokens == v->output_tokens (the expansion of this very
 * verification; e->bonus_tokens NULL) and the same B and K.  The results are
 * those of spec_verify_launch followed by spec_expand_launch; the expansion's
 * work runs inside the verification's sampling stage (its hidden rows and the
 * metadata after the decision, a sampled request's bonus id with the draw),
 * so no expansion kernel of its own is launched.  Argument errors of either
 * part, or arrays that do not chain as above, return SPEC_EINVAL (or the
 * part's own status) before anything is enqueued. */
int spec_verify_expand_launch(const spec_verify_args* v, const spec_expand_args* e, hipStream_t stream);

/* ----------------------------------------------------------- draft sampling
 *
 * The next draft tokens, sampled from the drafter's logits at the new-token
 * indices of an expansion ("P-EAGLE" page, section "Triton Kernel": the
 * new-token indices are the rows at which the draft tokens are sampled; one
 * drafter pass predicts all K, section "核心方法").  Token k of request b is
 * drawn from q = softmax(logits[row_index[b, k]] / T_b) -- the distribution
 * the next verification checks it against (explainer page, section
 * "修正拒绝采样") -- by the inverse CDF in ascending vocabulary order with one
 * uniform: Philox4x32-10 counter {b + request_base, k, step, 1} (a stream
 * apart from the verification's, which uses word 3 = 0), key as for
 * verification, word 0, mapped as (w >> 8) * 2^-24.  Temperature 0 takes the
 * lowest-index argmax.
 *
 * Layout: logits [N, V] (row stride >= V elements), row_index [B, K] (for
 * instance the new_token_indices of spec_expand_launch), temperature [B].
 * A position whose row index is outside [0, N), a request whose temperature is
 * negative, NaN, infinite or positive below FLT_MIN, and (T > 0) a row
 * without a finite normaliser (no finite logit, or a NaN or +inf one) or
 * whose largest logit m has |ceil(m * log2(e) / T)| above 2^24 get token -1.
 */
typedef struct {
  int32_t B;                   /* requests, >= 0 */
  int32_t K;                   /* draft positions per request, >= 1 */
  int32_t V;                   /* vocabulary size, 1..SPEC_MAX_V */
  int32_t N;                   /* rows of the logits buffer, >= 0 */
  int32_t dtype;               /* spec_dtype of the logits */
  const void* logits;          /* device [N, V] drafter logits */
  int64_t row_stride;          /* elements between rows, >= V */
  const int32_t* row_index;    /* device [B, K]: logits row of position k of request b */
  const float* temperature;    /* device [B]; 0 = greedy */
  uint64_t seed;               /* Philox key */
  uint32_t step;               /* Philox counter word 2 */
  uint32_t request_base;       /* added to the request index in the counter */
  int32_t* tokens;             /* device out [B, K] */
  void* workspace;             /* device scratch, >= spec_draft_workspace_bytes(B, K, V), 16-B aligned */
  size_t workspace_bytes;
  void* stats_out;             /* device out [B, K] records of 16 bytes (16-byte aligned), or NULL: for a position drawn
                                  at T > 0, the row's normaliser S * 2^M of sum_v 2^(x_v * log2(e) / T)
                                  (float M, integer-valued, at byte 0; double S at byte 8) and the
                                  drawn token's logit as stored (bf16 bits zero-extended, or fp32
                                  bits; 4 bytes at byte 4) -- what spec_verify_args.draft_stats
                                  takes; zeros for T = 0 and for positions given token -1 */
} spec_draft_args;

/* Bytes of device workspace a draft sampling of this shape needs (0 for an
 * invalid shape); stateless, no initialisation, reusable for any shape it is
 * large enough for. */
size_t spec_draft_workspace_bytes(int32_t B, int32_t K, int32_t V);

/* Enqueue the draft sampling (two kernels). */
int spec_draft_sample_launch(const spec_draft_args* args, hipStream_t stream);

/* ---------------------------------------------------- vocab-sharded verify
 *
 * The verification of spec_verify_launch (same method, same uniforms, K
 * drafts for every request, one pass) with the vocabulary split over G
 * shards, each holding only its slice [v0, v0 + Vs) of every target and draft
 * row -- as a tensor-parallel target holds its logits (the MineDraft reading
 * notes verify with TP = 4).  Each quantity the method needs is a sum or a
 * maximum over the vocabulary, so shards exchange reductions, never logits:
 *   1. spec_shard_stats_launch on every shard writes its slot g of `records`;
 *      then every shard needs all G slots (an all-gather of
 *      G * B * (2K+1) * 32 bytes);
 *   2. spec_shard_decide_launch on every shard merges the records in shard
 *      order -- every shard takes the same decisions and writes the same
 *      accepted_counts and output_tokens, except the sampled token, left -1
 *      -- and writes its slot g of `masses` (its slice's residual and p
 *      masses); then every shard needs all G slots (all-gather of G * B * 16
 *      bytes);
 *   3. spec_shard_draw_launch on every shard: the shard whose slice holds the
 *      inverse-CDF crossing writes the sampled token (a global id) into its
 *      output_tokens; the others leave -1, so an element-wise maximum over
 *      the shards' output_tokens (the third exchange) completes them.
 * On one GPU the exchanges are the shared `records` and `masses` arrays.
 * Results equal spec_verify_launch's up to the order of the floating-point
 * merges (a decision may differ only within rounding of its threshold).
 * Invalid data is reported as by spec_verify_launch (the draft tokens are
 * global ids in [0, V)).
 *
 * Ragged draft counts (num_drafts), a draft row table (draft_row_index into
 * a buffer of draft rows, each shard holding its slice of them) and early
 * exit (phase_starts) mean what they mean for spec_verify_launch.  With
 * phase_starts != 0 the positions 0..K are cut into phases p = 0, 1, ...
 * at its set bits, and step 1 becomes, for each phase p in order: every
 * shard runs spec_shard_stats_launch with args->phase = p (records of that
 * phase's rows, only for requests still alive), the records are exchanged,
 * and -- unless p is the last phase -- every shard runs
 * spec_shard_phase_launch with args->phase = p (that phase's accept tests;
 * each shard keeps the same per-request state in its workspace).  Steps 2
 * and 3 follow as above.  The outputs are identical to the one-pass sharded
 * verification (phase_starts = 0, one statistics launch with phase 0); a row
 * of a phase after the one where a request stopped is never read.
 */
typedef struct {
  int32_t B, K, V;             /* requests, drafts (1..SPEC_MAX_K), full vocabulary (1..SPEC_MAX_V) */
  int32_t dtype;               /* spec_dtype */
  int32_t G, g;                /* shards, and this shard (0 <= g < G) */
  int32_t v0, Vs;              /* this shard's slice of the vocabulary: [v0, v0 + Vs), Vs >= 1 */
  const void* target_logits;   /* device: element (b, r, j) = target logit of token v0 + j at row r */
  int64_t t_req_stride, t_row_stride;  /* elements; row stride >= Vs; request stride 0 = shared */
  const void* draft_logits;    /* device: the same for the draft rows 0..K-1 */
  int64_t d_req_stride, d_row_stride;
  const int32_t* draft_tokens; /* device [B, K], global token ids */
  const float* temperature;    /* device [B] */
  uint64_t seed;
  uint32_t step, request_base;
  void* records;               /* device [G, B, 2K+1] records of 32 bytes (slot g written by stats) */
  double* masses;              /* device [G, B, 2] (slot g written by decide) */
  int32_t* accepted_counts;    /* device out [B] */
  int32_t* output_tokens;      /* device out [B, K+1] */
  void* workspace;             /* device, >= spec_shard_workspace_bytes(B, K, Vs), 16-byte aligned; the
                                  same workspace must serve every stage of one shard */
  size_t workspace_bytes;
  const int32_t* num_drafts;   /* device [B] or NULL: ragged draft counts K_b in [0, K] */
  const int32_t* draft_row_index; /* device [B, K] or NULL: draft row k of request b is row
                                  draft_row_index[b*K + k] of a [draft_rows, Vs] slice buffer at
                                  draft_logits (row stride d_row_stride; d_req_stride unused) */
  int32_t draft_rows;          /* rows of that buffer (entries outside [0, draft_rows) make a
                                  sampled request invalid) */
  uint64_t phase_starts;       /* early exit: bit k (1 <= k <= K) starts a phase at position k; 0 = one pass */
  int32_t phase;               /* the phase a statistics or phase-decision launch covers, 0-based */
} spec_shard_args;

size_t spec_shard_workspace_bytes(int32_t B, int32_t K, int32_t Vs);
int spec_shard_stats_launch(const spec_shard_args* args, hipStream_t stream);
/* The accept tests of phase args->phase (not the last phase) from every
 * shard's records of its rows: updates this shard's per-request state. */
int spec_shard_phase_launch(const spec_shard_args* args, hipStream_t stream);
int spec_shard_decide_launch(const spec_shard_args* args, hipStream_t stream);
int spec_shard_draw_launch(const spec_shard_args* args, hipStream_t stream);

/* Human-readable name of a spec_status value (static storage). */
const char* spec_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_VERIFY_H */
