// verify_kernels.hpp -- kernel parameter blocks and launchers behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "spec_verify.h"
#include "verify_layout.hpp"

namespace specv {

struct ExpandParams {
  int32_t B, K, H, N_in, G, mask_id;
  const int32_t* ids;
  const int64_t* pos;
  const int32_t* in_start;
  const int32_t* acc;
  const int32_t* bonus;
  const int32_t* vtok;  // verification output tokens [B, K+1] (bonus source) or null
  const uint16_t* th;
  int64_t th_stride;
  const uint16_t* mh;
  int32_t* out_ids;
  int64_t* out_pos;
  uint8_t* rej;
  uint8_t* msk;
  int32_t* nti;
  int32_t* hmap;
  int32_t* out_start;
  uint16_t* out_h;
  const int32_t* bt;  // block table (slot mapping) or null
  int64_t bt_stride;
  int32_t max_blocks, block_size;
  int64_t* slots;     // slot mapping out, or null
  int32_t hidden_only;  // gather the hidden rows only (no metadata, accepted counts unread)
  int32_t vec;          // 16-byte hidden-row copies (H % 8 == 0 and aligned rows)
};

struct VerifyParams {
  int32_t B, K, V, R, C1, chunk1, nseg;
  const char* target;
  int64_t t_req, t_row;
  const char* draft;
  int64_t d_req, d_row;
  const int32_t* dridx;  // draft row table [B, K] (rows of a [draft_rows, V] buffer) or null
  int32_t draft_rows;
  const int32_t* num_drafts;  // ragged draft counts [B] or null (all K)
  const RowPartial* dstats;   // draft row statistics [B, K] from the draft sampler, or null
  const int32_t* tokens;
  const float* temperature;
  uint64_t seed;
  uint32_t step, request_base;
  int32_t* accepted;
  int32_t* out_tokens;
  float* debug;
  RowPartial* rowp;
  ReqDesc* desc;
  double* seg;
  int32_t* err;    // count of invalid requests of this verification
  int32_t* state;  // per-request state between early-exit phases
  // rows of one early-exit phase: target rows [ph_lo, ph_lo + ph_nt), draft
  // rows [ph_lo, ph_lo + ph_nd), of which the row pass reads the first ph_rd
  // (none with draft statistics); ph_check: skip requests no longer alive
  int32_t ph_lo, ph_nt, ph_nd, ph_rd, ph_check;
  // start of the last phase when the rows were read in several phases, else 0
  int32_t last_lo, phased;
  // dynamic early exit (dyn): decisions taken inside the row pass as its
  // chunks finish.  epoch: the launch counter, which with salt (from the
  // workspace's address) gives the launch's tag E that its tagged records and
  // state words carry; dstate [B]: per request (E << 8) | (2 n + f),
  // positions before n known accepted and, with f, position n stops the
  // request; trec: tagged copies of rowp; dyn_shift: request groups between a
  // request's chunks of a position and its decider slot
  uint64_t* epoch;
  uint64_t salt;
  uint64_t* dstate;
  TaggedPartial* trec;
  int32_t dyn, dyn_shift;
  // a chained expansion of this verification's outputs, folded into its
  // sampling stage (ex_on): ex_G workgroups per request window
  ExpandParams ex;
  int32_t ex_on, ex_G;
};


// Decider slots of the dynamic early exit: a request's slot comes
// kDynShiftNum / kDynShiftDen of a position's request groups after its chunks
// of that position (late enough that most of the chunks have finished, early
// enough that the decision lands before its chunks of the next position).
constexpr int64_t kDynShiftNum = 3, kDynShiftDen = 10;

struct DraftParams {
  int32_t B, K, V, N, nseg, C;  // C: chunks of kDraftChunkSegs segments per row
  const char* logits;
  int64_t row_stride;
  const int32_t* row_index;
  const float* temperature;
  uint64_t seed;
  uint32_t step, request_base;
  int32_t* tokens;
  RowPartial* segp;  // per (request, position, segment) statistics [B * K * nseg]
  RowPartial* stats; // per (request, position): the row's normaliser and the drawn logit, or null
};

constexpr int kDraftChunkSegs = 8;  // segments per workgroup of the statistics pass

// Vocab-sharded verification: one shard's statistics of one row of its vocab
// slice (exchanged between shards).
struct ShardRec {
  float m;        // integer-valued reference (sampled) or max logit (greedy)
  int32_t idx;    // argmax as a global token id (greedy)
  double s;       // sum of 2^(x * s - m) over the slice (sampled)
  float z;        // logit at the position's draft token, when the slice holds it
  int32_t has_z;
  int64_t pad;
};
static_assert(sizeof(ShardRec) == 32, "ShardRec layout");

struct ShardParams {
  int32_t B, K, V, R, G, g, v0, Vs, nseg;  // nseg: 4096-logit segments of the slice
  const char* target;
  int64_t t_req, t_row;
  const char* draft;
  int64_t d_req, d_row;
  const int32_t* tokens;
  const float* temperature;
  uint64_t seed;
  uint32_t step, request_base;
  ShardRec* recs;    // [G, B, R]
  double* masses;    // [G, B, 2]: residual and p masses of each shard's slice
  int32_t* accepted;
  int32_t* out_tokens;
  ReqDesc* desc;     // [B] (this shard's workspace)
  double* seg;       // [B, nseg, 2] (this shard's workspace)
  int32_t* state;    // [B] request state between early-exit phases (this shard's workspace)
  const int32_t* dridx;       // draft row table [B, K] (rows of a [draft_rows, Vs] slice buffer) or null
  int32_t draft_rows;
  const int32_t* num_drafts;  // ragged draft counts [B] or null (all K)
  // rows of the phase a statistics or phase-decision launch covers: target
  // rows [ph_lo, ph_lo + ph_nt), draft rows [ph_lo, ph_lo + ph_nd); ph_check:
  // a later phase (skip requests no longer alive)
  int32_t ph_lo, ph_nt, ph_nd, ph_check;
  // the final decision: rows were read in phases (phased), the last phase
  // starting at position last_lo
  int32_t phased, last_lo;
};

hipError_t launch_shard_stats(const ShardParams& P, int dtype, bool vec, hipStream_t stream);
hipError_t launch_shard_phase(const ShardParams& P, int dtype, bool vec, hipStream_t stream);
hipError_t launch_shard_decide(const ShardParams& P, int dtype, bool vec, hipStream_t stream);
hipError_t launch_shard_draw(const ShardParams& P, int dtype, bool vec, hipStream_t stream);

// phase_starts: bit k (1 <= k <= K) starts an early-exit phase at draft
// position k; 0 reads every row in one pass.
hipError_t launch_verify(const VerifyParams& P, int dtype, bool vec, uint64_t phase_starts,
                         hipEvent_t phase_event, hipStream_t stream);
// Whether every kernel grid of a verification of this shape fits one dispatch
// (2^32 work-items); ex_items: the workgroups of a chained expansion.
bool verify_grids_fit(int32_t B, int32_t K, int32_t C1, int32_t nseg, bool dyn, bool dstats, int64_t ex_items);
hipError_t launch_expand(const ExpandParams& P, bool vec, hipStream_t stream);
hipError_t launch_draft(const DraftParams& P, int dtype, bool vec, hipStream_t stream);

}  // namespace specv
