// api.hip -- the C ABI: host-side argument validation, workspace sizing and
// kernel launches.  Every check here runs before anything is enqueued, and no
// launch entry point synchronises the stream or allocates memory (the host
// query spec_workspace_error waits for the stream it is given).
#include <stdint.h>

#include <mutex>

#include "spec_verify.h"
#include "verify_kernels.hpp"
#include "verify_layout.hpp"

using namespace specv;

// The workspace of spec_verify_launch_noalloc: one copy of this array per GPU
// the library runs on, held until the process ends.  Host code never passes
// its name to a kernel (on the host it is only a stand-in for the symbol): it
// uses the device address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kExpandRowsPerWG = 4;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Device address of `scratch` per device, looked up on the first call made
// with that device current (a lookup, not an allocation).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

int scratch_address(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_ELAUNCH;
  if (stream != nullptr) {  // the lookup is for the current device: the stream must be on it
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return SPEC_ELAUNCH;
    if (sdev != dev) return SPEC_EINVAL;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return SPEC_ELAUNCH;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return SPEC_OK;
}

// Whether a grid of `blocks` workgroups of `threads` fits one dispatch
// (2^32 work-items).
static bool fits_dispatch(int64_t blocks, int64_t threads) { return blocks * threads <= (int64_t)UINT32_MAX; }

int verify_check(const spec_verify_args* a) {
  if (!a) return SPEC_EINVAL;
  if (a->B < 0 || a->K < 1 || a->K > SPEC_MAX_K || a->V < 1 || a->V > SPEC_MAX_V) return SPEC_EINVAL;
  if (a->dtype != SPEC_F32 && a->dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (a->B == 0) return SPEC_OK;
  if (!a->target_logits || !a->draft_logits || !a->draft_tokens || !a->temperature ||
      !a->accepted_counts || !a->output_tokens || !a->workspace)
    return SPEC_EINVAL;
  if (a->t_row_stride < a->V || a->d_row_stride < a->V) return SPEC_EINVAL;
  if (a->t_req_stride != 0 && a->t_req_stride < (int64_t)(a->K + 1) * a->t_row_stride) return SPEC_EINVAL;
  if (!a->draft_row_index && a->d_req_stride != 0 && a->d_req_stride < (int64_t)a->K * a->d_row_stride)
    return SPEC_EINVAL;
  if (a->draft_row_index && a->draft_rows < 0) return SPEC_EINVAL;
  const Layout L = make_layout(a->B, a->K, a->V);
  if ((int64_t)a->B * L.R * L.C1 > INT32_MAX || (int64_t)a->B * L.nseg > INT32_MAX) return SPEC_EINVAL;
  if (!aligned16(a->workspace) || (a->draft_stats && !aligned16(a->draft_stats))) return SPEC_EALIGN;
  // position 0 always starts the first phase; bit 0 alone: dynamic early exit
  if ((a->phase_starts & 1u) && a->phase_starts != SPEC_PHASES_DYNAMIC) return SPEC_EINVAL;
  if (a->K < 63 && (a->phase_starts >> (a->K + 1)) != 0) return SPEC_EINVAL;
  if ((int64_t)a->B * (L.R * L.C1 + a->K + 1) > INT32_MAX) return SPEC_EINVAL;  // the dynamic pass's grid
  if (!verify_grids_fit(a->B, a->K, L.C1, L.nseg, a->phase_starts == SPEC_PHASES_DYNAMIC, a->draft_stats != nullptr,
                        0))
    return SPEC_EINVAL;
  if (a->workspace_bytes < L.total) return SPEC_EWORKSPACE;
  return SPEC_OK;
}

int expand_check(const spec_expand_args* a) {
  if (!a) return SPEC_EINVAL;
  if (a->B < 0 || a->K < 1 || a->H < 0 || a->N_in < 0) return SPEC_EINVAL;
  if ((int64_t)a->N_in + (int64_t)a->B * (a->K - 1) > INT32_MAX) return SPEC_EINVAL;
  if (a->B == 0) return SPEC_OK;
  if (!fits_dispatch(a->B, 256)) return SPEC_EINVAL;  // one 256-thread workgroup per request at least
  if (!a->bonus_tokens == !a->verify_output_tokens) return SPEC_EINVAL;  // exactly one bonus source
  if (!a->in_start || !a->accepted_counts || !a->out_token_ids ||
      !a->out_positions || !a->rejected_mask || !a->masked_mask || !a->new_token_indices || !a->out_start)
    return SPEC_EINVAL;
  if (a->N_in > 0 && (!a->in_token_ids || !a->in_positions || !a->hidden_map)) return SPEC_EINVAL;
  if (a->out_hidden) {
    if (a->H > 0 && (!a->mask_hidden || (a->N_in > 0 && !a->target_hidden))) return SPEC_EINVAL;
    if (a->hidden_row_stride < a->H) return SPEC_EINVAL;
  }
  if (a->slot_mapping) {
    if (a->block_size < 1 || a->max_blocks < 0 || a->bt_row_stride < a->max_blocks) return SPEC_EINVAL;
    if (a->max_blocks > 0 && !a->block_table) return SPEC_EINVAL;
  }
  return SPEC_OK;
}

size_t draft_ws_bytes(int32_t B, int32_t K, int32_t V) {
  const int64_t nseg = ((int64_t)V + kSeg - 1) / kSeg;
  return align256((size_t)B * K * nseg * sizeof(RowPartial));
}

int draft_check(const spec_draft_args* a) {
  if (!a) return SPEC_EINVAL;
  if (a->B < 0 || a->K < 1 || a->V < 1 || a->V > SPEC_MAX_V || a->N < 0) return SPEC_EINVAL;
  if (a->dtype != SPEC_F32 && a->dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (a->B == 0) return SPEC_OK;
  if (!a->row_index || !a->temperature || !a->tokens || !a->workspace) return SPEC_EINVAL;
  if (a->N > 0 && !a->logits) return SPEC_EINVAL;
  if (a->row_stride < a->V) return SPEC_EINVAL;
  const int64_t nseg = ((int64_t)a->V + kSeg - 1) / kSeg;
  const int64_t C = (nseg + kDraftChunkSegs - 1) / kDraftChunkSegs;
  if ((int64_t)a->B * a->K * C > INT32_MAX) return SPEC_EINVAL;
  if (!fits_dispatch((int64_t)a->B * a->K * C, 256) || !fits_dispatch((int64_t)a->B * a->K, 64)) return SPEC_EINVAL;
  if (!aligned16(a->workspace) || (a->stats_out && !aligned16(a->stats_out))) return SPEC_EALIGN;
  if (a->workspace_bytes < draft_ws_bytes(a->B, a->K, a->V)) return SPEC_EWORKSPACE;
  return SPEC_OK;
}

size_t shard_ws_bytes(int32_t B, int32_t Vs) {
  const int64_t nseg = ((int64_t)Vs + kSeg - 1) / kSeg;
  return align256((size_t)B * sizeof(ReqDesc)) + align256((size_t)B * nseg * 2 * sizeof(double)) +
         align256((size_t)B * sizeof(int32_t));
}

// Phase p of a cut (bit k of `starts` starts a phase at position k; 0 = one
// phase): positions [lo, hi) with hi = K + 1 for the last; the number of
// phases and the start of the last.
struct PhaseRange {
  int lo, hi, count, last_lo;
};

PhaseRange phase_range(uint64_t starts, int K, int p) {
  PhaseRange r{0, K + 1, 0, 0};
  int lo = 0;
  for (int j = 0; lo <= K; ++j) {
    int hi = lo + 1;
    while (hi <= K && !((starts >> hi) & 1u)) ++hi;
    if (j == p) {
      r.lo = lo;
      r.hi = hi;
    }
    r.count = j + 1;
    r.last_lo = lo;
    lo = hi;
  }
  return r;
}

int shard_check(const spec_shard_args* a) {
  if (!a) return SPEC_EINVAL;
  if (a->B < 0 || a->K < 1 || a->K > SPEC_MAX_K || a->V < 1 || a->V > SPEC_MAX_V) return SPEC_EINVAL;
  if (a->dtype != SPEC_F32 && a->dtype != SPEC_BF16) return SPEC_EDTYPE;
  if (a->G < 1 || a->g < 0 || a->g >= a->G) return SPEC_EINVAL;
  if (a->Vs < 1 || a->v0 < 0 || (int64_t)a->v0 + a->Vs > a->V) return SPEC_EINVAL;
  if (a->B == 0) return SPEC_OK;
  if (!a->target_logits || !a->draft_logits || !a->draft_tokens || !a->temperature || !a->records ||
      !a->masses || !a->accepted_counts || !a->output_tokens || !a->workspace)
    return SPEC_EINVAL;
  if (a->t_row_stride < a->Vs || a->d_row_stride < a->Vs) return SPEC_EINVAL;
  if (a->t_req_stride != 0 && a->t_req_stride < (int64_t)(a->K + 1) * a->t_row_stride) return SPEC_EINVAL;
  if (!a->draft_row_index && a->d_req_stride != 0 && a->d_req_stride < (int64_t)a->K * a->d_row_stride)
    return SPEC_EINVAL;
  if (a->draft_row_index && a->draft_rows < 0) return SPEC_EINVAL;
  if ((int64_t)a->B * (2 * a->K + 1) > INT32_MAX) return SPEC_EINVAL;
  if (!fits_dispatch((int64_t)a->B * (2 * a->K + 1), 256) || !fits_dispatch(a->B, 1024)) return SPEC_EINVAL;
  if (a->phase_starts & 1u) return SPEC_EINVAL;  // position 0 always starts the first phase
  if (a->K < 63 && (a->phase_starts >> (a->K + 1)) != 0) return SPEC_EINVAL;
  if (a->phase < 0 || a->phase >= phase_range(a->phase_starts, a->K, 0).count) return SPEC_EINVAL;
  if (!aligned16(a->workspace)) return SPEC_EALIGN;
  if (a->workspace_bytes < shard_ws_bytes(a->B, a->Vs)) return SPEC_EWORKSPACE;
  return SPEC_OK;
}

ShardParams shard_params(const spec_shard_args* a) {
  ShardParams P;
  P.B = a->B;
  P.K = a->K;
  P.V = a->V;
  P.R = 2 * a->K + 1;
  P.G = a->G;
  P.g = a->g;
  P.v0 = a->v0;
  P.Vs = a->Vs;
  P.nseg = (int32_t)(((int64_t)a->Vs + kSeg - 1) / kSeg);
  P.target = static_cast<const char*>(a->target_logits);
  P.t_req = a->t_req_stride;
  P.t_row = a->t_row_stride;
  P.draft = static_cast<const char*>(a->draft_logits);
  P.d_req = a->d_req_stride;
  P.d_row = a->d_row_stride;
  P.tokens = a->draft_tokens;
  P.temperature = a->temperature;
  P.seed = a->seed;
  P.step = a->step;
  P.request_base = a->request_base;
  P.recs = static_cast<ShardRec*>(a->records);
  P.masses = a->masses;
  P.accepted = a->accepted_counts;
  P.out_tokens = a->output_tokens;
  char* ws = static_cast<char*>(a->workspace);
  P.desc = reinterpret_cast<ReqDesc*>(ws);
  const size_t off_seg = align256((size_t)a->B * sizeof(ReqDesc));
  P.seg = reinterpret_cast<double*>(ws + off_seg);
  P.state = reinterpret_cast<int32_t*>(ws + off_seg + align256((size_t)a->B * P.nseg * 2 * sizeof(double)));
  P.dridx = a->draft_row_index;
  P.draft_rows = a->draft_row_index ? a->draft_rows : 0;
  P.num_drafts = a->num_drafts;
  const PhaseRange ph = phase_range(a->phase_starts, a->K, a->phase);
  P.ph_lo = ph.lo;
  P.ph_nt = ph.hi - ph.lo;
  P.ph_nd = (ph.hi < a->K ? ph.hi : a->K) - ph.lo;
  P.ph_check = a->phase > 0;
  P.phased = ph.count > 1;
  P.last_lo = ph.last_lo;
  return P;
}

bool shard_vec(const spec_shard_args* a) {
  const int es = a->dtype == SPEC_BF16 ? 2 : 4;
  return aligned16(a->target_logits) && aligned16(a->draft_logits) && (a->t_row_stride * es) % 16 == 0 &&
         (a->t_req_stride * es) % 16 == 0 && (a->d_row_stride * es) % 16 == 0 &&
         (a->draft_row_index || (a->d_req_stride * es) % 16 == 0);
}

}  // namespace

extern "C" {

size_t spec_shard_workspace_bytes(int32_t B, int32_t K, int32_t Vs) {
  if (B < 0 || K < 1 || K > SPEC_MAX_K || Vs < 1 || Vs > SPEC_MAX_V) return 0;
  return shard_ws_bytes(B, Vs);
}

int spec_shard_stats_launch(const spec_shard_args* a, hipStream_t stream) {
  const int rc = shard_check(a);
  if (rc != SPEC_OK || a->B == 0) return rc;
  return launch_shard_stats(shard_params(a), a->dtype, shard_vec(a), stream) == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

int spec_shard_phase_launch(const spec_shard_args* a, hipStream_t stream) {
  if (!a || a->K < 1 || a->K > SPEC_MAX_K) return SPEC_EINVAL;
  if (a->phase >= phase_range(a->phase_starts, a->K, 0).count - 1) return SPEC_EINVAL;  // not the last phase
  const int rc = shard_check(a);
  if (rc != SPEC_OK) return rc;
  if (a->B == 0) return SPEC_OK;
  return launch_shard_phase(shard_params(a), a->dtype, shard_vec(a), stream) == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

int spec_shard_decide_launch(const spec_shard_args* a, hipStream_t stream) {
  const int rc = shard_check(a);
  if (rc != SPEC_OK || a->B == 0) return rc;
  return launch_shard_decide(shard_params(a), a->dtype, shard_vec(a), stream) == hipSuccess ? SPEC_OK
                                                                                            : SPEC_ELAUNCH;
}

int spec_shard_draw_launch(const spec_shard_args* a, hipStream_t stream) {
  const int rc = shard_check(a);
  if (rc != SPEC_OK || a->B == 0) return rc;
  return launch_shard_draw(shard_params(a), a->dtype, shard_vec(a), stream) == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

size_t spec_draft_workspace_bytes(int32_t B, int32_t K, int32_t V) {
  if (B < 0 || K < 1 || V < 1 || V > SPEC_MAX_V) return 0;
  return draft_ws_bytes(B, K, V);
}

int spec_draft_sample_launch(const spec_draft_args* a, hipStream_t stream) {
  const int rc = draft_check(a);
  if (rc != SPEC_OK || a->B == 0) return rc;
  const int es = a->dtype == SPEC_BF16 ? 2 : 4;
  DraftParams P;
  P.B = a->B;
  P.K = a->K;
  P.V = a->V;
  P.N = a->N;
  P.nseg = (int32_t)(((int64_t)a->V + kSeg - 1) / kSeg);
  P.C = (P.nseg + kDraftChunkSegs - 1) / kDraftChunkSegs;
  P.logits = static_cast<const char*>(a->logits);
  P.row_stride = a->row_stride;
  P.row_index = a->row_index;
  P.temperature = a->temperature;
  P.seed = a->seed;
  P.step = a->step;
  P.request_base = a->request_base;
  P.tokens = a->tokens;
  P.segp = static_cast<RowPartial*>(a->workspace);
  P.stats = static_cast<RowPartial*>(a->stats_out);
  const bool vec = aligned16(a->logits) && (a->row_stride * es) % 16 == 0;
  return launch_draft(P, a->dtype, vec, stream) == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

uint64_t spec_verify_plan_phases(int32_t K, const double* survival, double sampled_fraction, double phase_cost) {
  if (K < 1 || K > SPEC_MAX_K || !survival) return 0;
  if (!(sampled_fraction >= 0.0 && sampled_fraction <= 1.0) || !(phase_cost >= 0.0 && phase_cost < 1e300)) return 0;
  for (int k = 0; k <= K; ++k)
    if (!(survival[k] >= 0.0 && survival[k] <= 1.0)) return 0;
  // best[s]: least expected cost of positions s..K when a phase starts at s
  double best[SPEC_MAX_K + 2];
  int next[SPEC_MAX_K + 2];
  best[K + 1] = 0.0;
  for (int s = K; s >= 0; --s) {
    best[s] = -1.0;
    for (int e = K + 1; e > s; --e) {
      const double rows = (double)(e - s) + sampled_fraction * (double)((e < K ? e : K) - s);
      const double c = survival[s] * rows + (e <= K ? phase_cost : 0.0) + best[e];
      if (best[s] < 0.0 || c < best[s]) {  // ties keep the longer phase, found first
        best[s] = c;
        next[s] = e;
      }
    }
  }
  uint64_t mask = 0;
  for (int s = next[0]; s <= K; s = next[s]) mask |= (uint64_t)1 << s;
  return mask;
}

double spec_verify_phase_cost(int32_t B, int32_t K, int32_t V, int32_t dtype) {
  if (B < 1 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return -1.0;
  if (dtype != SPEC_F32 && dtype != SPEC_BF16) return -1.0;
  // measured on MI355X (see the header): the boundary's fixed cost, the extra
  // when a phase's rows cannot fill the chip, the slots of the row pass
  // (256 compute units x 5 resident 256-thread workgroups) and its rate
  constexpr double kBoundaryUs = 12.0, kUnderfillUs = 7.7, kSlots = 256.0 * 5.0, kRowBytesPerUs = 6.8e6;
  const Layout L = make_layout(1, K, V);
  const double per_row_unit = (double)B * (double)L.C1;  // workgroups reading one row of every request
  const double fill = per_row_unit < kSlots ? 1.0 - per_row_unit / kSlots : 0.0;
  const double boundary_us = kBoundaryUs + kUnderfillUs * fill;
  const double row_us = (double)B * (double)V * (dtype == SPEC_BF16 ? 2.0 : 4.0) / kRowBytesPerUs;
  return boundary_us / row_us;
}

size_t spec_verify_workspace_bytes(int32_t B, int32_t K, int32_t V) {
  if (B < 0 || K < 1 || K > SPEC_MAX_K || V < 1 || V > SPEC_MAX_V) return 0;
  return make_layout(B, K, V).total;
}

// The kernel parameters of a checked verification (B >= 1); vec: 16-byte
// row loads are possible.
static VerifyParams verify_params(const spec_verify_args* a, bool& vec) {
  const Layout L = make_layout(a->B, a->K, a->V);
  const int es = a->dtype == SPEC_BF16 ? 2 : 4;
  VerifyParams P;
  P.B = a->B;
  P.K = a->K;
  P.V = a->V;
  P.R = L.R;
  P.C1 = L.C1;
  P.chunk1 = L.chunk1;
  P.nseg = L.nseg;
  P.target = static_cast<const char*>(a->target_logits);
  P.t_req = a->t_req_stride;
  P.t_row = a->t_row_stride;
  P.draft = static_cast<const char*>(a->draft_logits);
  P.d_req = a->d_req_stride;
  P.d_row = a->d_row_stride;
  P.dridx = a->draft_row_index;
  P.num_drafts = a->num_drafts;
  P.dstats = static_cast<const RowPartial*>(a->draft_stats);
  P.draft_rows = a->draft_row_index ? a->draft_rows : 0;
  P.tokens = a->draft_tokens;
  P.temperature = a->temperature;
  P.seed = a->seed;
  P.step = a->step;
  P.request_base = a->request_base;
  P.accepted = a->accepted_counts;
  P.out_tokens = a->output_tokens;
  P.debug = a->debug_probs;
  char* ws = static_cast<char*>(a->workspace);
  P.rowp = reinterpret_cast<RowPartial*>(ws + L.off_rowp);
  P.desc = reinterpret_cast<ReqDesc*>(ws + L.off_desc);
  P.seg = reinterpret_cast<double*>(ws + L.off_seg);
  vec = aligned16(a->target_logits) && aligned16(a->draft_logits) && (a->t_row_stride * es) % 16 == 0 &&
        (a->t_req_stride * es) % 16 == 0 && (a->d_row_stride * es) % 16 == 0 &&
        (a->draft_row_index || (a->d_req_stride * es) % 16 == 0);
  P.err = reinterpret_cast<int32_t*>(ws + L.off_err);
  P.state = reinterpret_cast<int32_t*>(ws + L.off_state);
  P.epoch = reinterpret_cast<uint64_t*>(ws + L.off_epoch);
  // a workspace's launches are tagged by its counter plus this salt (an odd
  // multiple of the address: different workspaces, different salts)
  P.salt = (uint64_t)(uintptr_t)a->workspace * 0x9E3779B97F4A7C15ull;
  P.dstate = reinterpret_cast<uint64_t*>(ws + L.off_dstate);
  P.trec = reinterpret_cast<TaggedPartial*>(ws + L.off_trec);
  P.dyn = a->phase_starts == SPEC_PHASES_DYNAMIC;
  // a request's decider slot sits this many request groups after its chunks
  P.dyn_shift = (int32_t)min((int64_t)a->B - 1, (int64_t)a->B * kDynShiftNum / kDynShiftDen);
  P.ph_lo = P.ph_nt = P.ph_nd = P.ph_rd = P.ph_check = 0;
  P.last_lo = P.phased = 0;
  P.ex_on = 0;
  P.ex_G = 1;
  return P;
}

static int verify_enqueue(const VerifyParams& P, const spec_verify_args* a, bool vec, hipStream_t stream) {
  return launch_verify(P, a->dtype, vec, a->phase_starts, static_cast<hipEvent_t>(a->phase_event), stream) ==
                 hipSuccess
             ? SPEC_OK
             : SPEC_ELAUNCH;
}

int spec_verify_launch(const spec_verify_args* a, hipStream_t stream) {
  const int rc = verify_check(a);
  if (rc != SPEC_OK || a->B == 0) return rc;
  bool vec;
  const VerifyParams P = verify_params(a, vec);
  return verify_enqueue(P, a, vec, stream);
}

int spec_verify_launch_noalloc(const spec_verify_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  if (a->B < 0 || a->K < 1 || a->K > SPEC_MAX_K || a->V < 1 || a->V > SPEC_MAX_V) return SPEC_EINVAL;
  if (a->B == 0) return verify_check(a);  // nothing to enqueue (a bad dtype is still reported)
  if (make_layout(a->B, a->K, a->V).total > (size_t)SPEC_NOALLOC_SCRATCH_BYTES) return SPEC_EWORKSPACE;
  void* ws = nullptr;
  const int rs = scratch_address(stream, &ws);
  if (rs != SPEC_OK) return rs;
  // the same checks and kernels as spec_verify_launch, with this device's
  // scratch array as the workspace
  spec_verify_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = SPEC_NOALLOC_SCRATCH_BYTES;
  const int rc = verify_check(&b);
  if (rc != SPEC_OK) return rc;
  bool vec;
  const VerifyParams P = verify_params(&b, vec);
  return verify_enqueue(P, &b, vec, stream);
}

// The kernel parameters of a checked expansion (B >= 1), G workgroups per
// request window.
static ExpandParams expand_params(const spec_expand_args* a, bool hidden_only, int64_t rows_per_wg) {
  ExpandParams P;
  P.hidden_only = hidden_only ? 1 : 0;
  P.B = a->B;
  P.K = a->K;
  P.H = a->H;
  P.N_in = a->N_in;
  P.mask_id = a->mask_token_id;
  // about rows_per_wg output rows per workgroup on average; a request's
  // window is shared by G workgroups row-interleaved
  const int64_t n_out = (int64_t)a->N_in + (int64_t)a->B * (a->K - 1);
  const int64_t avg_window = (n_out + a->B - 1) / a->B;
  int64_t G = (avg_window + rows_per_wg - 1) / rows_per_wg;
  if (G < 1) G = 1;
  if (G > 64) G = 64;
  if ((int64_t)a->B * G > INT32_MAX || !fits_dispatch((int64_t)a->B * G, 256)) G = 1;
  P.G = (int32_t)G;
  P.ids = a->in_token_ids;
  P.pos = a->in_positions;
  P.in_start = a->in_start;
  P.acc = a->accepted_counts;
  P.bonus = a->bonus_tokens;
  P.vtok = a->verify_output_tokens;
  P.th = a->target_hidden;
  P.th_stride = a->hidden_row_stride;
  P.mh = a->mask_hidden;
  P.out_ids = a->out_token_ids;
  P.out_pos = a->out_positions;
  P.rej = a->rejected_mask;
  P.msk = a->masked_mask;
  P.nti = a->new_token_indices;
  P.hmap = a->hidden_map;
  P.out_start = a->out_start;
  P.out_h = (a->H > 0) ? a->out_hidden : nullptr;
  P.slots = a->slot_mapping;
  P.bt = a->block_table;
  P.bt_stride = a->bt_row_stride;
  P.max_blocks = a->slot_mapping ? a->max_blocks : 0;
  P.block_size = a->slot_mapping ? a->block_size : 1;
  P.vec = (a->H % 8) == 0 && (a->hidden_row_stride % 8) == 0 && aligned16(a->target_hidden) &&
          aligned16(a->mask_hidden) && aligned16(a->out_hidden);
  return P;
}

static int expand_launch(const spec_expand_args* a, bool hidden_only, hipStream_t stream) {
  const ExpandParams P = expand_params(a, hidden_only, kExpandRowsPerWG);
  return launch_expand(P, P.vec != 0, stream) == hipSuccess ? SPEC_OK : SPEC_ELAUNCH;
}

int spec_expand_launch(const spec_expand_args* a, hipStream_t stream) {
  const int rc = expand_check(a);
  if (rc != SPEC_OK || a->B == 0) return rc;
  return expand_launch(a, false, stream);
}

int spec_expand_hidden_launch(const spec_expand_args* a, hipStream_t stream) {
  if (!a) return SPEC_EINVAL;
  if (a->B < 0 || a->K < 1 || a->H < 0 || a->N_in < 0) return SPEC_EINVAL;
  if ((int64_t)a->N_in + (int64_t)a->B * (a->K - 1) > INT32_MAX) return SPEC_EINVAL;
  if (a->B == 0 || a->H == 0) return SPEC_OK;
  if (!a->in_start || !a->out_hidden || !a->mask_hidden || (a->N_in > 0 && !a->target_hidden))
    return SPEC_EINVAL;
  if (a->hidden_row_stride < a->H) return SPEC_EINVAL;
  return expand_launch(a, true, stream);
}

int spec_verify_expand_launch(const spec_verify_args* v, const spec_expand_args* e, hipStream_t stream) {
  int rc = verify_check(v);
  if (rc != SPEC_OK) return rc;
  rc = expand_check(e);
  if (rc != SPEC_OK) return rc;
  // the expansion reads this verification's outputs: same batch, the counts
  // and the bonus source are the verification's own output arrays
  if (e->B != v->B || e->K != v->K) return SPEC_EINVAL;
  if (v->B == 0) return SPEC_OK;
  if (e->accepted_counts != v->accepted_counts || e->verify_output_tokens != v->output_tokens) return SPEC_EINVAL;
  bool vec;
  VerifyParams P = verify_params(v, vec);
  P.ex = expand_params(e, false, 1);  // one output row per wave on average
  P.ex_on = 1;
  P.ex_G = P.ex.G;
  if ((int64_t)P.B * P.nseg + (int64_t)P.B * P.ex_G > INT32_MAX) return SPEC_EINVAL;
  if (!verify_grids_fit(P.B, P.K, P.C1, P.nseg, P.dyn != 0, P.dstats != nullptr, (int64_t)P.B * P.ex_G))
    return SPEC_EINVAL;
  return verify_enqueue(P, v, vec, stream);
}

int spec_workspace_error(const void* workspace, hipStream_t stream) {
  if (workspace == nullptr) return SPEC_EINVAL;
  if (hipStreamSynchronize(stream) != hipSuccess) return SPEC_ELAUNCH;
  int32_t n = 0;
  if (hipMemcpy(&n, workspace, sizeof(n), hipMemcpyDeviceToHost) != hipSuccess) return SPEC_ELAUNCH;
  return n;
}

const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_EINVAL: return "SPEC_EINVAL: invalid argument (null pointer, size or stride out of range)";
    case SPEC_EDTYPE: return "SPEC_EDTYPE: unknown logits dtype";
    case SPEC_EALIGN: return "SPEC_EALIGN: workspace or statistics records not 16-byte aligned";
    case SPEC_EWORKSPACE: return "SPEC_EWORKSPACE: workspace too small";
    case SPEC_ELAUNCH: return "SPEC_ELAUNCH: kernel launch failed";
    default: return "unknown spec_status";
  }
}

}  // extern "C"
