// verify_layout.hpp -- chunking of a vocabulary row and the layout of the
// verification workspace (host and device).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace specv {

// Segments: the sampling pass sums its weights over runs of kSeg consecutive
// logits, one run per wave64 (8 groups of 8 logits per lane), and the draw
// then searches a single segment.
constexpr int kSegGroups = 8;
constexpr int kSeg = 64 * 8 * kSegGroups;  // 4096 logits

// Row pass: one 256-thread workgroup streams ~32K logits of one row, long
// enough to hide its start-up, still thousands of workgroups per batch.
constexpr int kRowChunkTarget = 32768;

struct RowPartial {  // one chunk of one row
  float m;           // integer-valued reference exponent (sampled) or max logit (greedy)
  int32_t idx;       // argmax index (greedy); sampled rows of draft positions: the logit at
                     // the position's draft token as stored (bf16 bits zero-extended, or
                     // fp32 bits) if this chunk holds it, else 0
  double s;          // sum of 2^(x*s - m) over the chunk (sampled)
};

struct ReqDesc {  // decision of one request, read by the draw
  int32_t mode;   // kModeNone / kModeResidual / kModeBonus
  int32_t a;      // accepted drafts = the sampling row
  float s_hi, s_lo;
  double mp, sp;  // reference exponent and normaliser of p at row a
  double mq, sq;  // same for q (residual mode)
  double u;       // the sampling uniform of row a
  int64_t qoff;   // element offset of draft row a from the draft base (residual mode)
};

// A chunk's RowPartial as read by workgroups of the same row-pass launch
// (dynamic early exit): eight 64-bit words, each stored by one single-copy
// atomic store and each carrying a 48-bit tag of the launch in its high bits
// and 16 bits of the record in its low bits (words 0-3: m's bits, then idx,
// low half first; words 4-7: s's bits, lowest 16 first).  Every tag is odd,
// so that zeroed memory never carries one, and each word's differs for any
// two launches less than 2^47 apart.  A reader that finds the launch's tags
// in all eight words has the whole record of this launch; anything else (a
// record still being written, left by an earlier launch, or memory never
// written) it treats as not yet there.
struct TaggedPartial {
  uint64_t w[8];
};

static_assert(sizeof(RowPartial) == 16, "RowPartial layout");
static_assert(sizeof(TaggedPartial) == 64, "TaggedPartial layout");
static_assert(sizeof(ReqDesc) == 64, "ReqDesc layout");

enum { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };

// Request state between the phases of an early-exit verification: >= 0 the
// request stopped at that draft position, kStateInvalid its data is invalid,
// kStateAlive every accept test so far passed.
constexpr int32_t kStateInvalid = -1;
constexpr int32_t kStateAlive = -2;

struct Layout {
  int32_t R;           // rows per request the row pass may read: K+1 target + K draft
  int32_t C1, chunk1;  // row-pass chunks per row and their length
  int32_t nseg;        // segments per row
  // the invalid-request count sits at byte 0 of the workspace (read by
  // spec_workspace_error without knowing the shape), the launch counter of
  // the dynamic early exit at byte 8
  size_t off_err, off_epoch, off_rowp, off_desc, off_seg, off_state, off_dstate, off_trec, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Cut V into chunks of about `target` logits, each a multiple of kSeg.
__host__ __device__ inline void chunking(int32_t V, int32_t target, int32_t& C, int32_t& chunk) {
  int64_t n = ((int64_t)V + target - 1) / target;
  if (n < 1) n = 1;
  int64_t per = ((int64_t)V + n - 1) / n;
  per = (per + kSeg - 1) / kSeg * kSeg;
  chunk = (int32_t)per;
  C = (int32_t)(((int64_t)V + per - 1) / per);
}

__host__ __device__ inline Layout make_layout(int32_t B, int32_t K, int32_t V) {
  Layout L;
  L.R = 2 * K + 1;
  chunking(V, kRowChunkTarget, L.C1, L.chunk1);
  L.nseg = (int32_t)(((int64_t)V + kSeg - 1) / kSeg);
  size_t off = 0;
  L.off_err = off;
  L.off_epoch = off + 8;
  off = align256(off + 16);
  L.off_rowp = off;
  off = align256(off + (size_t)B * L.R * L.C1 * sizeof(RowPartial));
  L.off_desc = off;
  off = align256(off + (size_t)B * sizeof(ReqDesc));
  L.off_seg = off;
  off = align256(off + (size_t)B * L.nseg * 2 * sizeof(double));
  L.off_state = off;
  off = align256(off + (size_t)B * sizeof(int32_t));
  L.off_dstate = off;
  off = align256(off + (size_t)B * sizeof(uint64_t));
  L.off_trec = off;
  off = align256(off + (size_t)B * L.R * L.C1 * sizeof(TaggedPartial));
  L.total = off;
  return L;
}

}  // namespace specv
