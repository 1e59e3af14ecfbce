// verify_layout.hpp -- chunking of a vocabulary row and the layout of the
// verification workspace (host and device).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace specv {

// A row of V logits is cut into C chunks of `chunk` elements (a multiple of
// the 512-element segment, so segment sums of the sampling pass tile a row
// exactly); one workgroup streams one chunk.  ~32K elements per chunk keeps
// each workgroup's stream long enough to hide its start-up and gives
// thousands of workgroups at the workload sizes of interest.
constexpr int kChunkTarget = 32768;
constexpr int kSeg = 512;  // elements per segment = one wave64 x 8 elements

struct RowPartial {  // one chunk of one row
  float m;           // integer-valued reference exponent (sampled) or max logit (greedy)
  int32_t idx;       // argmax index (greedy)
  double s;          // sum of 2^(x*s - m) over the chunk (sampled)
};

struct ReqDesc {  // decision of one request, consumed by the sampling pass
  int32_t mode;   // kModeNone / kModeResidual / kModeBonus
  int32_t a;      // accepted drafts = the sampling row
  float s_hi, s_lo;
  double mp, sp;  // reference exponent and normaliser of p at row a
  double mq, sq;  // same for q (residual mode)
  double u;       // the sampling uniform of row a
  double pad;
};
static_assert(sizeof(RowPartial) == 16, "RowPartial layout");
static_assert(sizeof(ReqDesc) == 64, "ReqDesc layout");

enum { kModeNone = 0, kModeResidual = 1, kModeBonus = 2 };

struct Layout {
  int32_t R, C, chunk, nseg;
  size_t off_rowp, off_desc, off_seg, total;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline Layout make_layout(int32_t B, int32_t K, int32_t V) {
  Layout L;
  L.R = 2 * K + 1;
  int64_t C = ((int64_t)V + kChunkTarget - 1) / kChunkTarget;
  if (C < 1) C = 1;
  int64_t per = ((int64_t)V + C - 1) / C;
  per = (per + kSeg - 1) / kSeg * kSeg;
  L.chunk = (int32_t)per;
  L.C = (int32_t)(((int64_t)V + per - 1) / per);
  L.nseg = (int32_t)(((int64_t)V + kSeg - 1) / kSeg);
  size_t off = 0;
  L.off_rowp = off;
  off = align256(off + (size_t)B * L.R * L.C * sizeof(RowPartial));
  L.off_desc = off;
  off = align256(off + (size_t)B * sizeof(ReqDesc));
  L.off_seg = off;
  off = align256(off + (size_t)B * L.nseg * 2 * sizeof(double));
  L.total = off;
  return L;
}

}  // namespace specv
