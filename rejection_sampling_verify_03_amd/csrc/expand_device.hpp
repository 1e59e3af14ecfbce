// expand_device.hpp -- device pieces of the P-EAGLE batch expansion, shared
// by its own kernel and by the verification's sampling stage when the
// expansion of a verification's outputs is chained onto it.
//
// "P-EAGLE: parallel speculative decoding in vLLM" page, sections "Triton
// Kernel" and "Hidden State 管理": request b owns the fixed window of
// n_b + K - 1 output slots starting at in_start[b] + b*(K-1); slot r < n_b
// takes the shifted id (the bonus token at r = a_b), the position + 1 and the
// hidden row of input slot r; the K-1 slots after them are MASK slots with
// the learned placeholder row and advancing positions; rejected slots
// (r > a_b) get no KV-cache slot.
#pragma once

#include "device_common.hpp"
#include "verify_kernels.hpp"

namespace specv {

// KV-cache slot of output slot position pos of request b (-1: none).
__device__ __forceinline__ int64_t cache_slot(const ExpandParams& P, int b, int64_t pos, bool rejected) {
  if (rejected || pos < 0) return -1;
  const int64_t blk = pos / P.block_size;
  if (blk >= P.max_blocks) return -1;
  const int32_t phys = P.bt[(int64_t)b * P.bt_stride + blk];
  return phys < 0 ? -1 : (int64_t)phys * P.block_size + pos % P.block_size;
}

// Request b's window: input slots [s, s + n), output slots [o, o + W), the
// accepted count a (0 for a hidden-only gather), and whether it is valid.
struct ExpandWindow {
  int s, n, o, W, a;
  bool gvalid;  // in_start[0] == 0 and in_start[B] == N_in
  bool valid;
};

__device__ __forceinline__ ExpandWindow expand_window(const ExpandParams& P, int b) {
  ExpandWindow w;
  w.gvalid = P.in_start[0] == 0 && P.in_start[P.B] == P.N_in;
  w.s = P.in_start[b];
  const int s1 = P.in_start[b + 1];
  w.n = s1 - w.s;
  w.a = P.hidden_only ? 0 : P.acc[b];
  w.o = w.s + b * (P.K - 1);
  w.W = w.n + P.K - 1;
  const int a_max = P.vtok ? min(w.n - 1, P.K) : w.n - 1;
  const bool window_ok = w.gvalid && w.n >= 1 && w.s >= 0 && s1 <= P.N_in;
  w.valid = window_ok && (P.hidden_only || (w.a >= 0 && w.a <= a_max));
  return w;
}

// The request's output start (and the total after the last request),
// written whenever the input starts are consistent, valid request or not
// (one thread per request).
__device__ __forceinline__ void expand_out_start(const ExpandParams& P, int b, const ExpandWindow& w) {
  if (!w.gvalid || P.hidden_only) return;
  P.out_start[b] = w.o;
  if (b == P.B - 1) P.out_start[P.B] = P.N_in + P.B * (P.K - 1);
}

// What a request with invalid data writes: its new-token indices, all -1
// (workgroup g == 0 of the request only).
__device__ __forceinline__ void expand_invalid(const ExpandParams& P, int b, int tid, int nthreads) {
  for (int m = tid; m < P.K; m += nthreads) P.nti[(int64_t)b * P.K + m] = -1;
}

constexpr int kCopyBatch = 8;  // 16-byte cells per lane loaded before any is stored

// The hidden rows g, g + G, ... of request window w, copied by `nthreads`
// threads (tid in [0, nthreads)): slot o + r takes input row s + r (r < n)
// or the MASK placeholder; loads of a batch are all issued before its stores,
// and the output is written once (non-temporal stores).  A lane past the last
// cell reloads the last cell and stores nothing: with every load of a batch
// unconditional the compiler can wait for each load by its own count, where
// loads under a branch made it drain the whole queue before every store.
template <bool VEC>
__device__ __forceinline__ void expand_copy_rows(const ExpandParams& P, const ExpandWindow& w, int g, int G, int tid,
                                                 int nthreads) {
  if (g >= w.W) return;
  const int nr = (int)(((int64_t)w.W - g + G - 1) / G);  // rows g, g + G, ... of the window
  if constexpr (VEC) {
    const int ncols = P.H >> 3;
    // cells are counted in 32 bits, in passes of at most 2^30 cells
    const int pass_rows = max(1, (1 << 30) / max(ncols, 1));
    for (int r0 = 0; r0 < nr; r0 += pass_rows) {
      const int cells = min(nr - r0, pass_rows) * ncols;
      for (int c0 = tid; c0 < cells; c0 += nthreads * kCopyBatch) {
        u32x4 v[kCopyBatch];
        int64_t dst[kCopyBatch];
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u) {
          const int c = c0 + u * nthreads;
          const int cl = min(c, cells - 1);
          const int rl = cl / ncols, col = cl - rl * ncols;
          const int r = g + G * (r0 + rl);
          const uint16_t* src = r < w.n ? P.th + (int64_t)(w.s + r) * P.th_stride : P.mh;
          v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + col);
          dst[u] = c < cells ? (int64_t)(w.o + r) * ncols + col : -1;
        }
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u)
          if (dst[u] >= 0) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(P.out_h) + dst[u]);
      }
    }
  } else {
    const int64_t cells = (int64_t)nr * P.H;
    for (int64_t c = tid; c < cells; c += nthreads) {
      const int64_t rl = c / P.H;
      const int col = (int)(c - rl * P.H);
      const int r = g + G * (int)rl;
      const uint16_t* src = r < w.n ? P.th + (int64_t)(w.s + r) * P.th_stride : P.mh;
      P.out_h[(int64_t)(w.o + r) * P.H + col] = src[col];
    }
  }
}

// The metadata of slots g, g + G, ... of request b's window, one thread per
// slot (tid in [0, nthreads)).  With bonus_later the bonus id at slot a is
// left for the caller that samples it.
__device__ __forceinline__ void expand_meta_rows(const ExpandParams& P, int b, const ExpandWindow& w, int g, int G,
                                                 int tid, int nthreads, bool bonus_later) {
  const int K = P.K;
  const int a = w.a;
  const int bonus = bonus_later ? 0 : (P.vtok ? P.vtok[(int64_t)b * (K + 1) + a] : P.bonus[b]);
  for (int64_t rr = g + (int64_t)G * tid; rr < w.W; rr += (int64_t)G * nthreads) {
    const int r = (int)rr;
    const int slot = w.o + r;
    int64_t pos;
    bool rejected;
    if (r < w.n) {
      pos = P.pos[w.s + r] + 1;
      rejected = r > a;
      P.hmap[w.s + r] = slot;
      if (r != a || !bonus_later) P.out_ids[slot] = (r == a) ? bonus : P.ids[w.s + min(r + 1, w.n - 1)];
      P.rej[slot] = (uint8_t)rejected;
      P.msk[slot] = 0;
      if (r == a) P.nti[(int64_t)b * K] = slot;
    } else {
      const int m = r - w.n + 1;  // 1..K-1
      pos = P.pos[w.s + a] + 1 + m;
      rejected = false;
      P.out_ids[slot] = P.mask_id;
      P.rej[slot] = 0;
      P.msk[slot] = 1;
      P.nti[(int64_t)b * K + m] = slot;
    }
    P.out_pos[slot] = pos;
    if (P.slots) P.slots[slot] = cache_slot(P, b, pos, rejected);
  }
}

}  // namespace specv
