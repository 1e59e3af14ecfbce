// expand.hip -- P-EAGLE parallel-drafting batch expansion and hidden-state
// gather on gfx950, as one kernel.
//
// "P-EAGLE: parallel speculative decoding in vLLM" page: the drafter batch
// appends K-1 MASK slots per request ("并行草稿生成的挑战"); one pass copies the
// old token ids and positions into shifted slots, inserts the bonus token,
// fills the MASK slots and emits the rejected / masked masks, the new-token
// indices and the hidden-state mapping ("Triton Kernel"); the hidden rows are
// the mapped target rows, the MASK slots take the learned placeholder
// ("Hidden State 管理").  The page writes the hidden rows as a scatter through
// the mapping followed by a masked overwrite; here every output row is
// written exactly once as a gather, which gives the same rows because the
// mapping is injective and, with the MASK slots, covers the output.
//
// With a block table, each output slot also gets its KV-cache slot in the
// paged cache (block_table[b, pos / block_size] * block_size + pos %
// block_size), and rejected slots, or positions with no block, get
// PADDING_SLOT_ID = -1 ("Hidden State 管理": no cache write for them).
//
// The hidden rows depend only on the windows (not on the accepted counts), so
// they can also be gathered alone, on another stream, while the verification
// that produces the counts is still running (spec_expand_hidden_launch).
//
// Request b owns the fixed window of n_b + K - 1 slots starting at
// in_start[b] + b*(K-1), so no scan is needed; G workgroups share a request's
// window row-interleaved, each writing the metadata of its rows and copying
// its hidden rows with 16-byte loads and stores.
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

constexpr int kCopyBatch = 8;  // 16-byte cells per lane loaded before any is stored

template <bool VEC>
__global__ __launch_bounds__(kWG) void expand_kernel(ExpandParams P) {
  const int b = blockIdx.x / P.G;
  const int g = blockIdx.x % P.G;
  const int K = P.K;
  const int tid = threadIdx.x;
  const bool gvalid = P.in_start[0] == 0 && P.in_start[P.B] == P.N_in;
  const int s = P.in_start[b];
  const int s1 = P.in_start[b + 1];
  const int n = s1 - s;
  const int a = P.hidden_only ? 0 : P.acc[b];
  const int o = s + b * (K - 1);
  const int a_max = P.vtok ? min(n - 1, K) : n - 1;
  if (gvalid && g == 0 && tid == 0 && !P.hidden_only) {
    P.out_start[b] = o;
    if (b == P.B - 1) P.out_start[P.B] = P.N_in + P.B * (K - 1);
  }
  const bool window_ok = gvalid && n >= 1 && s >= 0 && s1 <= P.N_in;
  const bool valid = window_ok && (P.hidden_only || (a >= 0 && a <= a_max));
  if (!valid) {
    if (P.hidden_only) return;
    if (g == 0)
      for (int m = tid; m < K; m += kWG) P.nti[(int64_t)b * K + m] = -1;
    return;
  }
  const int Wb = n + K - 1;  // slots of this request's window

  // The hidden copy and the metadata are independent, and the metadata is a
  // chain of dependent loads (the bonus token after the accepted count, the
  // block table after the position), so with both to do the last wave writes
  // the metadata while the other waves copy.
  const bool do_meta = !P.hidden_only;
  const bool do_copy = P.out_h != nullptr && g < Wb;
  const int meta_first = (do_meta && P.out_h != nullptr) ? kWG - 64 : 0;  // metadata threads from here on
  const int copy_threads = do_meta ? meta_first : kWG;

  // hidden rows g, g+G, ... of the window: slot o+r takes input row s+r
  // (r < n) or the MASK placeholder; loads of a batch are all issued before
  // its stores, and the output is written once (non-temporal stores)
  if (do_copy && tid < copy_threads) {
    const int nr = (Wb - g + P.G - 1) / P.G;
    if constexpr (VEC) {
      const int ncols = P.H >> 3;
      const int cells = nr * ncols;
      for (int c0 = tid; c0 < cells; c0 += copy_threads * kCopyBatch) {
        u32x4 v[kCopyBatch];
        int64_t dst[kCopyBatch];
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u) {
          const int c = c0 + u * copy_threads;
          dst[u] = -1;
          if (c < cells) {
            const int rl = c / ncols, col = c - rl * ncols;
            const int r = g + P.G * rl;
            const uint16_t* src = r < n ? P.th + (int64_t)(s + r) * P.th_stride : P.mh;
            v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + col);
            dst[u] = (int64_t)(o + r) * ncols + col;
          }
        }
#pragma unroll
        for (int u = 0; u < kCopyBatch; ++u)
          if (dst[u] >= 0) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4*>(P.out_h) + dst[u]);
      }
    } else {
      const int cells = nr * P.H;
      for (int c = tid; c < cells; c += copy_threads) {
        const int rl = c / P.H, col = c - rl * P.H;
        const int r = g + P.G * rl;
        const uint16_t* src = r < n ? P.th + (int64_t)(s + r) * P.th_stride : P.mh;
        P.out_h[(int64_t)(o + r) * P.H + col] = src[col];
      }
    }
  }

  if (!do_meta || tid < meta_first) return;

  // metadata: one thread per slot r of this workgroup's rows g, g+G, ...
  const int mt = tid - meta_first, meta_threads = kWG - meta_first;
  const int bonus = P.vtok ? P.vtok[(int64_t)b * (K + 1) + a] : P.bonus[b];
  for (int r = g + P.G * mt; r < Wb; r += P.G * meta_threads) {
    const int slot = o + r;
    int64_t pos;
    bool rejected;
    if (r < n) {
      pos = P.pos[s + r] + 1;
      rejected = r > a;
      P.hmap[s + r] = slot;
      P.out_ids[slot] = (r == a) ? bonus : P.ids[s + min(r + 1, n - 1)];
      P.rej[slot] = (uint8_t)rejected;
      P.msk[slot] = 0;
      if (r == a) P.nti[(int64_t)b * K] = slot;
    } else {
      const int m = r - n + 1;  // 1..K-1
      pos = P.pos[s + a] + 1 + m;
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

hipError_t launch_expand(const ExpandParams& P, bool vec, hipStream_t stream) {
  const int64_t grid = (int64_t)P.B * P.G;
  if (vec) hipLaunchKernelGGL(expand_kernel<true>, dim3((unsigned)grid), dim3(kWG), 0, stream, P);
  else hipLaunchKernelGGL(expand_kernel<false>, dim3((unsigned)grid), dim3(kWG), 0, stream, P);
  return hipGetLastError();
}

}  // namespace specv
