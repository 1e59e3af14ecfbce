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
#include "expand_device.hpp"
#include "verify_kernels.hpp"

namespace specv {

template <bool VEC>
__global__ __launch_bounds__(kWG) void expand_kernel(ExpandParams P) {
  const int b = blockIdx.x / P.G;
  const int g = blockIdx.x % P.G;
  const int tid = threadIdx.x;
  const ExpandWindow w = expand_window(P, b);
  if (g == 0 && tid == 0) expand_out_start(P, b, w);
  if (!w.valid) {
    if (!P.hidden_only && g == 0) expand_invalid(P, b, tid, kWG);
    return;
  }
  // The hidden copy and the metadata are independent, and the metadata is a
  // chain of dependent loads (the bonus token after the accepted count, the
  // block table after the position), so with both to do the last wave writes
  // the metadata while the other waves copy.
  const bool do_meta = !P.hidden_only;
  const int meta_first = (do_meta && P.out_h != nullptr) ? kWG - 64 : 0;  // metadata threads from here on
  const int copy_threads = do_meta ? meta_first : kWG;
  if (P.out_h != nullptr && tid < copy_threads) expand_copy_rows<VEC>(P, w, g, P.G, tid, copy_threads);
  if (do_meta && tid >= meta_first) expand_meta_rows(P, b, w, g, P.G, tid - meta_first, kWG - meta_first, false);
}

hipError_t launch_expand(const ExpandParams& P, bool vec, hipStream_t stream) {
  const int64_t grid = (int64_t)P.B * P.G;
  if (vec) hipLaunchKernelGGL(expand_kernel<true>, dim3((unsigned)grid), dim3(kWG), 0, stream, P);
  else hipLaunchKernelGGL(expand_kernel<false>, dim3((unsigned)grid), dim3(kWG), 0, stream, P);
  return hipGetLastError();
}

}  // namespace specv
