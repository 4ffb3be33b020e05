// Several new query tokens per sequence (q_len > 1), causal within them.
//
// New token t of sequence b sits at position T_b - q_len + t and attends to
// cache tokens [0, T_b - q_len + t + 1) ([deepseek(2) 關鍵技術] §1: the sum
// over the tokens up to the query's own position; §2.2: the multi-token
// prediction modules may be kept for decoding, which gives q_len > 1).
//
// Each (sequence, new token) pair becomes one virtual sequence b' = b*q_len + t
// of the ordinary decode: its length is T_b - q_len + t + 1 (0 if negative) and
// its block-table row is sequence b's.  A workgroup cannot hold more than one
// token's 128 heads (their fp32 accumulators fill half a CU's register file), so
// every virtual sequence streams the pages itself; the copies of one sequence
// are adjacent in the work-item order, which puts them on the same XCD at
// about the same time, so the repeated page reads are served from L2 and the
// Infinity Cache rather than from HBM.
//
// expand_kernel writes the virtual lengths and block table (one workgroup per
// virtual sequence).
#include "kernels.h"

namespace mla {

__global__ __launch_bounds__(256) void expand_kernel(const int32_t* __restrict__ seq_lens,
                                                     const int32_t* __restrict__ block_table, int q_len,
                                                     int max_pages, int32_t* __restrict__ lens_out,
                                                     int32_t* __restrict__ bt_out) {
  const int vb = blockIdx.x;
  const int b = vb / q_len, t = vb % q_len;
  const int32_t* src = block_table + int64_t(b) * max_pages;
  int32_t* dst = bt_out + int64_t(vb) * max_pages;
  for (int p = threadIdx.x; p < max_pages; p += 256) dst[p] = src[p];
  if (threadIdx.x == 0) lens_out[vb] = max(load_const(seq_lens, b) - q_len + t + 1, 0);
}

hipError_t launch_expand(const int32_t* seq_lens, const int32_t* block_table, int batch, int q_len, int max_pages,
                         int32_t* lens_out, int32_t* bt_out, hipStream_t st) {
  expand_kernel<<<batch * q_len, 256, 0, st>>>(seq_lens, block_table, q_len, max_pages, lens_out, bt_out);
  return hipGetLastError();
}

}  // namespace mla
