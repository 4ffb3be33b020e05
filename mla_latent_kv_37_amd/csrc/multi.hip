// Several new query tokens per sequence (q_len > 1), causal within them.
//
// New token t of sequence b sits at position T_b - q_len + t and attends to
// cache tokens [0, T_b - q_len + t + 1) ([deepseek(2) 關鍵技術] §1: the sum
// over the tokens up to the query's own position; §2.2: the multi-token
// prediction modules may be kept for decoding, which gives q_len > 1).
//
// Each (sequence, new token) pair becomes one virtual sequence b' = b*q_len + t
// of the ordinary decode: its length is T_b - q_len + t + 1 (0 if negative),
// and the decode kernels read its pages from block-table row b' / q_len, that
// is sequence b's row, in place.  A workgroup cannot hold more than one token's
// 128 heads (their fp32 accumulators fill half a CU's register file), so every
// virtual sequence streams the pages itself; the copies of one sequence are
// adjacent in the work-item order, which puts them on the same XCD at about
// the same time, so the repeated page reads are served from L2 and the
// Infinity Cache rather than from HBM.
//
// expand_kernel writes the virtual lengths.
#include "kernels.h"

namespace mla {

__global__ __launch_bounds__(256) void expand_kernel(const int32_t* __restrict__ seq_lens, int batch, int q_len,
                                                     int32_t* __restrict__ lens_out) {
  const int vb = blockIdx.x * 256 + threadIdx.x;
  if (vb >= batch * q_len) return;
  const int b = vb / q_len, t = vb % q_len;
  lens_out[vb] = max(seq_lens[b] - q_len + t + 1, 0);
}

hipError_t launch_expand(const int32_t* seq_lens, int batch, int q_len, int32_t* lens_out, hipStream_t st) {
  expand_kernel<<<ceil_div(batch * q_len, 256), 256, 0, st>>>(seq_lens, batch, q_len, lens_out);
  return hipGetLastError();
}

}  // namespace mla
