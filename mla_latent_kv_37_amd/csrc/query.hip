// Query side of one decode step, before absorption:
//   c^Q = W^DQ h,  q^C = W^UQ c^Q,  q^R = RoPE(W^QR c^Q)
// ([DeepSeek-V2 explainer] §2.2.1 query compression, §2.2.2 decoupled RoPE;
// [deepseek(2) 關鍵技術] §1 per-head formulas).  Two weight-streaming products
// (gemm.hip) with these kernels after each:
//   reduce_cast_kernel - adds the k slices of c^Q and rounds it to the weights'
//                        dtype (it is the next product's operand);
//   query_finish_kernel - adds the k slices of [q^C ; q^R], rotates each head's
//                        q^R pairs (2k, 2k+1) by pos * base^(-2k/d_h^R) (angle in
//                        fp64) and writes q_nope [B, n_h, d_h], q_pe [B, n_h, d_h^R].
#include "kernels.h"

namespace mla {

__global__ __launch_bounds__(256) void reduce_cast_kernel(const float* __restrict__ slices, int n_slices,
                                                          int64_t count, void* out, mla_dtype_t out_dt) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= count) return;
  float v = slices[i];
  for (int s = 1; s < n_slices; ++s) v += slices[int64_t(s) * count + i];
  store_any(out, i, v, out_dt);
}

__global__ __launch_bounds__(256) void query_finish_kernel(QueryFinishArgs a) {
  const int b = blockIdx.y;
  const int pair = blockIdx.x * 256 + threadIdx.x;          // columns 2*pair, 2*pair + 1
  const int nc = a.n_heads * a.d_head, nr = a.n_heads * a.d_rope, N = nc + nr;
  if (2 * pair >= N) return;
  const int64_t count = int64_t(a.batch) * N;
  const int64_t i = int64_t(b) * N + 2 * pair;
  float x0 = a.slices[i], x1 = a.slices[i + 1];
  for (int s = 1; s < a.n_slices; ++s) {
    x0 += a.slices[int64_t(s) * count + i];
    x1 += a.slices[int64_t(s) * count + i + 1];
  }
  const int c = 2 * pair;
  if (c < nc) {   // q^C (d_head is even, so a pair never straddles q^C and q^R)
    store_any(a.q_nope, int64_t(b) * nc + c, x0, a.out_dt);
    store_any(a.q_nope, int64_t(b) * nc + c + 1, x1, a.out_dt);
    return;
  }
  const int r = c - nc, j = r % a.d_rope;                   // j even: pair j/2 of a head
  if (a.rope.base > 0.f) {
    const int pos = load_const(a.positions, b);
    const double theta = rope_theta(j >> 1, a.d_rope, a.rope);
    const double ang = double(pos) * theta;
    const double cs = cos(ang), sn = sin(ang);
    const double y0 = double(x0) * cs - double(x1) * sn, y1 = double(x0) * sn + double(x1) * cs;
    x0 = float(y0);
    x1 = float(y1);
  }
  store_any(a.q_pe, int64_t(b) * nr + r, x0, a.out_dt);
  store_any(a.q_pe, int64_t(b) * nr + r + 1, x1, a.out_dt);
}

hipError_t launch_reduce_cast(const float* slices, int n_slices, int64_t count, void* out, mla_dtype_t out_dt,
                              hipStream_t st) {
  reduce_cast_kernel<<<unsigned((count + 255) / 256), 256, 0, st>>>(slices, n_slices, count, out, out_dt);
  return hipGetLastError();
}

hipError_t launch_query_finish(const QueryFinishArgs& a, hipStream_t st) {
  const int N = a.n_heads * (a.d_head + a.d_rope);
  query_finish_kernel<<<dim3(ceil_div(N / 2, 256), a.batch), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
