// Query side of one decode step, before absorption:
//   c^Q = W^DQ h,  q^C = W^UQ c^Q,  q^R = RoPE(W^QR c^Q)
// ([DeepSeek-V2 explainer] §2.2.1 query compression, §2.2.2 decoupled RoPE;
// [deepseek(2) 關鍵技術] §1 per-head formulas).  Two weight-streaming products
// (gemm.hip) with these kernels after each:
//   reduce_cast_kernel - adds the k slices of c^Q and rounds it to the weights'
//                        dtype (it is the next product's operand); extra
//                        workgroups of the same launch compute the (cos, sin)
//                        table of each sequence's q^R rotation when the second
//                        product finishes the query itself (one k slice: the V2
//                        shapes), which then writes q_nope and the rotated q_pe
//                        from its accumulators;
//   query_finish_kernel - otherwise: adds the k slices of [q^C ; q^R], rotates
//                        each head's q^R pairs (2k, 2k+1) by pos * theta_k (angle
//                        in fp64) and writes q_nope [B, n_h, d_h], q_pe [B, n_h, d_h^R].
#include "kernels.h"

namespace mla {

__device__ __forceinline__ void rope_table_entry(const RopeTableArgs& t, int idx);

__global__ __launch_bounds__(256) void reduce_cast_kernel(const float* __restrict__ slices, int n_slices,
                                                          int64_t count, void* out, mla_dtype_t out_dt,
                                                          RopeTableArgs tab, int red_blocks) {
  if (int(blockIdx.x) >= red_blocks) {
    rope_table_entry(tab, (int(blockIdx.x) - red_blocks) * 256 + int(threadIdx.x));
    return;
  }
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
  // every slice's loads go out before the first addition (the slices were just
  // written: a chain of dependent cache round trips otherwise)
  float u0[kQueryMaxSlices], u1[kQueryMaxSlices];
#pragma unroll
  for (int s = 0; s < kQueryMaxSlices; ++s)
    if (s < a.n_slices) {
      u0[s] = a.slices[int64_t(s) * count + i];
      u1[s] = a.slices[int64_t(s) * count + i + 1];
    }
  float x0 = u0[0], x1 = u1[0];
#pragma unroll
  for (int s = 1; s < kQueryMaxSlices; ++s)
    if (s < a.n_slices) {
      x0 += u0[s];
      x1 += u1[s];
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

// Four consecutive elements per thread with 16-byte loads and stores, where the
// width and pointers allow (the V2 shapes do); the additions and roundings are
// the same as above, element by element.
// Workgroups past the reduction's compute the RoPE table of the query epilogue
// (one (cos, sin) pair per thread), in the same launch.
__device__ __forceinline__ void rope_table_entry(const RopeTableArgs& t, int idx) {
  const int half = t.d_rope >> 1;
  if (idx >= t.batch * half) return;
  const int b = idx / half, p = idx % half;
  const double ang = double(load_const(t.positions, b)) * rope_theta(p, t.d_rope, t.rope);
  t.table[2 * idx] = cos(ang);
  t.table[2 * idx + 1] = sin(ang);
}

__global__ __launch_bounds__(256) void reduce_cast_v4_kernel(const float* __restrict__ slices, int n_slices,
                                                             int64_t count, void* out, mla_dtype_t out_dt,
                                                             RopeTableArgs tab, int red_blocks) {
  if (int(blockIdx.x) >= red_blocks) {
    rope_table_entry(tab, (int(blockIdx.x) - red_blocks) * 256 + int(threadIdx.x));
    return;
  }
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i >= count) return;
  // every slice's load goes out before the first addition (the slices were just
  // written: a chain of dependent cache round trips otherwise)
  f32x4 x[kQueryMaxSlices];
#pragma unroll
  for (int s = 0; s < kQueryMaxSlices; ++s)
    if (s < n_slices) x[s] = *reinterpret_cast<const f32x4*>(slices + int64_t(s) * count + i);
  f32x4 v = x[0];
#pragma unroll
  for (int s = 1; s < kQueryMaxSlices; ++s)
    if (s < n_slices) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += x[s][e];
    }
  if (out_dt == MLA_BF16) {
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (__bf16)v[e];
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(out) + i) = o;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + i) = v;
  }
}

hipError_t launch_reduce_cast(const float* slices, int n_slices, int64_t count, void* out, mla_dtype_t out_dt,
                              const RopeTableArgs& tab, hipStream_t st) {
  const int tab_blocks = tab.table != nullptr ? ceil_div(tab.batch * (tab.d_rope >> 1), 256) : 0;
  if (count % 4 == 0 && n_slices <= kQueryMaxSlices && (reinterpret_cast<uintptr_t>(slices) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    const int red = int((count / 4 + 255) / 256);
    reduce_cast_v4_kernel<<<unsigned(red + tab_blocks), 256, 0, st>>>(slices, n_slices, count, out, out_dt, tab, red);
  } else {
    const int red = int((count + 255) / 256);
    reduce_cast_kernel<<<unsigned(red + tab_blocks), 256, 0, st>>>(slices, n_slices, count, out, out_dt, tab, red);
  }
  return hipGetLastError();
}

hipError_t launch_query_finish(const QueryFinishArgs& a, hipStream_t st) {
  const int N = a.n_heads * (a.d_head + a.d_rope);
  query_finish_kernel<<<dim3(ceil_div(N / 2, 256), a.batch), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
