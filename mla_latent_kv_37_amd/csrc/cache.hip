// Writing new tokens into the paged latent cache.
//
// A cached token row is [c^KV (d_c) | k^R (d_h^R)] with k^R stored after its
// rotation ([DeepSeek-V2 explainer] §2.2.2: only c^KV and the rotated k^R are
// cached; §2.2.1: c^KV = W^DKV h).  Token t of sequence b goes to page
// block_table[b][t / page_size], slot t % page_size.
//
// cache_store_kernel: one workgroup per sequence, one wavefront per 128-column
// group, two adjacent columns per lane (so a RoPE pair (2k, 2k+1) is in one
// lane).  Storage rounding:
//   f32  - stored as is;
//   bf16 - round to nearest, ties to even;
//   fp8  - per group, scale = amax / 448 in binary32 (1 for an all-zero group),
//          code = E4M3(x / scale), the quotient in binary32 and rounded to the
//          nearest E4M3 value by the hardware convert (the 1x128 per-token-group
//          format of the V3 interview notes, section F8量化策略).
// RoPE: pairs (x[2k], x[2k+1]) of the last d_h^R columns are rotated by
// pos * base^(-2k/d_h^R); the angle and its sine and cosine are evaluated in
// fp64, since positions reach 1e5 and a binary32 angle would be off by 1e-2.
//
// The projection rows[b] = [W^DKV h_b ; W^KR h_b] of mla_cache_append is the
// weight-streaming product of gemm.hip, in k slices that this kernel adds up.
#include "kernels.h"

namespace mla {

constexpr int kGroup = 128;
constexpr float kE4m3Max = 448.f;

__global__ __launch_bounds__(640) void cache_store_kernel(CacheStoreArgs a) {
  const int b = blockIdx.x;
  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int W = a.d_latent + a.d_rope;
  const int ng = (W + kGroup - 1) / kGroup;
  if (g >= ng) return;
  // A position outside the block table or a page id outside the cache skips
  // the cache write only: the projection slices are still summed into rows[b].
  const int pos = load_const(a.positions, b);
  const bool pos_ok = pos >= 0 && pos < a.max_pages * a.page_size;
  const int page = pos_ok ? load_const(a.block_table, int64_t(b) * a.max_pages + pos / a.page_size) : -1;
  const bool store = pos_ok && page >= 0 && page < a.num_pages;   // never write outside the cache
  const int64_t row = int64_t(store ? page : 0) * a.page_size + (store ? pos % a.page_size : 0);

  const int c0 = g * kGroup + 2 * lane;
  const int gend = min(W, (g + 1) * kGroup);
  const bool live = c0 < gend;   // W is even, so c0 + 1 < gend too
  float x0 = 0.f, x1 = 0.f;
  if (live) {
    x0 = load_any(a.rows, int64_t(b) * W + c0, a.rows_dt);
    x1 = load_any(a.rows, int64_t(b) * W + c0 + 1, a.rows_dt);
    if (a.n_partials > 1) {
      // projection slices (fp32), summed in slice order; the sum replaces slice
      // 0.  Every slice's load goes out before the first addition (the slices
      // were just written: a chain of dependent cache round trips otherwise).
      const float* pr = static_cast<const float*>(a.rows) + int64_t(b) * W + c0;
      float p0[kGemmMaxSlices], p1[kGemmMaxSlices];
#pragma unroll
      for (int q = 1; q < kGemmMaxSlices; ++q)
        if (q < a.n_partials) {
          p0[q] = pr[int64_t(q) * a.batch * W];
          p1[q] = pr[int64_t(q) * a.batch * W + 1];
        }
#pragma unroll
      for (int q = 1; q < kGemmMaxSlices; ++q)
        if (q < a.n_partials) {
          x0 += p0[q];
          x1 += p1[q];
        }
      float* r0 = static_cast<float*>(const_cast<void*>(a.rows)) + int64_t(b) * W + c0;
      r0[0] = x0;
      r0[1] = x1;
    }
    if (store && a.rope.base > 0.f && c0 >= a.d_latent) {
      const int k = (c0 - a.d_latent) >> 1;
      const double theta = rope_theta(k, a.d_rope, a.rope);
      const double ang = double(pos) * theta;
      const double c = cos(ang), s = sin(ang);
      const double y0 = double(x0) * c - double(x1) * s, y1 = double(x0) * s + double(x1) * c;
      x0 = float(y0);
      x1 = float(y1);
    }
  }
  if (!store) return;
  if (a.kv_dt == MLA_F32) {
    if (live) {
      float* dst = static_cast<float*>(a.kv) + row * W + c0;
      dst[0] = x0;
      dst[1] = x1;
    }
  } else if (a.kv_dt == MLA_BF16) {
    if (live) {
      const uint32_t pair = uint32_t(f32_to_bf16(x0)) | (uint32_t(f32_to_bf16(x1)) << 16);
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(a.kv) + row * W + c0) = pair;
    }
  } else {
    float m = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float scale = m > 0.f ? m / kE4m3Max : 1.f;
    if (live) {
      const float q0 = x0 / scale, q1 = x1 / scale;
      const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
      *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(a.kv) + row * W + c0) = uint16_t(packed & 0xFFFF);
    }
    if (lane == 0) a.scales[row * ng + g] = scale;
  }
}

hipError_t launch_cache_store(const CacheStoreArgs& a, int batch, hipStream_t st) {
  const int W = a.d_latent + a.d_rope;
  const int ng = (W + kGroup - 1) / kGroup;
  cache_store_kernel<<<batch, 64 * ng, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
