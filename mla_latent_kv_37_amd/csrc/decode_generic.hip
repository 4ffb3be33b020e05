// Generic MLA decode: any head count and widths (d_c + d_h^R <= 1280), any cache
// dtype, fp32 arithmetic on the vector ALUs.  One workgroup per (work item, head).
//
// Per head i and segment [t0, t1) of sequence b it computes, tile by tile,
//   s_j = (q_lat_i . c^KV_j + q^R_i . k^R_j) * scale        (absorbed score,
//         [deepseek(2) 關鍵技術] §1 with [DeepSeek-V2 explainer] §2.2.2)
// with an online softmax (running max m, running sum l) and o = sum_j p_j c^KV_j.
#include "kernels.h"

namespace mla {

constexpr int kGenThreads = 256;
constexpr int kGenMaxRow = 1280;
constexpr int kGenMaxCols = 4;  // d_latent <= 4 * 256


// row < 0: a token of an out-of-range page, read as a zero row
template <mla_dtype_t KV>
__device__ __forceinline__ float cache_val(const GenericDecodeArgs& a, int64_t row, int c, int W, int ng) {
  if (row < 0) return 0.f;
  float v = Elem<KV>::load(a.kv, row * W + c);
  if (KV == MLA_FP8_E4M3) v *= a.scales[row * ng + c / 128];
  return v;
}

template <mla_dtype_t KV>
__global__ __launch_bounds__(kGenThreads) void decode_generic_kernel(GenericDecodeArgs a) {
  __shared__ float qs[kGenMaxRow];
  __shared__ float ps[kGenThreads];
  __shared__ int64_t rows[kGenThreads];
  __shared__ float red[kGenThreads / 64];

  const int tid = threadIdx.x;
  const int head = blockIdx.y;
  const int W = a.d_latent + a.d_rope;
  const int ng = (W + 127) / 128;
  const int page = a.pp.page_size;

  auto block_reduce = [&](float v, bool is_max) -> float {
    for (int off = 32; off > 0; off >>= 1) {
      float o = __shfl_xor(v, off);
      v = is_max ? fmaxf(v, o) : v + o;
    }
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kGenThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    __syncthreads();
    return r;
  };

  SegmentIter it;
  it.init(a.pp, a.seq_lens, blockIdx.x, a.meta);
  Segment sg;
  while (it.next(sg)) {
    const int b = sg.b;
    const int64_t qoff = (int64_t(b) * a.n_heads + head);
    for (int c = tid; c < W; c += kGenThreads)
      qs[c] = c < a.d_latent ? load_any(a.q_lat, qoff * a.d_latent + c, a.q_dt)
                             : load_any(a.q_pe, qoff * a.d_rope + (c - a.d_latent), a.q_dt);
    __syncthreads();
    float m = -INFINITY, l = 0.f;
    float o[kGenMaxCols];
#pragma unroll
    for (int k = 0; k < kGenMaxCols; ++k) o[k] = 0.f;
    const int32_t* bt = a.block_table + int64_t(b / a.bt_div) * a.max_pages;
    for (int tt = sg.t0; tt < sg.t1; tt += kGenThreads) {
      const int t = tt + tid;
      float s = -INFINITY;
      if (t < sg.t1) {
        const int pid = bt[t / page];
        const int64_t row = (pid >= 0 && pid < a.num_pages) ? int64_t(pid) * page + (t % page) : -1;
        rows[tid] = row;
        float acc = 0.f;
        for (int c = 0; c < W; ++c) acc += qs[c] * cache_val<KV>(a, row, c, W, ng);
        s = acc * a.scale;
      }
      const float mt = block_reduce(s, true);
      const float mn = fmaxf(m, mt);
      const float alpha = expf(m - mn);  // m = -inf on the first tile -> 0
      const float p = t < sg.t1 ? expf(s - mn) : 0.f;
      ps[tid] = p;
      l = l * alpha + block_reduce(p, false);
      m = mn;
      const int n = min(kGenThreads, sg.t1 - tt);
#pragma unroll
      for (int k = 0; k < kGenMaxCols; ++k) {
        const int c = tid + k * kGenThreads;
        if (c < a.d_latent) {
          float acc = 0.f;
          for (int j = 0; j < n; ++j) acc += ps[j] * cache_val<KV>(a, rows[j], c, W, ng);
          o[k] = o[k] * alpha + acc;
        }
      }
      __syncthreads();
    }
    const float inv = 1.f / l;
    const float lse = m + logf(l);
    if (sg.whole) {
      const int64_t ob = (int64_t(b) * a.n_heads + head) * a.d_latent;
#pragma unroll
      for (int k = 0; k < kGenMaxCols; ++k) {
        const int c = tid + k * kGenThreads;
        if (c < a.d_latent) store_any(a.o_lat, ob + c, o[k] * inv, a.o_dt);
      }
      if (tid == 0 && a.lse != nullptr) a.lse[int64_t(b) * a.n_heads + head] = lse;
    } else {
      const int64_t ob = (int64_t(sg.slot) * a.n_heads + head) * a.d_latent;
#pragma unroll
      for (int k = 0; k < kGenMaxCols; ++k) {
        const int c = tid + k * kGenThreads;
        if (c < a.d_latent) store_any(a.o_part, ob + c, o[k] * inv, a.o_dt);
      }
      if (tid == 0) a.lse_part[int64_t(sg.slot) * a.n_heads + head] = lse;
    }
    __syncthreads();
  }
}

hipError_t launch_decode_generic(const GenericDecodeArgs& a, int n_items, hipStream_t st) {
  dim3 grid(n_items, a.n_heads);
  switch (a.kv_dt) {
    case MLA_F32: decode_generic_kernel<MLA_F32><<<grid, kGenThreads, 0, st>>>(a); break;
    case MLA_BF16: decode_generic_kernel<MLA_BF16><<<grid, kGenThreads, 0, st>>>(a); break;
    default: decode_generic_kernel<MLA_FP8_E4M3><<<grid, kGenThreads, 0, st>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace mla
