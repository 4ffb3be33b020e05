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
// project kernels: rows[b] = [W^DKV h_b ; W^KR h_b] in fp32, a weight-streaming
// GEMM (v_mfma_f32_32x32x16_bf16 for bf16 operands and 32-aligned widths, in k
// slices that the store kernel adds up; else a VALU dot product).
#include "kernels.cuh"

namespace mla {

constexpr int kGroup = 128;
constexpr float kE4m3Max = 448.f;

__global__ __launch_bounds__(640) void cache_store_kernel(CacheStoreArgs a) {
  const int b = blockIdx.x;
  const int g = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int W = a.d_latent + a.d_rope;
  const int ng = (W + kGroup - 1) / kGroup;
  if (g >= ng) return;
  const int pos = load_const(a.positions, b);
  if (pos < 0 || pos >= a.max_pages * a.page_size) return;
  const int page = load_const(a.block_table, int64_t(b) * a.max_pages + pos / a.page_size);
  if (page < 0 || page >= a.num_pages) return;   // never write outside the cache
  const int64_t row = int64_t(page) * a.page_size + pos % a.page_size;

  const int c0 = g * kGroup + 2 * lane;
  const int gend = min(W, (g + 1) * kGroup);
  const bool live = c0 < gend;   // W is even, so c0 + 1 < gend too
  float x0 = 0.f, x1 = 0.f;
  if (live) {
    x0 = load_any(a.rows, int64_t(b) * W + c0, a.rows_dt);
    x1 = load_any(a.rows, int64_t(b) * W + c0 + 1, a.rows_dt);
    if (a.n_partials > 1) {
      // projection slices (fp32), summed in slice order; the sum replaces slice 0
      const float* pr = static_cast<const float*>(a.rows) + int64_t(b) * W + c0;
      for (int q = 1; q < a.n_partials; ++q) {
        x0 += pr[int64_t(q) * a.batch * W];
        x1 += pr[int64_t(q) * a.batch * W + 1];
      }
      float* r0 = static_cast<float*>(const_cast<void*>(a.rows)) + int64_t(b) * W + c0;
      r0[0] = x0;
      r0[1] = x1;
    }
    if (a.rope_base > 0.f && c0 >= a.d_latent) {
      const int k = (c0 - a.d_latent) >> 1;
      const double theta = pow(double(a.rope_base), -2.0 * k / double(a.d_rope));
      const double ang = double(pos) * theta;
      const double c = cos(ang), s = sin(ang);
      const double y0 = double(x0) * c - double(x1) * s, y1 = double(x0) * s + double(x1) * c;
      x0 = float(y0);
      x1 = float(y1);
    }
  }
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

// rows[b][n] = sum_k h[b][k] * Wn[k], Wn = row n of [W^DKV ; W^KR] (any shapes)
__global__ __launch_bounds__(256) void project_generic_kernel(ProjectArgs a) {
  const int b = blockIdx.x, n = blockIdx.y * 256 + threadIdx.x;
  const int W = a.d_latent + a.d_rope;
  if (n >= W) return;
  const void* w = n < a.d_latent ? a.w_dkv : a.w_kr;
  const int64_t wr = int64_t(n < a.d_latent ? n : n - a.d_latent) * a.d_model;
  float acc = 0.f;
  for (int k = 0; k < a.d_model; ++k)
    acc = __builtin_fmaf(load_any(a.h, int64_t(b) * a.d_model + k, a.h_dt), load_any(w, wr + k, a.w_dt), acc);
  a.rows[int64_t(b) * W + n] = acc;
}

// MFMA version for bf16 h and weights, (d_c + d_rope) % 32 == 0, d_model % 512 == 0:
// rows^T [n x b] = Wcat [n x k] . h^T [k x b].  Workgroup (32-row tile of n, one
// of kProjSplit slices of k): every weight is read once, and each weight
// fragment feeds two MFMAs (two 32-row batch tiles, 64 batch rows per pass).
// The 4 wavefronts split the slice again, with all their operand loads issued
// before the first MFMA (operands straight from global memory, contiguous
// along k), and add their partial tiles in LDS.  Slice s writes its partial
// rows to rows + s * batch * W; the store kernel sums the slices in order.
constexpr int kProjWaves = 4;
constexpr int kProjSteps = 10;   // k-steps of 16 per wavefront for d_model = 5120

__global__ __launch_bounds__(64 * kProjWaves) void project_mfma_kernel(ProjectArgs a) {
  __shared__ float red[kProjWaves - 1][2][16][64];
  const int nt = blockIdx.x * 32, slice = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5;
  const int n = nt + (lane & 31);
  const uint16_t* w = static_cast<const uint16_t*>(n < a.d_latent ? a.w_dkv : a.w_kr) +
                      int64_t(n < a.d_latent ? n : n - a.d_latent) * a.d_model;
  const int kw = a.d_model / (a.ksplit * kProjWaves);   // k per wavefront, a multiple of 16
  const int k0 = (slice * kProjWaves + wave) * kw;
  const int nsteps = kw / 16;
  const int W = a.d_latent + a.d_rope;
  float* out = a.rows + int64_t(slice) * a.batch * W;
  for (int bc = 0; bc < a.batch; bc += 64) {
    const uint16_t* h0 = static_cast<const uint16_t*>(a.h) + int64_t(min(bc + (lane & 31), a.batch - 1)) * a.d_model;
    const uint16_t* h1 = static_cast<const uint16_t*>(a.h) + int64_t(min(bc + 32 + (lane & 31), a.batch - 1)) * a.d_model;
    f32x16 acc0 = {}, acc1 = {};
    for (int s0 = 0; s0 < nsteps; s0 += kProjSteps) {
      bf16x8 wf[kProjSteps], x0[kProjSteps], x1[kProjSteps];
#pragma unroll
      for (int t = 0; t < kProjSteps; ++t) {
        const int k = k0 + (s0 + min(t, nsteps - 1 - s0)) * 16 + 8 * h;
        wf[t] = *reinterpret_cast<const bf16x8*>(w + k);
        x0[t] = *reinterpret_cast<const bf16x8*>(h0 + k);
        x1[t] = *reinterpret_cast<const bf16x8*>(h1 + k);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < kProjSteps; ++t) {
        if (s0 + t < nsteps) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t], x0[t], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t], x1[t], acc1, 0, 0, 0);
        }
      }
    }
    if (wave > 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        red[wave - 1][0][r][lane] = acc0[r];
        red[wave - 1][1][r][lane] = acc1[r];
      }
    }
    __syncthreads();
    if (wave == 0) {
      // D[n][b]: lane holds b = lane % 32, n = 8(r/4) + 4(lane/32) + r%4
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v0 = acc0[r], v1 = acc1[r];
#pragma unroll
        for (int q = 0; q < kProjWaves - 1; ++q) {
          v0 += red[q][0][r][lane];
          v1 += red[q][1][r][lane];
        }
        const int nn = nt + 8 * (r >> 2) + 4 * h + (r & 3);
        const int b0 = bc + (lane & 31), b1 = b0 + 32;
        if (b0 < a.batch) out[int64_t(b0) * W + nn] = v0;
        if (b1 < a.batch) out[int64_t(b1) * W + nn] = v1;
      }
    }
    __syncthreads();
  }
}

int project_ksplit(mla_dtype_t h_dt, mla_dtype_t w_dt, int width, int d_model) {
  constexpr int kSplit = 8;
  if (h_dt == MLA_BF16 && w_dt == MLA_BF16 && width % 32 == 0 && d_model % (kSplit * kProjWaves * 16) == 0)
    return kSplit;
  return 1;
}

hipError_t launch_cache_store(const CacheStoreArgs& a, int batch, hipStream_t st) {
  const int W = a.d_latent + a.d_rope;
  const int ng = (W + kGroup - 1) / kGroup;
  cache_store_kernel<<<batch, 64 * ng, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_project(const ProjectArgs& a, hipStream_t st) {
  const int W = a.d_latent + a.d_rope;
  if (a.ksplit > 1)
    project_mfma_kernel<<<dim3(W / 32, a.ksplit), 64 * kProjWaves, 0, st>>>(a);
  else
    project_generic_kernel<<<dim3(a.batch, ceil_div(W, 256)), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
