// Weight-streaming matrix product for the projections around the decode path:
//   out[s][b][n] = sum_{k in slice s} x[b][k] * W[n][k],
// W = rows [0, n0) of w0 stacked on rows [n0, N) of w1 (both row-major, K
// columns), x [batch, K], out fp32 [slices, batch, N].  With small batches every
// weight is read once and the product is bound by the weight stream, so the
// work is cut along n (32-row tiles) and along k (slices) to spread it over the
// whole chip; the consumer adds the slices in slice order (deterministic).
//
// gemm_ws_mfma_kernel (bf16 x and W, N % 32 == 0, K % (16 * 4 * slices) == 0):
// rows^T [n x b] = W [n x k] . x^T [k x b] on v_mfma_f32_32x32x16_bf16.  A
// workgroup owns one 32-row tile of n and one k slice; each weight fragment
// feeds two MFMAs (two 32-row batch tiles, 64 batch rows per pass); its 4
// wavefronts split the slice again and read their operands straight from global
// memory (contiguous along k), 10 k-steps of loads in flight before the first
// MFMA of a group, and add their partial tiles in LDS.
#include "kernels.cuh"

namespace mla {

constexpr int kGemmWaves = 4;
constexpr int kGemmSteps = 10;

__global__ __launch_bounds__(64 * kGemmWaves) void gemm_ws_mfma_kernel(GemmArgs a) {
  __shared__ float red[kGemmWaves - 1][2][16][64];
  const int nt = blockIdx.x * 32, slice = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5;
  const int n = nt + (lane & 31);
  const uint16_t* w = static_cast<const uint16_t*>(n < a.n0 ? a.w0 : a.w1) + int64_t(n < a.n0 ? n : n - a.n0) * a.K;
  const int kw = a.K / (a.slices * kGemmWaves);   // k per wavefront, a multiple of 16
  const int k0 = (slice * kGemmWaves + wave) * kw;
  const int nsteps = kw / 16;
  float* out = a.out + int64_t(slice) * a.batch * a.N;
  for (int bc = 0; bc < a.batch; bc += 64) {
    const uint16_t* x0 = static_cast<const uint16_t*>(a.x) + int64_t(min(bc + (lane & 31), a.batch - 1)) * a.K;
    const uint16_t* x1 = static_cast<const uint16_t*>(a.x) + int64_t(min(bc + 32 + (lane & 31), a.batch - 1)) * a.K;
    f32x16 acc0 = {}, acc1 = {};
    for (int s0 = 0; s0 < nsteps; s0 += kGemmSteps) {
      bf16x8 wf[kGemmSteps], xa[kGemmSteps], xb[kGemmSteps];
#pragma unroll
      for (int t = 0; t < kGemmSteps; ++t) {
        const int k = k0 + (s0 + min(t, nsteps - 1 - s0)) * 16 + 8 * h;
        wf[t] = *reinterpret_cast<const bf16x8*>(w + k);
        xa[t] = *reinterpret_cast<const bf16x8*>(x0 + k);
        xb[t] = *reinterpret_cast<const bf16x8*>(x1 + k);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < kGemmSteps; ++t) {
        if (s0 + t < nsteps) {
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t], xa[t], acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[t], xb[t], acc1, 0, 0, 0);
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
        for (int q = 0; q < kGemmWaves - 1; ++q) {
          v0 += red[q][0][r][lane];
          v1 += red[q][1][r][lane];
        }
        const int nn = nt + 8 * (r >> 2) + 4 * h + (r & 3);
        const int b0 = bc + (lane & 31), b1 = b0 + 32;
        if (b0 < a.batch) out[int64_t(b0) * a.N + nn] = v0;
        if (b1 < a.batch) out[int64_t(b1) * a.N + nn] = v1;
      }
    }
    __syncthreads();
  }
}

// any dtypes and shapes, one slice: a VALU dot product per (b, n)
__global__ __launch_bounds__(256) void gemm_ws_generic_kernel(GemmArgs a) {
  const int b = blockIdx.x, n = blockIdx.y * 256 + threadIdx.x;
  if (n >= a.N) return;
  const void* w = n < a.n0 ? a.w0 : a.w1;
  const int64_t wr = int64_t(n < a.n0 ? n : n - a.n0) * a.K;
  float acc = 0.f;
  for (int k = 0; k < a.K; ++k)
    acc = __builtin_fmaf(load_any(a.x, int64_t(b) * a.K + k, a.x_dt), load_any(w, wr + k, a.w_dt), acc);
  a.out[int64_t(b) * a.N + n] = acc;
}

int gemm_ws_slices(int N, int K) {
  if (N % 32 != 0 || K % (16 * kGemmWaves) != 0) return 1;
  // k slices until the tiles x slices cover the chip about four times
  const int tiles = N / 32;
  for (int sl : {8, 4, 2})
    if (K % (16 * kGemmWaves * sl) == 0 && tiles * sl <= 1024) return sl;
  return 1;
}

void gemm_ws_plan(GemmArgs& a) {
  a.use_mfma = a.x_dt == MLA_BF16 && a.w_dt == MLA_BF16 && a.N % 32 == 0 && a.K % (16 * kGemmWaves) == 0;
  a.slices = a.use_mfma ? gemm_ws_slices(a.N, a.K) : 1;
}

hipError_t launch_gemm_ws(const GemmArgs& a, hipStream_t st) {
  if (a.use_mfma)
    gemm_ws_mfma_kernel<<<dim3(a.N / 32, a.slices), 64 * kGemmWaves, 0, st>>>(a);
  else
    gemm_ws_generic_kernel<<<dim3(a.batch, ceil_div(a.N, 256)), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
