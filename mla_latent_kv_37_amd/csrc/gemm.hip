// Weight-streaming matrix product for the projections around the decode path:
//   out[s][b][n] = sum_{k in slice s} x[b][k] * W[n][k],
// W = rows [0, n0) of w0 stacked on rows [n0, N) of w1 (both row-major, K
// columns), x [batch, K], out fp32 [slices, batch, N].  With small batches every
// weight is read once and the product is bound by the weight stream, so the
// work is cut along n (64-row tiles) and along k (slices) to spread it over the
// whole chip; the consumer adds the slices in slice order (deterministic).
//
// gemm_ws_mfma_kernel (bf16 x and W, N % 64 == 0, K % (64 * slices) == 0):
// out^T [n x b] = W [n x k] . x^T [k x b] on v_mfma_f32_32x32x16_bf16.  A
// workgroup owns a tile of 64 weight rows by 64 batch rows (one 32 x 32 MFMA
// tile per wavefront) and one k slice, which it walks in chunks of 64.
// Operands reach LDS by plain loads in which 8 consecutive lanes read one
// row's 128-byte chunk (whole cache lines per instruction), kGemmDepth chunks
// ahead of use in registers; the chunk is written to one of two LDS buffers
// (row r's 16-byte piece p at r*128 + ((p ^ (r&7) ^ ((r>>3)&1)) * 16), so the
// MFMA fragment reads, 16 rows of one piece per 16 lanes, hit 64 distinct
// banks), then one barrier (no memory fence, so the loads in flight stay in
// flight) publishes it.  Batch rows past the end are clamped to the last row
// and not stored; batches above 64 take more workgroups along z, which read
// the weights again (from the caches when they run together).
#include "kernels.h"

namespace mla {

// kGemmDepth: chunks in flight per thread beyond the one being stored
// (registers).  Few chunks leave room for more resident workgroups: 8 chunks
// held 172 VGPRs (2 wavefronts per SIMD), 2 hold 66 and 1 holds 49 (5).
// Measured: query prep (384 workgroups) 59.6 us with 8, 52.9 with 2, 50.6
// with 1; the cache append (72 workgroups) and the fused query product (1152
// workgroups) are faster with 2 (16.1 vs 18.0 us; 97.9 vs 105.7 us).
template <int kGemmDepth>
__global__ __launch_bounds__(256) void gemm_ws_mfma_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lw[2][kGemmTile * kGemmChunk];
  __shared__ __attribute__((aligned(16))) uint16_t lx[2][kGemmTile * kGemmChunk];
  const int nt0 = blockIdx.x * kGemmTile, slice = blockIdx.y, bb = blockIdx.z * kGemmTile;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const int kslice = a.K / a.slices;
  const int k0 = slice * kslice;
  const int nch = kslice / kGemmChunk;
  // loader: rows lr and 32 + lr of the tile, 16-byte piece lp of the chunk
  const int lr = tid >> 3, lp = tid & 7;
  auto wrow = [&](int r) {
    const int n = nt0 + r;
    return static_cast<const uint16_t*>(n < a.n0 ? a.w0 : a.w1) + int64_t(n < a.n0 ? n : n - a.n0) * a.K;
  };
  auto xrow = [&](int r) { return static_cast<const uint16_t*>(a.x) + int64_t(min(bb + r, a.batch - 1)) * a.K; };
  const uint16_t* wp0 = wrow(lr) + k0 + lp * 8;
  const uint16_t* wp1 = wrow(32 + lr) + k0 + lp * 8;
  const uint16_t* xp0 = xrow(lr) + k0 + lp * 8;
  const uint16_t* xp1 = xrow(32 + lr) + k0 + lp * 8;
  auto sw = [](int r, int p) { return r * kGemmChunk + ((p ^ (r & 7) ^ ((r >> 3) & 1)) * 8); };
  const int so0 = sw(lr, lp), so1 = sw(32 + lr, lp);
  // fragments: wavefront (n tile wave&1, batch tile wave>>1); lane row l&31, piece 2*kstep + h
  const int fr_w = 32 * (wave & 1) + (lane & 31), fr_x = 32 * (wave >> 1) + (lane & 31);

  bf16x8 rw0[kGemmDepth], rw1[kGemmDepth], rx0[kGemmDepth], rx1[kGemmDepth];
  auto load = [&](int d, int c) {
    const int off = min(c, nch - 1) * kGemmChunk;
    rw0[d] = *reinterpret_cast<const bf16x8*>(wp0 + off);
    rw1[d] = *reinterpret_cast<const bf16x8*>(wp1 + off);
    rx0[d] = *reinterpret_cast<const bf16x8*>(xp0 + off);
    rx1[d] = *reinterpret_cast<const bf16x8*>(xp1 + off);
  };
  // prologue loads in the loop's order (chunk by chunk), so that the pending
  // loads at the loop head are in the same order on entry and on every trip
#pragma unroll
  for (int d = 0; d < kGemmDepth; ++d) {
    load(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  f32x16 acc = {};
  // Every step of a group stores, reloads and synchronises unconditionally (steps
  // past the last chunk store and reload copies of it), so the load queue looks
  // the same on every trip and the compiler can wait for one chunk's loads at a
  // time instead of draining all of them at the top of the loop.
  for (int c0 = 0; c0 < nch; c0 += kGemmDepth) {
#pragma unroll
    for (int d = 0; d < kGemmDepth; ++d) {
      const int c = c0 + d;
      // chunk c goes to buffer c & 1: the buffer it overwrites was last read
      // for chunk c - 2, before the barrier of chunk c - 1
      uint16_t MLA_LDS* bw = (uint16_t MLA_LDS*)lw[c & 1];
      uint16_t MLA_LDS* bx = (uint16_t MLA_LDS*)lx[c & 1];
      *reinterpret_cast<bf16x8 MLA_LDS*>(bw + so0) = rw0[d];
      *reinterpret_cast<bf16x8 MLA_LDS*>(bw + so1) = rw1[d];
      *reinterpret_cast<bf16x8 MLA_LDS*>(bx + so0) = rx0[d];
      *reinterpret_cast<bf16x8 MLA_LDS*>(bx + so1) = rx1[d];
      load(d, c + kGemmDepth);
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();
      if (c < nch) {
#pragma unroll
        for (int ks = 0; ks < kGemmChunk / 16; ++ks) {
          const bf16x8 fw = *reinterpret_cast<const bf16x8 MLA_LDS*>(bw + sw(fr_w, 2 * ks + h));
          const bf16x8 fx = *reinterpret_cast<const bf16x8 MLA_LDS*>(bx + sw(fr_x, 2 * ks + h));
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw, fx, acc, 0, 0, 0);
        }
      }
    }
  }
  // D[n][b]: lane holds b = l&31, n = 8(r/4) + 4h + r%4 of the wavefront's tile
  const int b = bb + 32 * (wave >> 1) + (lane & 31);
  if (b < a.batch) {
    float* o = a.out + (int64_t(slice) * a.batch + b) * a.N + nt0 + 32 * (wave & 1) + 4 * h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 v = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      *reinterpret_cast<f32x4*>(o + 8 * q) = v;
    }
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

hipError_t launch_gemm_ws(const GemmArgs& a, hipStream_t st) {
  if (a.use_mfma) {
    const dim3 grid(a.N / kGemmTile, a.slices, ceil_div(a.batch, kGemmTile));
    const int64_t wgs = int64_t(grid.x) * grid.y * grid.z;
    if (wgs >= 256 && wgs <= 512) gemm_ws_mfma_kernel<1><<<grid, 256, 0, st>>>(a);
    else gemm_ws_mfma_kernel<2><<<grid, 256, 0, st>>>(a);
  } else {
    gemm_ws_generic_kernel<<<dim3(a.batch, ceil_div(a.N, 256)), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
