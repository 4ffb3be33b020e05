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
// tile per wavefront) and one k slice, which it walks in chunks of 64.  The
// product is bound by the weight stream, so what matters is how many bytes each
// workgroup keeps in flight: the chunks go straight from global memory to LDS
// (direct-to-LDS loads, no registers held), kStages - 1 chunks ahead of the one
// being multiplied, 16 KB each (8 KB of weight rows, 8 KB of batch rows).  Each
// one-KB load covers 8 whole rows (8 cache lines); a row's 16-byte piece p goes
// to slot p ^ (r & 7) ^ ((r >> 3) & 1) of its row, so that the MFMA fragment
// reads, 16 rows of one piece per 16 lanes, hit 64 distinct banks.  One
// barrier per chunk publishes it (each wavefront first waits for its own loads
// of the chunk) and frees the stage of the chunk before it.  Batch rows past
// the end are clamped to the last row and not stored; batches above 64 take
// more workgroups along z, which read the weights again (from the caches when
// they run together).
#include "kernels.h"

namespace mla {

constexpr int kGemmHalf = kGemmTile * kGemmChunk * 2;   // bytes of one operand's chunk (8 KB)
constexpr int kGemmStageBytes = 2 * kGemmHalf;          // weight rows + batch rows
constexpr int kGemmStages = 4;                          // 64 KB of LDS: two workgroups per compute unit

// Four consecutive outputs of one row, in the output dtype (8 or 16 bytes)
__device__ __forceinline__ void store4(void* base, int64_t i, const float (&v)[4], mla_dtype_t dt) {
  if (dt == MLA_BF16) {
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (__bf16)v[e];
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(base) + i) = o;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(base) + i) = f32x4{v[0], v[1], v[2], v[3]};
  }
}

template <int kStages, bool kFinish>
__global__ __launch_bounds__(256) void gemm_ws_mfma_kernel(GemmArgs a) {
  static_assert(kStages >= 2 && 4 * (kStages - 2) <= 15, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char stage_raw[kStages * kGemmStageBytes];
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(stage_raw));
  const int nt0 = blockIdx.x * kGemmTile, slice = blockIdx.y, bb = blockIdx.z * kGemmTile;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const int kslice = a.K / a.slices;
  const int k0 = slice * kslice;
  const int nch = kslice / kGemmChunk;
  // slot (16 bytes) s of an operand chunk holds row s >> 3, piece
  // (s & 7) ^ (r & 7) ^ ((r >> 3) & 1); wavefront w loads slots 128w + 64j + lane
  auto piece = [](int r, int q) { return q ^ (r & 7) ^ ((r >> 3) & 1); };
  const char* wsrc[2];
  const char* xsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int sl = 128 * wave + 64 * j + lane, r = sl >> 3, p = piece(r, sl & 7);
    const int n = nt0 + r;
    const uint16_t* wr = static_cast<const uint16_t*>(n < a.n0 ? a.w0 : a.w1) + int64_t(n < a.n0 ? n : n - a.n0) * a.K;
    const uint16_t* xr = static_cast<const uint16_t*>(a.x) + int64_t(min(bb + r, a.batch - 1)) * a.K;
    wsrc[j] = reinterpret_cast<const char*>(wr + k0 + 8 * p);
    xsrc[j] = reinterpret_cast<const char*>(xr + k0 + 8 * p);
  }
  auto issue = [&](int c) {
    const uint32_t st = lds + uint32_t((c % kStages) * kGemmStageBytes + wave * 2048);
    const int64_t off = int64_t(c) * (kGemmChunk * 2);
    dma16(wsrc[0] + off, st);
    dma16(wsrc[1] + off, st + 1024u);
    dma16(xsrc[0] + off, st + uint32_t(kGemmHalf));
    dma16(xsrc[1] + off, st + uint32_t(kGemmHalf + 1024));
  };
  // fragments: wavefront (n tile wave&1, batch tile wave>>1); lane row l&31, piece 2*kstep + h
  const int fr_w = 32 * (wave & 1) + (lane & 31), fr_x = 32 * (wave >> 1) + (lane & 31);

#pragma unroll
  for (int c = 0; c < kStages - 1; ++c)
    if (c < nch) issue(c);
  f32x16 acc = {};
  for (int c = 0; c < nch; ++c) {
    // this wavefront's loads of chunk c are complete when at most the loads of
    // the chunks issued after it remain; then chunk c is complete for everyone,
    // and everyone is done with chunk c - 1, whose stage takes chunk c + kStages - 1
    wait_vm(4 * min(kStages - 2, nch - 1 - c));
    raw_barrier();
    if (c + kStages - 1 < nch) issue(c + kStages - 1);
    const uint32_t st = lds + uint32_t((c % kStages) * kGemmStageBytes);
    // all of the chunk's fragments are read before its first MFMA
    bf16x8 fw[kGemmChunk / 16], fx[kGemmChunk / 16];
#pragma unroll
    for (int ks = 0; ks < kGemmChunk / 16; ++ks) {
      fw[ks] = *reinterpret_cast<const bf16x8 MLA_LDS*>(
          (const char MLA_LDS*)(uintptr_t)(st + uint32_t(fr_w * 128 + piece(fr_w, 2 * ks + h) * 16)));
      fx[ks] = *reinterpret_cast<const bf16x8 MLA_LDS*>(
          (const char MLA_LDS*)(uintptr_t)(st + uint32_t(kGemmHalf + fr_x * 128 + piece(fr_x, 2 * ks + h) * 16)));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < kGemmChunk / 16; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[ks], fx[ks], acc, 0, 0, 0);
  }
  // D[n][b]: lane holds b = l&31, n = 8(r/4) + 4h + r%4 of the wavefront's tile
  const int b = bb + 32 * (wave >> 1) + (lane & 31);
  if (b >= a.batch) return;
  if constexpr (kFinish) {
    // the query's columns straight to q^C / q^R (no fp32 round trip): the
    // rotation of the unfused finish, on the same fp32 sums and fp64 table
    const int nr = a.N - a.n0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = nt0 + 32 * (wave & 1) + 8 * q + 4 * h;
      float v[4] = {acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
      if (n < a.n0) {
        store4(a.fin_nope, int64_t(b) * a.n0 + n, v, a.fin_dt);
      } else {
        const int r = n - a.n0;
        if (a.fin_rope != nullptr) {
          const double* t = a.fin_rope + 2 * (int64_t(b) * (a.fin_drope >> 1) + ((r % a.fin_drope) >> 1));
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const double cs = t[e], sn = t[e + 1];
            const double y0 = double(v[e]) * cs - double(v[e + 1]) * sn, y1 = double(v[e]) * sn + double(v[e + 1]) * cs;
            v[e] = float(y0);
            v[e + 1] = float(y1);
          }
        }
        store4(a.fin_pe, int64_t(b) * nr + r, v, a.fin_dt);
      }
    }
  } else {
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
    if (a.fin_nope != nullptr) gemm_ws_mfma_kernel<kGemmStages, true><<<grid, 256, 0, st>>>(a);
    else gemm_ws_mfma_kernel<kGemmStages, false><<<grid, 256, 0, st>>>(a);
  } else {
    gemm_ws_generic_kernel<<<dim3(a.batch, ceil_div(a.N, 256)), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mla
