// The two per-head weight products around the decode:
//   absorb:   q_lat[b,i,:] = (W^UK_i)^T q^C[b,i,:]      (W^UK moved to the query side)
//   out proj: o[b, i*d_h:(i+1)*d_h] = W^UV_i o_lat[b,i,:] (W^UV applied after attention)
// [DeepSeek-V2 explainer] §2.2.2 (W^UK absorbed on the query side, W^UV on the
// output side); head i owns rows i*d_h..(i+1)*d_h-1 of W^UK and W^UV.
//
// Both are weight-streaming products (each weight element is used B times), so
// they are bound by HBM; the V2-shape kernels run them on MFMA so the matrix
// work stays far below the time to stream the 16.8 MB weight.
#include "kernels.h"

namespace mla {

// ---------------------------------------------------------------------------
// generic VALU kernels (any widths), one workgroup per (b, head)
// ---------------------------------------------------------------------------
constexpr int kProjThreads = 256;

__global__ __launch_bounds__(kProjThreads) void absorb_generic_kernel(
    const void* q, mla_dtype_t q_dt, const void* w, mla_dtype_t w_dt, void* out, mla_dtype_t o_dt,
    int n_heads, int d_head, int d_latent) {
  __shared__ float qs[1024];
  const int b = blockIdx.x, i = blockIdx.y;
  const int64_t qrow = (int64_t(b) * n_heads + i) * d_head;
  for (int k = threadIdx.x; k < d_head; k += kProjThreads) qs[k] = load_any(q, qrow + k, q_dt);
  __syncthreads();
  const int64_t wrow0 = int64_t(i) * d_head;
  for (int c = threadIdx.x; c < d_latent; c += kProjThreads) {
    float acc = 0.f;
    for (int k = 0; k < d_head; ++k) acc += qs[k] * load_any(w, (wrow0 + k) * d_latent + c, w_dt);
    store_any(out, (int64_t(b) * n_heads + i) * d_latent + c, acc, o_dt);
  }
}

__global__ __launch_bounds__(kProjThreads) void outproj_generic_kernel(
    const void* o, mla_dtype_t o_dt, const void* w, mla_dtype_t w_dt, void* out, mla_dtype_t out_dt,
    int n_heads, int d_head, int d_latent) {
  __shared__ float os[1024];
  const int b = blockIdx.x, i = blockIdx.y;
  const int64_t orow = (int64_t(b) * n_heads + i) * d_latent;
  for (int c = threadIdx.x; c < d_latent; c += kProjThreads) os[c] = load_any(o, orow + c, o_dt);
  __syncthreads();
  for (int k = threadIdx.x; k < d_head; k += kProjThreads) {
    const int64_t wrow = (int64_t(i) * d_head + k) * d_latent;
    float acc = 0.f;
    for (int c = 0; c < d_latent; ++c) acc += load_any(w, wrow + c, w_dt) * os[c];
    store_any(out, int64_t(b) * n_heads * d_head + int64_t(i) * d_head + k, acc, out_dt);
  }
}

hipError_t launch_absorb_generic(const void* q, mla_dtype_t q_dt, const void* w, mla_dtype_t w_dt, void* out,
                                 mla_dtype_t o_dt, int batch, int n_heads, int d_head, int d_latent, hipStream_t st) {
  absorb_generic_kernel<<<dim3(batch, n_heads), kProjThreads, 0, st>>>(q, q_dt, w, w_dt, out, o_dt, n_heads, d_head,
                                                                      d_latent);
  return hipGetLastError();
}

hipError_t launch_outproj_generic(const void* o, mla_dtype_t o_dt, const void* w, mla_dtype_t w_dt, void* out,
                                  mla_dtype_t out_dt, int batch, int n_heads, int d_head, int d_latent,
                                  hipStream_t st) {
  outproj_generic_kernel<<<dim3(batch, n_heads), kProjThreads, 0, st>>>(o, o_dt, w, w_dt, out, out_dt, n_heads,
                                                                       d_head, d_latent);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// d_h = 128, d_c = 512 (V2 and V2-Lite), any head count, bf16, v_mfma_f32_32x32x16_bf16
// ---------------------------------------------------------------------------
constexpr int kPH = 128, kPL = 512;   // d_h, d_c

// absorb, computed transposed: q_lat^T [cols x batch] = W^T [cols x k] . q^T [k x batch].
// Workgroup (head i, 128-column block, 64-row batch tile): the W^UK block
// [128 k x 128 cols] (row pitch 288 B, so a 4-row transposing read hits
// distinct banks) and the query tile [64 rows x 128 k] (row pitch 272 B) are
// staged in LDS, with every global load issued before the first wait;
// wavefront w owns columns 32w..32w+31 and both 32-row halves of the batch
// tile, so each weight fragment feeds two MFMAs and every weight byte is read
// once for up to 64 sequences.  Query rows past the batch are clamped to the
// last row; their results are not stored.
constexpr int kWPitch = 144;  // bf16 elements per staged weight row
constexpr int kQPitch = 136;  // bf16 elements per staged query row

__global__ __launch_bounds__(256) void absorb_v2_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ w,
                                                        uint16_t* __restrict__ out, int batch, int n_heads) {
  __shared__ __attribute__((aligned(16))) uint16_t ws[kPH * kWPitch];
  __shared__ __attribute__((aligned(16))) uint16_t qs[64 * kQPitch];
  const int i = blockIdx.x, cb = blockIdx.y * 128, bt = blockIdx.z * 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  // W^UK[i*128 + k][cb .. cb+127]: 128 rows x 16 chunks of 16 B, 8 per thread;
  // q[bt + r][i][:]: 64 rows x 16 chunks, 4 per thread
  uint4 wv[8], qv[4];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int e = tid + 256 * r, k = e >> 4, ch = e & 15;
    wv[r] = *reinterpret_cast<const uint4*>(w + (int64_t(i) * kPH + k) * kPL + cb + ch * 8);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = tid + 256 * r, row = e >> 4, ch = e & 15;
    const int bq = min(bt + row, batch - 1);
    qv[r] = *reinterpret_cast<const uint4*>(q + (int64_t(bq) * n_heads + i) * kPH + ch * 8);
  }
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int e = tid + 256 * r, k = e >> 4, ch = e & 15;
    *reinterpret_cast<uint4*>(ws + k * kWPitch + ch * 8) = wv[r];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = tid + 256 * r, row = e >> 4, ch = e & 15;
    *reinterpret_cast<uint4*>(qs + row * kQPitch + ch * 8) = qv[r];
  }
  __syncthreads();
  // transposing read: lane (group g = lane/16, j = lane%16) -> row kbase + j/4, cols 16(g&1) + 4(j&3)
  const int g = lane >> 4, j = lane & 15;
  const uint16_t MLA_LDS* wl = (const uint16_t MLA_LDS*)ws;
  const uint16_t MLA_LDS* ql = (const uint16_t MLA_LDS*)qs + (lane & 31) * kQPitch + 8 * h;
  const int col_l = wave * 32 + 16 * (g & 1) + 4 * (j & 3);
  f32x16 acc0 = {}, acc1 = {};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const int r0 = 16 * kk + 8 * h + (j >> 2);
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 MLA_LDS*)(wl + r0 * kWPitch + col_l));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 MLA_LDS*)(wl + (r0 + 4) * kWPitch + col_l));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const bf16x8 b0 = *reinterpret_cast<const bf16x8 MLA_LDS*>(ql + 16 * kk);
    const bf16x8 b1 = *reinterpret_cast<const bf16x8 MLA_LDS*>(ql + 32 * kQPitch + 16 * kk);
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), b0, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), b1, acc1, 0, 0, 0);
  }
  // D[col][b]: lane has b = lane%32 (+32 for acc1), cols 8(r/4) + 4h + r%4 of the
  // wave's 32 columns.  The output tile (64 rows x 128 columns) goes through the
  // freed weight area so that every global store is part of a whole 256-byte
  // row piece: 16-byte chunk c of row r at slot c ^ (r & 15).
  __syncthreads();   // every wavefront is done with the weight tile
  uint16_t MLA_LDS* os = (uint16_t MLA_LDS*)ws;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const f32x16& acc = half ? acc1 : acc0;
    const int r = 32 * half + (lane & 31);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * q4 + e];
      const int c = wave * 4 + q4;
      *reinterpret_cast<bf16x4 MLA_LDS*>(os + r * 128 + ((c ^ (r & 15)) * 8) + 4 * h) = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = tid + 256 * j, r = e >> 4, c = e & 15;
    if (bt + r < batch)
      *reinterpret_cast<bf16x8*>(out + (int64_t(bt + r) * n_heads + i) * kPL + cb + c * 8) =
          *reinterpret_cast<const bf16x8 MLA_LDS*>(os + r * 128 + ((c ^ (r & 15)) * 8));
  }
}

// out proj, computed transposed: o^T [k x batch] = W^UV_i [k x c] . o_lat^T [c x batch].
// Both operands are read straight from global memory (c is contiguous in both).
// Workgroup (head i, 32-row batch tile); wavefront w owns rows k = 32w..32w+31.
// The 32 k-steps run in 4 groups of 8 whose operand loads are issued one group
// ahead; batch rows past the end are clamped to the last row and not stored.
template <bool OF32>
__global__ __launch_bounds__(256) void outproj_v2_kernel(const void* __restrict__ o_lat, const uint16_t* __restrict__ w,
                                                         uint16_t* __restrict__ out, int batch, int n_heads) {
  const int i = blockIdx.x, bt = blockIdx.y * 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const int krow = wave * 32 + (lane & 31);
  const int bq = bt + (lane & 31);
  const int bl = min(bq, batch - 1);
  const bf16x8* wr = reinterpret_cast<const bf16x8*>(w + (int64_t(i) * kPH + krow) * kPL) + h;
  const int64_t orow = (int64_t(bl) * n_heads + i) * kPL + 8 * h;
  constexpr int kG = 8;  // k-steps per group
  struct Ops { bf16x8 a[kG], b[kG]; };
  auto load = [&](int grp, Ops& o) {
#pragma unroll
    for (int t = 0; t < kG; ++t) {
      const int kk = grp * kG + t;
      o.a[t] = wr[2 * kk];
      if (OF32) {
        const float* op = static_cast<const float*>(o_lat) + orow + 16 * kk;
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(op), x1 = *reinterpret_cast<const f32x4*>(op + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) { o.b[t][e] = (__bf16)x0[e]; o.b[t][4 + e] = (__bf16)x1[e]; }
      } else {
        o.b[t] = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(o_lat) + orow + 16 * kk);
      }
    }
  };
  f32x16 acc = {};
  Ops cur, nxt;
  load(0, cur);
#pragma unroll
  for (int grp = 0; grp < kPL / 16 / kG; ++grp) {
    if (grp + 1 < kPL / 16 / kG) load(grp + 1, nxt);
    __builtin_amdgcn_sched_barrier(0);  // the next group's loads go out before this group's MFMAs
#pragma unroll
    for (int t = 0; t < kG; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[t], cur.b[t], acc, 0, 0, 0);
    cur = nxt;
  }
  if (bq < batch) {
    uint16_t* o = out + (int64_t(bq) * n_heads + i) * kPH + wave * 32 + 4 * h;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * q4 + e];
      *reinterpret_cast<bf16x4*>(o + 8 * q4) = v;
    }
  }
}

hipError_t launch_absorb_v2(const void* q, const void* w, void* out, int batch, int n_heads, hipStream_t st) {
  absorb_v2_kernel<<<dim3(n_heads, kPL / 128, ceil_div(batch, 64)), 256, 0, st>>>(static_cast<const uint16_t*>(q),
                                                              static_cast<const uint16_t*>(w),
                                                              static_cast<uint16_t*>(out), batch, n_heads);
  return hipGetLastError();
}

hipError_t launch_outproj_v2(const void* o_lat, bool o_f32, const void* w, void* out, int batch, int n_heads,
                             hipStream_t st) {
  dim3 grid(n_heads, ceil_div(batch, 32));
  if (o_f32)
    outproj_v2_kernel<true><<<grid, 256, 0, st>>>(o_lat, static_cast<const uint16_t*>(w), static_cast<uint16_t*>(out),
                                                  batch, n_heads);
  else
    outproj_v2_kernel<false><<<grid, 256, 0, st>>>(o_lat, static_cast<const uint16_t*>(w), static_cast<uint16_t*>(out),
                                                   batch, n_heads);
  return hipGetLastError();
}

}  // namespace mla
