// Log-sum-exp merge of split partials.  Each split s of a sequence carries its
// own normalised output o_s and lse_s = log sum_{j in s} exp(score_j); the whole
// sequence has lse = log sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s.
// This is the exact softmax identity used for split-K attention; it is not
// printed on the pages.  Partials are stored in the output dtype.  One
// wavefront per (sequence, head); each lane owns d_c/64 consecutive columns
// (8 for d_c = 512: one 16-byte load per partial in bf16, two in fp32).
#include "kernels.h"

namespace mla {

constexpr int kMergeWaves = 4;

// COLS: columns per lane when d_c == 64 * COLS (vector path), 0 = any d_c;
// BF16: partials (and output) in bf16, else fp32 (vector path only)
template <int COLS, bool BF16>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(MergeArgs a) {
  const int b = blockIdx.x;
  const int head = blockIdx.y * kMergeWaves + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (head >= a.n_heads) return;
  const int T = seq_len_of(load_const(a.seq_lens, seq_len_index(b, a.pp)), b, a.pp);
  const int64_t out_row = (int64_t(b) * a.n_heads + head);
  if (T <= 0) {
    for (int c = lane; c < a.d_latent; c += 64) store_any(a.o_lat, out_row * a.d_latent + c, 0.f, a.o_dt);
    if (lane == 0 && a.lse != nullptr) a.lse[out_row] = -INFINITY;
    return;
  }
  int first, count;
  if (a.pp.mode == PART_FIXED) {
    count = ceil_div(T, a.pp.split_tokens);
    first = b * a.pp.fixed_slots;
  } else if (a.pp.mode == PART_BALANCED) {
    const int wf = a.meta[b], wl = a.meta[a.pp.batch + b];
    count = wl - wf + 1;
    first = wf + b;
  } else {
    return;
  }
  if (count <= 1) return;
  // the partials' loads are independent: unrolled so that several are in flight
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < count; ++s) M = fmaxf(M, a.lse_part[int64_t(first + s) * a.n_heads + head]);
  float Z = 0.f;
  if (COLS > 0) {
    float acc[COLS > 0 ? COLS : 1];
#pragma unroll
    for (int e = 0; e < COLS; ++e) acc[e] = 0.f;
    // partial s's columns of this lane, as floats
    const int64_t stride = int64_t(a.n_heads) * a.d_latent;
    const int64_t src0 = (int64_t(first) * a.n_heads + head) * a.d_latent + lane * COLS;
    auto load_cols = [&](int s, float* x) {
      const int64_t src = src0 + s * stride;
      if (BF16 && COLS == 8) {
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(a.o_part) + src);
#pragma unroll
        for (int e = 0; e < COLS; ++e) x[e] = float(v[e % 8]);
      } else if (!BF16) {
        const f32x4* x4 = reinterpret_cast<const f32x4*>(static_cast<const float*>(a.o_part) + src);
#pragma unroll
        for (int v = 0; v < COLS / 4; ++v) {
          const f32x4 y = x4[v];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * v + e] = y[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < COLS; ++e) x[e] = load_any(a.o_part, src + e, a.o_dt);
      }
    };
    // the parts of merge_parts(count), each from zero, added in order
    const int P = merge_parts(count), L = ceil_div(count, P);
    for (int q = 0; q < P; ++q) {
      const int s1 = min(count, (q + 1) * L);
      float Zq = 0.f, accq[COLS > 0 ? COLS : 1];
#pragma unroll
      for (int e = 0; e < COLS; ++e) accq[e] = 0.f;
      // four partials per step: their loads are issued together
      int s = q * L;
      for (; s + 4 <= s1; s += 4) {
        float l[4], x[4][COLS > 0 ? COLS : 1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          l[j] = a.lse_part[int64_t(first + s + j) * a.n_heads + head];
          load_cols(s + j, x[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float w = __expf(l[j] - M);
          Zq += w;
#pragma unroll
          for (int e = 0; e < COLS; ++e) accq[e] += w * x[j][e];
        }
      }
      for (; s < s1; ++s) {
        float x[COLS > 0 ? COLS : 1];
        const float w = __expf(a.lse_part[int64_t(first + s) * a.n_heads + head] - M);
        load_cols(s, x);
        Zq += w;
#pragma unroll
        for (int e = 0; e < COLS; ++e) accq[e] += w * x[e];
      }
      // (the first part is taken as it is: adding it to zero could flip the
      // sign of a zero)
      Z = q == 0 ? Zq : Z + Zq;
#pragma unroll
      for (int e = 0; e < COLS; ++e) acc[e] = q == 0 ? accq[e] : acc[e] + accq[e];
    }
    const float invZ = 1.f / Z;
    const int64_t base = out_row * a.d_latent + lane * COLS;
    if (BF16) {
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < COLS; ++e) o[e % 8] = (__bf16)(acc[e] * invZ);
      if (COLS == 8) *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(a.o_lat) + base) = o;
      else
        for (int e = 0; e < COLS; ++e) store_any(a.o_lat, base + e, acc[e] * invZ, a.o_dt);
    } else {
#pragma unroll
      for (int e = 0; e < COLS; ++e) static_cast<float*>(a.o_lat)[base + e] = acc[e] * invZ;
    }
  } else {
    for (int s = 0; s < count; ++s) Z += __expf(a.lse_part[int64_t(first + s) * a.n_heads + head] - M);
    const float invZ = 1.f / Z;
    for (int c = lane; c < a.d_latent; c += 64) {
      float acc = 0.f;
      for (int s = 0; s < count; ++s) {
        const int64_t slot = first + s;
        acc += __expf(a.lse_part[slot * a.n_heads + head] - M) * load_any(a.o_part, (slot * a.n_heads + head) * a.d_latent + c, a.o_dt);
      }
      store_any(a.o_lat, out_row * a.d_latent + c, acc * invZ, a.o_dt);
    }
  }
  if (lane == 0 && a.lse != nullptr) a.lse[out_row] = M + __logf(Z);
}

hipError_t launch_merge(const MergeArgs& a, int batch, hipStream_t st) {
  dim3 grid(batch, ceil_div(a.n_heads, kMergeWaves));
  if (a.d_latent == 512 && a.o_dt == MLA_BF16) merge_kernel<8, true><<<grid, 64 * kMergeWaves, 0, st>>>(a);
  else if (a.d_latent == 512 && a.o_dt == MLA_F32) merge_kernel<8, false><<<grid, 64 * kMergeWaves, 0, st>>>(a);
  else merge_kernel<0, false><<<grid, 64 * kMergeWaves, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
