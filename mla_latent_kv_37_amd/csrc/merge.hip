// Log-sum-exp merge of split partials.  Each split s of a sequence carries its
// own normalised output o_s and lse_s = log sum_{j in s} exp(score_j); the whole
// sequence has lse = log sum_s exp(lse_s) and o = sum_s exp(lse_s - lse) o_s.
// This is the exact softmax identity used for split-K attention; it is not
// printed on the pages.  One wavefront per (sequence, head).
#include "kernels.cuh"

namespace mla {


constexpr int kMergeWaves = 4;

__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(MergeArgs a) {
  const int b = blockIdx.x;
  const int head = blockIdx.y * kMergeWaves + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (head >= a.n_heads) return;
  const int T = a.seq_lens[b];
  const int64_t out_row = (int64_t(b) * a.n_heads + head);
  if (T <= 0) {
    for (int c = lane; c < a.d_latent; c += 64) store_any(a.o_lat, out_row * a.d_latent + c, 0.f, a.o_dt);
    if (lane == 0 && a.lse != nullptr) a.lse[out_row] = -INFINITY;
    return;
  }
  int first, count, stride;
  if (a.pp.mode == PART_FIXED) {
    count = ceil_div(T, a.pp.split_tokens);
    first = b * a.pp.fixed_slots;
    stride = 1;
  } else if (a.pp.mode == PART_BALANCED) {
    const int wf = a.meta[b], wl = a.meta[a.pp.batch + b];
    count = wl - wf + 1;
    first = wf + b;
    stride = 1;
  } else {
    return;
  }
  if (count <= 1) return;
  float M = -INFINITY;
  for (int s = 0; s < count; ++s) M = fmaxf(M, a.lse_part[int64_t(first + s * stride) * a.n_heads + head]);
  float Z = 0.f;
  for (int s = 0; s < count; ++s) Z += expf(a.lse_part[int64_t(first + s * stride) * a.n_heads + head] - M);
  const float invZ = 1.f / Z;
  for (int c = lane; c < a.d_latent; c += 64) {
    float acc = 0.f;
    for (int s = 0; s < count; ++s) {
      const int64_t slot = first + s * stride;
      const float w = expf(a.lse_part[slot * a.n_heads + head] - M);
      acc += w * a.o_part[(slot * a.n_heads + head) * a.d_latent + c];
    }
    store_any(a.o_lat, out_row * a.d_latent + c, acc * invZ, a.o_dt);
  }
  if (lane == 0 && a.lse != nullptr) a.lse[out_row] = M + logf(Z);
}

hipError_t launch_merge(const MergeArgs& a, int batch, hipStream_t st) {
  dim3 grid(batch, ceil_div(a.n_heads, kMergeWaves));
  merge_kernel<<<grid, 64 * kMergeWaves, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
