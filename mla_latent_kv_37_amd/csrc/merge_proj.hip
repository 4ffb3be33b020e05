// Split merge fused with the output projection: for head i and a tile of 16
// sequences, merge each sequence's split partials into its latent output
// o_lat[b, i, :] and multiply by W^UV_i in the same workgroup, so the merged
// rows go from registers to LDS to the matrix cores without a round trip
// through memory and without a second launch.
//
// Merge: the log-sum-exp identity of split-K attention (not printed on the
// pages): lse = log sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s, computed
// with exactly the operations and order of merge_kernel<8, true>, so o_lat and
// lse (written for split sequences, as mla_merge_splits does) are the same bits.
// Projection: o[b, i*d_h + k] = sum_c W^UV[i*d_h + k, c] o_lat[b, i, c]
// ([DeepSeek-V2 explainer] §2.2.2: W^UV applied after attention), as
// o^T [k x b] = W^UV_i [k x c] . o_lat^T [c x b] on v_mfma_f32_32x32x16_bf16.
//
// Workgroup of 16 wavefronts for R = 2, 4, 8, 16 or 32 sequences (the largest
// that still gives a workgroup per compute unit: the fewer workgroups read each
// head's W^UV, the less traffic; fewer rows for few heads, as in V2-Lite, where
// 8 rows took the kernel from 9.4 to 8.8 us, or few sequences: 4 long ones in
// 2-row tiles, 1.3% off their step).  Wavefront w = 4q + kb owns
// output rows k = 32kb..32kb+31 and the contraction quarter c = 128q..128q+127.
// Phase 0: the head's whole W^UV_i (128 rows x 1 KB) is copied into LDS by
// direct-to-LDS loads issued before anything else (8 rows per wavefront; chunk
// c of row k at slot c ^ (k & 15), so the fragment reads are conflict-free), so
// the weight and the split partials stream from memory at the same time
// (measured: 8.7% less time than loading the fragments into registers after
// the merge).  Phase 1: wavefront w merges tile rows w, w + 16 (lane = 8 columns): a row's
// split lse values are loaded lane-parallel together with its first 8 partials
// (two memory round trips for up to 8 splits); in a tile of at most 4 rows each
// row's parts (the association of kernels.h) go to four wavefronts and meet in
// the first through LDS.  The merged rows go into an LDS copy of the R rows
// (bf16, 16-byte chunk j of row r at slot j ^ (r & 15): conflict-free for the
// row writes and the MFMA operand reads).  Phase 2: after the weight loads are
// waited for, 8 MFMAs per wavefront (for
// R < 32 the 32-wide batch operand repeats the R rows and only the first R
// columns are stored); quarters 1-3 pass their fp32 partial products through
// LDS (the weight area, once every wavefront has read its fragments) and
// quarter 0 adds them in order and rounds to bf16 into LDS, from where the
// output rows are stored whole.
#include "kernels.h"

namespace mla {

constexpr int kMPH = 128, kMPL = 512;   // d_h, d_c
constexpr int kMPWaves = 16;
constexpr int kXchRow = 64 * 8 * 4 + 64 * 4;   // part exchange slot of one row (bytes)

__device__ __forceinline__ uint32_t mp_row_off(int r, int chunk) {
  return uint32_t(r * 1024 + ((chunk ^ (r & 15)) * 16));
}

// Split slots of row b: [first, first + count); count 0 for an empty sequence.
__device__ __forceinline__ void mp_splits(const MergeArgs& a, int b, int& first, int& count) {
  const int T = seq_len_of(load_const(a.seq_lens, seq_len_index(b, a.pp)), b, a.pp);
  first = 0;
  count = T > 0 ? 1 : 0;
  if (T <= 0) return;
  if (a.pp.mode == PART_FIXED) {
    count = ceil_div(T, a.pp.split_tokens);
    first = b * a.pp.fixed_slots;
  } else if (a.pp.mode == PART_BALANCED) {
    const int wf = load_const(a.meta, b), wl = load_const(a.meta, int64_t(a.pp.batch) + b);
    count = wl - wf + 1;
    first = wf + b;
  }
}

// A wavefront with no row of its own (tiles with fewer rows than wavefronts)
// reads split partials 8 + j, 8 + j + nh, ... of row b (the owner's first 8 go
// out with its lse loads) and discards them, so that the owner's later 8-split
// chunks find them in L2.  The owner's arithmetic is unchanged.
__device__ __forceinline__ void mp_touch_row(const MergeArgs& a, int b, int head, int lane, int j, int nh) {
  int first, count;
  mp_splits(a, b, first, count);
  if (count <= 8) return;
  const int64_t stride = int64_t(a.n_heads) * kMPL;
  const uint16_t* const src0 = static_cast<const uint16_t*>(a.o_part) + (int64_t(first) * a.n_heads + head) * kMPL + lane * 8;
  uint32_t sink = 0;
  int n = 0;
  for (int s = 8 + j; s < count; s += nh) {
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(src0 + s * stride);
    sink ^= __builtin_bit_cast(uint32_t, __builtin_shufflevector(x, x, 0, 1));
    if (++n == 8) {
      asm volatile("" : : "v"(sink));
      n = 0;
    }
  }
  asm volatile("" : : "v"(sink));
}

// Sums over the parts [q0, q1) of a row's splits (merge_parts of kernels.h),
// 8 columns per lane: each part from zero in split order, the parts added in
// order, the weight of split s being exp(lse_s - M).  The first chunk of 8
// partials goes out with the lse loads; M, the maximum over all of the row's
// splits, is exact in any order.
struct MpPart {
  float Z;
  float acc[8];
};

__device__ __forceinline__ MpPart mp_sum(const MergeArgs& a, int head, int lane, int first, int count, int q0, int q1,
                                         float& M_out) {
  const int P = merge_parts(count), L = ceil_div(count, P);
  const float* const lsp = a.lse_part + int64_t(first) * a.n_heads + head;
  // lse_s of split s sits in lane s (splits beyond 64 are read per split below)
  const float lv = lane < count ? lsp[int64_t(lane) * a.n_heads] : -INFINITY;
  const int64_t stride = int64_t(a.n_heads) * kMPL;
  const uint16_t* const src0 = static_cast<const uint16_t*>(a.o_part) + (int64_t(first) * a.n_heads + head) * kMPL + lane * 8;
  const int sb = q0 * L, se = min(count, q1 * L);
  bf16x8 x8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (sb + j < se) x8[j] = *reinterpret_cast<const bf16x8*>(src0 + (sb + j) * stride);
  float M = lv;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  for (int s = 64; s < count; ++s) M = fmaxf(M, lsp[int64_t(s) * a.n_heads]);
  M_out = M;
  auto lse_of = [&](int s) {
    return s < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), s)) : lsp[int64_t(s) * a.n_heads];
  };
  MpPart tot;
  for (int q = q0; q < q1; ++q) {
    const int s0 = q * L, s1 = min(count, s0 + L);
    float Zq = 0.f, accq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) accq[e] = 0.f;
    for (int c0 = s0; c0 < s1; c0 += 8) {
      if (c0 != sb) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (c0 + j < s1) x8[j] = *reinterpret_cast<const bf16x8*>(src0 + (c0 + j) * stride);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (c0 + j < s1) {
          const float w = __expf(lse_of(c0 + j) - M);
          Zq += w;
#pragma unroll
          for (int e = 0; e < 8; ++e) accq[e] += w * float(x8[j][e]);
        }
      }
    }
    // (the first part is taken as it is: adding it to zero could flip the sign of a zero)
    tot.Z = q == q0 ? Zq : tot.Z + Zq;
#pragma unroll
    for (int e = 0; e < 8; ++e) tot.acc[e] = q == q0 ? accq[e] : tot.acc[e] + accq[e];
  }
  return tot;
}

// The merged row from its sums: o_lat and lse written (for a split sequence),
// the bf16 row returned
__device__ __forceinline__ bf16x8 mp_finish(const MergeArgs& a, int b, int head, int lane, const MpPart& t, float M) {
  const int64_t out_row = int64_t(b) * a.n_heads + head;
  const float invZ = 1.f / t.Z;
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (__bf16)(t.acc[e] * invZ);
  *reinterpret_cast<bf16x8*>(static_cast<uint16_t*>(a.o_lat) + out_row * kMPL + lane * 8) = o;
  if (lane == 0 && a.lse != nullptr) a.lse[out_row] = M + __logf(t.Z);
  return o;
}

// A row of at most kMergeOneSplits splits (one part: the splits in order) by
// one wavefront, 8 columns per lane; writes o_lat / lse for sequences that
// were split or are empty, like merge_kernel.  (Kept apart from mp_sum: the
// common short rows run measurably faster through this straight-line form.)
__device__ __forceinline__ bf16x8 mp_merge_row_short(const MergeArgs& a, int b, int head, int lane, int first,
                                                     int count) {
  const int64_t out_row = int64_t(b) * a.n_heads + head;
  uint16_t* const orow = static_cast<uint16_t*>(a.o_lat) + out_row * kMPL + lane * 8;
  bf16x8 o = {};
  if (count == 0) {
    *reinterpret_cast<bf16x8*>(orow) = o;
    if (lane == 0 && a.lse != nullptr) a.lse[out_row] = -INFINITY;
    return o;
  }
  // one work item covered the sequence: mla_decode wrote the final row
  if (count <= 1) return *reinterpret_cast<const bf16x8*>(orow);
  // lse_s of split s sits in lane s (splits beyond 64 are read per split below);
  // the maximum is exact in any order, so M is merge_kernel's M
  const float* const lsp = a.lse_part + int64_t(first) * a.n_heads + head;
  const float lv = lane < count ? lsp[int64_t(lane) * a.n_heads] : -INFINITY;
  const int64_t stride = int64_t(a.n_heads) * kMPL;
  const uint16_t* const src0 = static_cast<const uint16_t*>(a.o_part) + (int64_t(first) * a.n_heads + head) * kMPL + lane * 8;
  // the first 8 partials go out with the lse loads
  bf16x8 x8[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (j < count) x8[j] = *reinterpret_cast<const bf16x8*>(src0 + j * stride);
  float M = lv;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  for (int s = 64; s < count; ++s) M = fmaxf(M, lsp[int64_t(s) * a.n_heads]);
  auto lse_of = [&](int s) {
    return s < 64 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), s)) : lsp[int64_t(s) * a.n_heads];
  };
  // accumulate in split order with merge_kernel's expressions
  float Z = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j < count) {
      const float w = __expf(lse_of(j) - M);
      Z += w;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += w * float(x8[j][e]);
    }
  }
  for (int s0 = 8; s0 < count; s0 += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (s0 + j < count) x8[j] = *reinterpret_cast<const bf16x8*>(src0 + (s0 + j) * stride);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (s0 + j < count) {
        const float w = __expf(lse_of(s0 + j) - M);
        Z += w;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += w * float(x8[j][e]);
      }
    }
  }
  const float invZ = 1.f / Z;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (__bf16)(acc[e] * invZ);
  *reinterpret_cast<bf16x8*>(orow) = o;
  if (lane == 0 && a.lse != nullptr) a.lse[out_row] = M + __logf(Z);
  return o;
}

// Merged (or single-split) row b of head `head` by one wavefront, every part
// in order; writes o_lat / lse for sequences that were split or are empty,
// like merge_kernel.
__device__ __forceinline__ bf16x8 mp_merge_row(const MergeArgs& a, int b, int head, int lane) {
  int first, count;
  mp_splits(a, b, first, count);
  if (count <= kMergeOneSplits) return mp_merge_row_short(a, b, head, lane, first, count);
  float M;
  const MpPart t = mp_sum(a, head, lane, first, count, 0, kMergeParts, M);
  return mp_finish(a, b, head, lane, t, M);
}

template <int R>
__global__ __launch_bounds__(64 * kMPWaves) void merge_proj_kernel(MergeArgs a, const uint16_t* __restrict__ w,
                                                                   uint16_t* __restrict__ out, int batch) {
  __shared__ __attribute__((aligned(1024))) char wl[kMPH * 1024];
  __shared__ __attribute__((aligned(1024))) char rows[R * 1024];
  // part exchange (tiles of at most kMPWaves / kMergeParts rows): per row, 64
  // lanes x 8 fp32 sums, then 64 lanes x Z
  constexpr bool kParts = R <= 16;
  __shared__ __attribute__((aligned(16))) char xch[kParts ? (kMPWaves / kMergeParts) * kXchRow : 16];
  float MLA_LDS* const red = (float MLA_LDS*)(uintptr_t)uint32_t(reinterpret_cast<uintptr_t>(wl));
  const int i = blockIdx.x, bt = blockIdx.y * R;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5;
  const int kb = wave & 3, cq = wave >> 2;
  // W^UV_i into LDS: wavefront w copies rows 8w..8w+7, one 1 KB row per load;
  // lane l of row k's load reads chunk l ^ (k & 15), which lands in slot l.
  // Untracked by the compiler (inline assembly): waited for before the barrier
  // that precedes the fragment reads.
  const uint32_t w_lds = uint32_t(reinterpret_cast<uintptr_t>(wl));
  {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const uint64_t base = reinterpret_cast<uint64_t>(w + int64_t(i) * kMPH * kMPL);
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    i32x4 rsrc;
    rsrc[0] = uniform(int(uint32_t(base)));
    rsrc[1] = uniform(int(uint32_t(base >> 32) & 0xFFFFu));
    rsrc[2] = kMPH * kMPL * 2;
    rsrc[3] = int(0x00020000u);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = 8 * wave + j;
      const int voff = (ln ^ (k & 15)) * 16;
      const int m0 = uniform(int(w_lds + uint32_t(k * 1024)));
      const int soff = uniform(k * 1024);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                   : : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
    }
  }
  const uint32_t rows_lds = uint32_t(reinterpret_cast<uintptr_t>(rows));
  const int nvalid = min(R, batch - bt);
  if (kParts && nvalid * kMergeParts <= kMPWaves) {
    // Few rows: wavefront w takes part w / nvalid of row w % nvalid (rows of
    // more than kMergeOneSplits splits are added in kMergeParts parts), and
    // parts 1.. reach the row's first wavefront through the exchange area one
    // at a time, so that it adds them in order.  Every wavefront passes the
    // same barriers.
    const uint32_t xch_lds = uint32_t(reinterpret_cast<uintptr_t>(xch));
    const int r = wave % nvalid, q = wave / nvalid, b = bt + r;
    int first = 0, count = 0;
    if (q < kMergeParts) mp_splits(a, b, first, count);
    const bool mine = q < kMergeParts && count > kMergeOneSplits;   // rows of several parts
    MpPart t{};
    float M = 0.f;
    if (mine) t = mp_sum(a, i, lane, first, count, q, q + 1, M);
    const uint32_t xa = xch_lds + uint32_t(r * kXchRow + lane * 32), xz = xch_lds + uint32_t(r * kXchRow + 2048 + lane * 4);
    for (int qq = 1; qq < kMergeParts; ++qq) {
      if (mine && q == qq) {
        *reinterpret_cast<f32x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)xa) = f32x4{t.acc[0], t.acc[1], t.acc[2], t.acc[3]};
        *reinterpret_cast<f32x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(xa + 16)) = f32x4{t.acc[4], t.acc[5], t.acc[6], t.acc[7]};
        *reinterpret_cast<float MLA_LDS*>((char MLA_LDS*)(uintptr_t)xz) = t.Z;
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();
      if (mine && q == 0) {
        const f32x4 u0 = *reinterpret_cast<const f32x4 MLA_LDS*>((const char MLA_LDS*)(uintptr_t)xa);
        const f32x4 u1 = *reinterpret_cast<const f32x4 MLA_LDS*>((const char MLA_LDS*)(uintptr_t)(xa + 16));
        t.Z += *reinterpret_cast<const float MLA_LDS*>((const char MLA_LDS*)(uintptr_t)xz);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          t.acc[e] += u0[e];
          t.acc[4 + e] += u1[e];
        }
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();   // the slot is read before the next part overwrites it
    }
    if (q == 0) {
      const bf16x8 o = mine ? mp_finish(a, b, i, lane, t, M) : mp_merge_row_short(a, b, i, lane, first, count);
      *reinterpret_cast<bf16x8 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(rows_lds + mp_row_off(r, lane))) = o;
    }
#pragma unroll
    for (int rz = wave; rz < R; rz += kMPWaves)
      if (rz >= nvalid)
        *reinterpret_cast<bf16x8 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(rows_lds + mp_row_off(rz, lane))) = bf16x8{};
  } else {
    if (nvalid < kMPWaves && wave >= nvalid) {
      const int hw = wave - nvalid, r = hw % nvalid;
      const int nh = (kMPWaves - nvalid - r + nvalid - 1) / nvalid;
      mp_touch_row(a, bt + r, i, lane, hw / nvalid, nh);
    }
#pragma unroll
    for (int r = wave; r < R; r += kMPWaves) {
      const int b = bt + r;
      const bf16x8 o = b < batch ? mp_merge_row(a, b, i, lane) : bf16x8{};
      *reinterpret_cast<bf16x8 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(rows_lds + mp_row_off(r, lane))) = o;
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  __syncthreads();
  // W^UV fragments of this wavefront: row 32kb + (lane & 31), columns 128cq + 16kk + 8h
  bf16x8 wa[8];
  {
    const int kr = 32 * kb + (lane & 31);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int c = 16 * cq + 2 * kk + h;
      wa[kk] = *reinterpret_cast<const bf16x8 MLA_LDS*>(
          (const char MLA_LDS*)(uintptr_t)(w_lds + uint32_t(kr * 1024 + ((c ^ (kr & 15)) * 16))));
    }
  }
  // o_lat^T fragment of k-step kk: row lane % R, columns 128cq + 16kk + 8h (chunk 16cq + 2kk + h)
  f32x16 acc = {};
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 bo = *reinterpret_cast<const bf16x8 MLA_LDS*>(
        (const char MLA_LDS*)(uintptr_t)(rows_lds + mp_row_off(lane & (R - 1), 16 * cq + 2 * kk + h)));
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[kk], bo, acc, 0, 0, 0);
  }
  __syncthreads();   // every wavefront has read its weight fragments (red reuses that area)
  // red: quarter q (1..3) of row block kb at (4(q-1) + kb) * 1024 floats, [q4][lane] f32x4
  if (cq > 0) {
    float MLA_LDS* dst = (float MLA_LDS*)red + (4 * (cq - 1) + kb) * 1024 + lane * 4;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<f32x4 MLA_LDS*>(dst + q4 * 256) =
          f32x4{acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]};
  }
  __syncthreads();
  if (cq == 0) {
#pragma unroll
    for (int q = 1; q < 4; ++q) {
      const float MLA_LDS* src = (const float MLA_LDS*)red + (4 * (q - 1) + kb) * 1024 + lane * 4;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = *reinterpret_cast<const f32x4 MLA_LDS*>(src + q4 * 256);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[4 * q4 + e] += v[e];
      }
    }
    // D[k][b]: lane holds b = lane & 31 (for R = 16 columns 16-31 repeat 0-15),
    // k = 8(e/4) + 4h + e%4 of the row block.  Staged in the (no longer read)
    // row area as [b][128 k] bf16, 16-byte chunk c of row b at slot c ^ (b & 15),
    // so that the global stores below are whole 256-byte rows.
    const int b = lane & 31;
    if (b < R) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[4 * q4 + e];
        const int c = 4 * kb + q4;
        *reinterpret_cast<bf16x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(rows_lds + uint32_t(b * 256 + ((c ^ (b & 15)) * 16) + 8 * h))) = v;
      }
    }
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < R * 16) {
    const int r = t >> 4, c = t & 15;
    if (bt + r < batch)
      *reinterpret_cast<bf16x8*>(out + (int64_t(bt + r) * a.n_heads + i) * kMPH + c * 8) =
          *reinterpret_cast<const bf16x8 MLA_LDS*>((const char MLA_LDS*)(uintptr_t)(rows_lds + uint32_t(r * 256 + ((c ^ (r & 15)) * 16))));
  }
}

hipError_t launch_merge_proj(const MergeArgs& a, const void* w_uv, void* o_heads, int batch, hipStream_t st) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidDevice;
  const uint16_t* w = static_cast<const uint16_t*>(w_uv);
  uint16_t* out = static_cast<uint16_t*>(o_heads);
  // the largest tile that still gives a workgroup per compute unit (fewer
  // workgroups read each head's W^UV): 32, 16, 8, 4 or 2 rows
  auto fits = [&](int r) { return int64_t(a.n_heads) * ceil_div(batch, r) >= cus; };
  if (fits(32)) merge_proj_kernel<32><<<dim3(a.n_heads, ceil_div(batch, 32)), 64 * kMPWaves, 0, st>>>(a, w, out, batch);
  else if (fits(16)) merge_proj_kernel<16><<<dim3(a.n_heads, ceil_div(batch, 16)), 64 * kMPWaves, 0, st>>>(a, w, out, batch);
  else if (fits(8)) merge_proj_kernel<8><<<dim3(a.n_heads, ceil_div(batch, 8)), 64 * kMPWaves, 0, st>>>(a, w, out, batch);
  else if (fits(4)) merge_proj_kernel<4><<<dim3(a.n_heads, ceil_div(batch, 4)), 64 * kMPWaves, 0, st>>>(a, w, out, batch);
  else merge_proj_kernel<2><<<dim3(a.n_heads, ceil_div(batch, 2)), 64 * kMPWaves, 0, st>>>(a, w, out, batch);
  return hipGetLastError();
}

}  // namespace mla
