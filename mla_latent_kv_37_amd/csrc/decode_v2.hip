// MLA decode at DeepSeek-V2 shapes on gfx950 matrix cores.
//
// Shapes: n_h = 128 heads, latent d_c = 512, RoPE key d_h^R = 64, so every cached
// token is one 576-wide row [c^KV | k^R] ([DeepSeek-V2 explainer] §2.2.2, §3.1.1).
// With W^UK absorbed into the query, all heads score against the same row and
// the values are the first 512 columns of that row, so per sequence the decode
// is two dense contractions, both on v_mfma_f32_32x32x16_bf16:
//   S^T [tokens x heads] = K [tokens x 576] . Q^T [576 x heads]
//   O^T [512 x heads]   += V^T [512 x tokens] . P^T [tokens x heads]
//
// Work decomposition.  A work item is a list of (sequence, token range)
// segments (partition.cuh).  Two workgroups serve each work item, one per half
// of the heads (64 heads each); their ids are spaced by 8 so both land on the
// same XCD and the second read of every cache line is served by that XCD's L2.
// Inside a workgroup the 4 wavefronts form two pairs; a pair owns 32 heads.
// Wavefront (pair p, half d) multiplies the row dims [288d, 288d+288) for the
// scores and owns output columns [256d, 256d+256).  The pair adds its two fp32
// partial score blocks through LDS, both members run the (identical) softmax,
// and each accumulates its 256 columns.  Per wavefront that is 72 registers of
// query and 128 of accumulator, and every staged byte is read from LDS once per
// head group.
//
// Data movement.  32-token tiles (36,864 B) are staged in LDS, triple-buffered,
// by buffer loads that write LDS directly (16 B per lane).  The descriptor's
// size is the tile's valid bytes, so rows past the end of a sequence read as
// zeros (their scores are masked to -inf, and a zero value row keeps 0 * v
// finite even when the slot holds NaN).  LDS tile layout is chunk-major: the
// 16-byte chunk c (8 bf16) of token row t sits at c*512 + (t ^ 4*(c&1))*16.  A
// load instruction fills two chunk columns, a K fragment (32 rows of one chunk)
// is 512 contiguous bytes, the row XOR on odd chunks puts the two chunks a
// transposing V read touches (4 rows x 32 B) on disjoint banks, and every LDS
// address is a per-lane base plus an immediate.
//
// Softmax.  Scores are kept in the log2 domain (scale * log2 e folded into one
// FMA).  The running max is raised lazily: the accumulators are rescaled only
// when a head's max grows by more than 8 (a factor 256), which keeps every
// probability <= 256 in bf16 and fp32 and skips almost every rescale.
#include "kernels.cuh"

namespace mla {

constexpr int kV2Heads = 128, kV2Lat = 512, kV2Rope = 64, kV2Row = 576, kV2Page = 64;
constexpr int kRowBytes = kV2Row * 2;                 // 1152
constexpr int kTileTok = 32;
constexpr int kTileBytes = kTileTok * kRowBytes;      // 36864
constexpr int kNumBuf = 3;
constexpr int kXsOffset = kNumBuf * kTileBytes;       // partial-score exchange area
constexpr int kLdsBytes = kXsOffset + 4 * 4096;       // 126976
constexpr int kDecThreads = 256;
constexpr int kLoadsPerWave = 9;                      // 36 two-column loads per tile
constexpr float kRescaleSlack = 8.0f;                 // log2 units
constexpr uint32_t kBufferFlags = 0x00020000u;        // raw buffer, 32-bit data format


// Direct-to-LDS loads of one 32-token tile.  Wavefront w issues column pairs
// 9w .. 9w+8; `voff_lane` = ((lane&31) ^ 4*(lane>>5)) * 1152 + (lane>>5) * 16.
__device__ __forceinline__ void issue_tile(const char* tile_ptr, int valid, char MLA_LDS* buf, int wave, int voff_lane) {
  __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(tile_ptr), 0, valid * kRowBytes, kBufferFlags);
  // The column offset is a scalar offset: with or without it in the hardware
  // range check, global row t is in range exactly when t < valid.
#pragma unroll
  for (int j = 0; j < kLoadsPerWave; ++j) {
    const int q = wave * kLoadsPerWave + j;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, buf + q * 1024, 16, voff_lane, q * 32, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 lds_read_b128(const char MLA_LDS* p) {
  return *reinterpret_cast<const bf16x8 MLA_LDS*>(p);
}

__device__ __forceinline__ bf16x8 lds_read_tr_pair(const char MLA_LDS* p0, const char MLA_LDS* p1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 MLA_LDS*)(p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 MLA_LDS*)(p1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& p, int base) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[base + i];
  return r;
}

__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_v2_bf16_kernel(V2DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kLdsBytes];
  char MLA_LDS* smem = (char MLA_LDS*)smem_raw;
  // workgroup id -> (work item, head half); ids 16k + x and 16k + 8 + x share an XCD
  const int bid = blockIdx.x;
  const int item = (bid >> 4) * 8 + (bid & 7);
  const int hh = (bid >> 3) & 1;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, h = lane >> 5;
  const int pair = wave & 1, dh = wave >> 1;
  const int head = hh * 64 + pair * 32 + (lane & 31);
  if (item >= a.n_items) return;

  // per-lane address parts
  const int voff_lane = ((lane & 31) ^ (4 * h)) * kRowBytes + h * 16;
  const int kbase = (36 * dh + h) * 512 + ((lane & 31) ^ (4 * h)) * 16;   // + kk*1024
  int vbase;                                                                // + mt*2048 + ks*256 (+128)
  {
    const int g = lane >> 4, j = lane & 15, bsel = (j >> 1) & 1;
    vbase = (32 * dh + 2 * (g & 1) + bsel) * 512 + (((4 * h + (j >> 2)) ^ (4 * bsel)) * 16) + (j & 1) * 8;
  }
  char MLA_LDS* xs_mine = smem + kXsOffset + wave * 4096 + lane * 16;
  const char MLA_LDS* xs_peer = smem + kXsOffset + (wave ^ 2) * 4096 + lane * 16;
  int cur = 0;  // buffer of the next tile to issue; advances across segments

  SegmentIter it;
  it.init(a.pp, a.seq_lens, item, reinterpret_cast<int*>(smem_raw), a.meta);
  Segment sg;
  while (it.next(sg)) {
    const int b = uniform(sg.b);
    const int t0 = uniform(sg.t0), t1 = uniform(sg.t1);
    // query slice: dims 288*dh + 16*kk + 8*h .. +8 of head `head` (B operand of S^T = K Q^T)
    bf16x8 qf[18];
    {
      const uint16_t* ql = a.q_lat + (int64_t(b) * kV2Heads + head) * kV2Lat;
      const uint16_t* qp = a.q_pe + (int64_t(b) * kV2Heads + head) * kV2Rope;
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        const int d = 288 * dh + 16 * kk + 8 * h;
        qf[kk] = *reinterpret_cast<const bf16x8*>(d < kV2Lat ? ql + d : qp + (d - kV2Lat));
      }
    }
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
    float m_run = -INFINITY, lsum = 0.f;

    const int32_t* bt = a.block_table + int64_t(b) * a.max_pages;
    const char* kv = static_cast<const char*>(a.kv);
    const int ntiles = ceil_div(t1 - t0, kTileTok);
    auto tile_ptr = [&](int k) -> const char* {
      const int tok = t0 + k * kTileTok;
      return kv + int64_t(uniform(bt[tok / kV2Page])) * (kV2Page * kRowBytes) + (tok % kV2Page) * kRowBytes;
    };
    issue_tile(tile_ptr(0), min(kTileTok, t1 - t0), smem + cur * kTileBytes, wave, voff_lane);
    if (ntiles > 1)
      issue_tile(tile_ptr(1), min(kTileTok, t1 - t0 - kTileTok), smem + ((cur + 1) % kNumBuf) * kTileBytes, wave,
                 voff_lane);

    for (int k = 0; k < ntiles; ++k) {
      const int valid = min(kTileTok, t1 - t0 - k * kTileTok);
      if (k + 1 < ntiles) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (k + 2 < ntiles)
        issue_tile(tile_ptr(k + 2), min(kTileTok, t1 - t0 - (k + 2) * kTileTok),
                   smem + ((cur + 2) % kNumBuf) * kTileBytes, wave, voff_lane);
      const char MLA_LDS* tile = smem + cur * kTileBytes;

      // ---- partial S^T over this wavefront's 288 row dims (18 k-steps)
      f32x16 s = {};
      {
        const char MLA_LDS* kp = tile + kbase;
        bf16x8 kf[2][2];
        kf[0][0] = lds_read_b128(kp);
        kf[0][1] = lds_read_b128(kp + 1024);
#pragma unroll
        for (int grp = 0; grp < 9; ++grp) {
          if (grp + 1 < 9) {
            kf[(grp + 1) & 1][0] = lds_read_b128(kp + (2 * grp + 2) * 1024);
            kf[(grp + 1) & 1][1] = lds_read_b128(kp + (2 * grp + 3) * 1024);
          }
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[grp & 1][0], qf[2 * grp], s, 0, 0, 0);
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[grp & 1][1], qf[2 * grp + 1], s, 0, 0, 0);
        }
      }
      // ---- exchange partial scores within the pair
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v = {s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
        *reinterpret_cast<f32x4 MLA_LDS*>(xs_mine + q4 * 1024) = v;
      }
      __syncthreads();
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = *reinterpret_cast<const f32x4 MLA_LDS*>(xs_peer + q4 * 1024);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * q4 + e] += v[e];
      }
      // ---- online softmax (lane: head `head`, 16 of the tile's tokens; lane^32 the other 16)
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tok = 8 * (r >> 2) + 4 * h + (r & 3);
        if (tok >= valid) s[r] = -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      if (__any(m_new > m_run + kRescaleSlack)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= alpha;
        lsum *= alpha;
        m_run = m_new;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, -m_run));
        lsum += s[r];
      }
      const bf16x8 pk0 = pack8(s, 0), pk1 = pack8(s, 8);
      // ---- O^T += V^T . P^T over this wavefront's 256 columns
      {
        const char MLA_LDS* vp = tile + vbase;
        bf16x8 vf[2][2];
        vf[0][0] = lds_read_tr_pair(vp, vp + 128);
        vf[0][1] = lds_read_tr_pair(vp + 256, vp + 384);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          if (mt + 1 < 8) {
            const char MLA_LDS* q = vp + (mt + 1) * 2048;
            vf[(mt + 1) & 1][0] = lds_read_tr_pair(q, q + 128);
            vf[(mt + 1) & 1][1] = lds_read_tr_pair(q + 256, q + 384);
          }
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[mt & 1][0], pk0, acc[mt], 0, 0, 0);
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[mt & 1][1], pk1, acc[mt], 0, 0, 0);
        }
      }
      cur = (cur + 1) % kNumBuf;
    }

    // ---- epilogue: normalise, write o (final or partial) and lse
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = 1.f / ltot;
    const float lse_nat = (m_run + __log2f(ltot)) * kLn2;
    const int colbase = 256 * dh + 4 * h;
    if (sg.whole) {
      const int64_t orow = (int64_t(b) * kV2Heads + head) * kV2Lat + colbase;
      if (a.o_dt == MLA_BF16) {
        uint16_t* o = static_cast<uint16_t*>(a.o_lat) + orow;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[mt][4 * q4 + e] * inv);
            *reinterpret_cast<bf16x4*>(o + 32 * mt + 8 * q4) = v;
          }
      } else {
        float* o = static_cast<float*>(a.o_lat) + orow;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[mt][4 * q4 + e] * inv;
            *reinterpret_cast<f32x4*>(o + 32 * mt + 8 * q4) = v;
          }
      }
      if (h == 0 && dh == 0 && a.lse != nullptr) a.lse[int64_t(b) * kV2Heads + head] = lse_nat;
    } else {
      float* o = a.o_part + (int64_t(sg.slot) * kV2Heads + head) * kV2Lat + colbase;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[mt][4 * q4 + e] * inv;
          *reinterpret_cast<f32x4*>(o + 32 * mt + 8 * q4) = v;
        }
      if (h == 0 && dh == 0) a.lse_part[int64_t(sg.slot) * kV2Heads + head] = lse_nat;
    }
  }
}

// Grid: two workgroups per work item, padded so that ids map one-to-one onto
// (item, head half) with both halves of an item on the same XCD.
int decode_v2_grid(int n_items) { return 2 * ((n_items + 7) / 8) * 8; }

hipError_t launch_decode_v2(const V2DecodeArgs& a, hipStream_t st) {
  decode_v2_bf16_kernel<<<decode_v2_grid(a.n_items), kDecThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
