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
// segments (partition.cuh); one workgroup of 8 wavefronts (2 per SIMD, so one
// wavefront's memory and LDS waits are covered by the other's matrix work)
// serves one work item for all 128 heads.  The wavefronts form 4 pairs; pair p
// owns heads 32p..32p+31 and its two members sit on the same SIMD.  Member d
// multiplies half of the 576 row dims for the scores (latent dims
// [256d, 256d+256) plus RoPE dims [32d, 32d+32)) and owns output columns
// [256d, 256d+256).  The pair adds its two fp32 partial score blocks through
// LDS, both members run the (identical) softmax, and each accumulates its 256
// columns.  Per wavefront that is 64 registers of query (the RoPE part of the
// query is read from LDS) and 128 of accumulator, which fits two wavefronts per
// SIMD.
//
// Data movement.  32-token tiles (36,864 B) are staged in LDS by buffer loads
// that write LDS directly (16 B per lane); three tile buffers give a prefetch
// distance of two tiles.  The descriptor's size is the tile's valid bytes, so
// rows past the end of a sequence read as zeros (their scores are masked to
// -inf, and a zero value row keeps 0 * v finite even when the slot holds NaN).
// LDS tile layout: 1 KB blocks of 8 rows x 8 chunks (a chunk is 16 B = 8 bf16);
// chunk c of row t sits at (c>>3)*4096 + (t>>3)*1024 + (t&7)*128 +
// ((c&7) ^ f(t))*16 with f(t) = (t&7 with bits 1 and 2 swapped) ^ ((t>>3)&1).
// One load instruction fills one block from 8 whole 128-byte row segments
// (full cache lines), and with 64 LDS banks both the K-fragment reads (32 rows
// of one chunk) and the transposing V reads (4 rows x 32 B) are free of bank
// conflicts.  Every LDS address is a per-lane base plus an immediate.
//
// Per tile k: wait for tile k, barrier, issue tile k+2, partial scores, write
// them, barrier, add the peer's, softmax, PV.
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
constexpr int kWaves = 8;
constexpr int kDecThreads = 64 * kWaves;
constexpr int kXsBytes = kWaves * 4096;               // partial-score exchange area
constexpr float kRescaleSlack = 8.0f;                 // log2 units
constexpr uint32_t kBufferFlags = 0x00020000u;        // raw buffer, 32-bit data format

typedef int i32x4 __attribute__((ext_vector_type(4)));

// chunk-slot swizzle of row t (see the layout note above)
__host__ __device__ constexpr int swz_f(int t) {
  return ((t & 1) | ((t & 2) << 1) | ((t & 4) >> 1)) ^ ((t >> 3) & 1);
}
__host__ __device__ constexpr int tile_offset(int t, int c) {
  return (c >> 3) * 4096 + (t >> 3) * 1024 + (t & 7) * 128 + (((c & 7) ^ swz_f(t)) * 16);
}

// Tile loads per wavefront: 36 one-block loads, 5 each for wavefronts 0-3
// (blocks 5w..5w+4) and 4 each for wavefronts 4-7 (blocks 20+4(w-4)..).
__device__ __forceinline__ int first_block(int wave) { return wave < 4 ? 5 * wave : 20 + 4 * (wave - 4); }
__device__ __forceinline__ int num_blocks(int wave) { return wave < 4 ? 5 : 4; }

// Direct-to-LDS loads of one 32-token tile (block i = 4*(chunk group) + row
// block).  Lane l of a block load reads row 8*rb + (l>>3), logical chunk
// 8*g + ((l&7) ^ f(row)), so that it lands at LDS offset i*1024 + 16*l.
// `voff_even` / `voff_odd` hold the per-lane row/chunk byte offset for even /
// odd row blocks; the row block's 9216 B step is added here and the chunk
// group's 128 B step is the scalar offset.  With or without the scalar offset
// in the hardware range check, a row is in range exactly when it is below
// `valid`, so rows past the sequence end read as zeros.
// The loads are inline assembly so that the compiler does not track them: they
// have no destination registers (data goes to LDS at M0 + 16*lane) and their
// completion is waited for explicitly (vmcnt) before the barrier that publishes
// a tile.  The compiler's own vmcnt waits for other loads stay correct, only
// possibly stricter, since these loads are not counted by it.
__device__ __forceinline__ void issue_tile(const char* tile_ptr, int valid, char MLA_LDS* buf, int wave) {
  int ln = threadIdx.x & 63;
  asm volatile("" : "+v"(ln));  // recomputed at each use instead of held across the loop
  const int r = ln >> 3, sl = ln & 7;
  const int voff_even = r * kRowBytes + ((sl ^ swz_f(r)) * 16);
  const int voff_odd = r * kRowBytes + ((sl ^ swz_f(r + 8)) * 16);
  const uint64_t base = reinterpret_cast<uint64_t>(tile_ptr);
  i32x4 rsrc;
  rsrc[0] = uniform(int(uint32_t(base)));
  rsrc[1] = uniform(int(uint32_t(base >> 32) & 0xFFFFu));  // stride 0
  rsrc[2] = uniform(valid * kRowBytes);
  rsrc[3] = int(kBufferFlags);
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(buf));
  const int b0 = first_block(wave), nb = num_blocks(wave);
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    if (j < nb) {
      const int i = b0 + j;
      const int rb = i & 3, g = i >> 2;
      const int m0 = uniform(int(lds0 + i * 1024));
      const int soff = uniform(g * 128);
      const int voff = ((rb & 1) ? voff_odd : voff_even) + rb * 8 * kRowBytes;
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %1, %2, %3 offen lds"
          :
          : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
          : "memory", "m0");
    }
  }
}

// wait until this wavefront's loads of the tile before the newest are done
__device__ __forceinline__ void wait_tile(int wave, bool newer_in_flight) {
  if (!newer_in_flight) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  else if (wave < 4) __builtin_amdgcn_s_waitcnt(waitcnt_vm(5));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
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

__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_v2_bf16_kernel(V2DecodeArgs a) {
  __shared__ __attribute__((aligned(1024))) char tiles_raw[kNumBuf * kTileBytes];
  __shared__ __attribute__((aligned(1024))) char xs_raw[kXsBytes];
  char MLA_LDS* const tiles = (char MLA_LDS*)tiles_raw;
  const int item = blockIdx.x;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, h = lane >> 5;
  const int pair = wave & 3, dh = wave >> 2;   // pair members w and w^4 share a SIMD
  const int head = pair * 32 + (lane & 31);
  if (item >= a.n_items) return;


  SegmentIter it;
  it.init(a.pp, a.seq_lens, item, reinterpret_cast<int*>(tiles_raw), a.meta);
  Segment sg;
  while (it.next(sg)) {
    const int b = uniform(sg.b);
    const int t0 = uniform(sg.t0), t1 = uniform(sg.t1);
    const int32_t* bt = a.block_table + int64_t(b) * a.max_pages;
    const char* kv = static_cast<const char*>(a.kv);
    const int ntiles = ceil_div(t1 - t0, kTileTok);
    auto tile_ptr = [&](int k) -> const char* {
      const int tok = t0 + k * kTileTok;
      return kv + int64_t(load_const(bt, tok / kV2Page)) * (kV2Page * kRowBytes) + (tok % kV2Page) * kRowBytes;
    };
    auto tile_valid = [&](int k) { return min(kTileTok, t1 - t0 - k * kTileTok); };
    auto tile_buf = [&](int k) { return tiles + (k % kNumBuf) * kTileBytes; };

    // every wavefront is done with the previous segment's tiles, scores and query
    raw_barrier();
    issue_tile(tile_ptr(0), tile_valid(0), tile_buf(0), wave);
    // query slices of head `head` (MFMA B operand: lane holds 8 consecutive dims):
    // latent dims 256*dh + 16*kk + 8*h .. +8, RoPE dims 32*dh + 16*j + 8*h .. +8
    bf16x8 qf[16], qr[2];
    {
      const uint16_t* ql = a.q_lat + (int64_t(b) * kV2Heads + head) * kV2Lat + 256 * dh + 8 * h;
#pragma unroll
      for (int kk = 0; kk < 16; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(ql + 16 * kk);
      const uint16_t* qp = a.q_pe + (int64_t(b) * kV2Heads + head) * kV2Rope + 32 * dh + 8 * h;
#pragma unroll
      for (int j = 0; j < 2; ++j) qr[j] = *reinterpret_cast<const bf16x8*>(qp + 16 * j);
    }
    // tile 0 and the query are needed first; an explicit full wait here also tells
    // the compiler that the query registers are ready, so it puts no waits for
    // them inside the tile loop (where they would drain the tile prefetches).
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if (ntiles > 1) issue_tile(tile_ptr(1), tile_valid(1), tile_buf(1), wave);

    // Per-lane LDS offsets inside a tile, without the chunk-group part (a
    // wavefront-uniform 16384*dh for its latent half, 32768 for the RoPE group,
    // n*4096 for later groups), which is added as a scalar or an immediate.  The
    // chunk slot occupies address bits 4-6 and every base is a multiple of 1024,
    // so moving to chunk c ^ x within a group is an XOR of the address with 16*x.
    // K fragment of latent k-step 4n+m: token lane&31, chunk 32dh + 2m + h:
    //   kb0 ^ 32m (+ n*4096).  RoPE k-step j: chunk 64 + 4dh + 2j + h:
    //   kb0 ^ (64dh + 32j) in the RoPE group.
    const int kb0 = tile_offset(lane & 31, h);
    // V^T fragment (transposing reads) of column tile 2n+p, token half ks, row
    // group sec: (vb[sec] ^ 64p) + n*4096 + ks*2048 in this wavefront's half.
    int vb[2];
    {
      const int g = lane >> 4, j = lane & 15;
#pragma unroll
      for (int sec = 0; sec < 2; ++sec) {
        const int cc = 2 * (g & 1) + ((j >> 1) & 1);
        const int r = 8 * sec + 4 * h + (j >> 2);
        vb[sec] = tile_offset(r, cc) + (j & 1) * 8;
      }
    }
    const int xs_lane = lane * 16;

    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
    float m_run = -INFINITY, lsum = 0.f;

    for (int k = 0; k < ntiles; ++k) {
      const int valid = tile_valid(k);
      // ---- tile k visible to all
      wait_tile(wave, k + 1 < ntiles);
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();
      if (k + 2 < ntiles) issue_tile(tile_ptr(k + 2), tile_valid(k + 2), tile_buf(k + 2), wave);
      // LDS byte address of this tile (scalar), kept opaque so that the
      // constant parts of the offsets stay in the instructions' immediates
      int tbase = uniform(int(uint32_t(reinterpret_cast<uintptr_t>(tile_buf(k)))));
      asm volatile("" : "+s"(tbase));
      const uint32_t kl = uint32_t(tbase + 16384 * dh) + kb0, krp = uint32_t(tbase + 32768) + kb0;

      // ---- partial S^T over this wavefront's 288 row dims; fragment reads run
      // two k-steps ahead of the (dependent) MFMA chain
      auto kfrag = [&](int st) -> bf16x8 {
        const uint32_t ad = st < 16 ? (kl ^ (32 * (st & 3))) + (st >> 2) * 4096 : krp ^ (64 * dh + 32 * (st - 16));
        return lds_read_b128((const char MLA_LDS*)(uintptr_t)ad);
      };
      f32x16 s = {};
      bf16x8 k0 = kfrag(0), k1 = kfrag(1);
#pragma unroll
      for (int st = 0; st < 18; ++st) {
        bf16x8 k2;
        if (st + 2 < 18) k2 = kfrag(st + 2);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, st < 16 ? qf[st] : qr[st - 16], s, 0, 0, 0);
        k0 = k1;
        k1 = k2;
      }
      // ---- exchange partial scores within the pair
      {
        char MLA_LDS* xm = (char MLA_LDS*)xs_raw + wave * 4096 + xs_lane;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v = {s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
          *reinterpret_cast<f32x4 MLA_LDS*>(xm + q4 * 1024) = v;
        }
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();
      {
        const char MLA_LDS* xp = (const char MLA_LDS*)xs_raw + (wave ^ 4) * 4096 + xs_lane;
        f32x4 v[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) v[q4] = *reinterpret_cast<const f32x4 MLA_LDS*>(xp + q4 * 1024);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[4 * q4 + e] += v[q4][e];
      }
      // ---- online softmax (lane: head `head`, 16 of the tile's tokens; lane^32 the other 16)
      if (valid < kTileTok) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int tok = 8 * (r >> 2) + 4 * h + (r & 3);
          s[r] = tok < valid ? s[r] : -INFINITY;
        }
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      if (__any(m_new > m_run + kRescaleSlack)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= alpha;
        lsum *= alpha;
        m_run = m_new;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], a.scale_log2, -m_run));
      {
        float t0 = (s[0] + s[1]) + (s[2] + s[3]), t1 = (s[4] + s[5]) + (s[6] + s[7]);
        float t2 = (s[8] + s[9]) + (s[10] + s[11]), t3 = (s[12] + s[13]) + (s[14] + s[15]);
        lsum += (t0 + t1) + (t2 + t3);
      }
      const bf16x8 pk0 = pack8(s, 0), pk1 = pack8(s, 8);
      // ---- O^T += V^T . P^T over this wavefront's 256 columns, fragment reads
      // two MFMAs ahead
      const uint32_t vl0 = uint32_t(tbase + 16384 * dh) + vb[0], vl1 = uint32_t(tbase + 16384 * dh) + vb[1];
      auto vfrag = [&](int st) -> bf16x8 {
        const int ks = st >> 3, mt = st & 7, p = mt & 1, n = mt >> 1;
        const uint32_t a0 = (vl0 ^ (64 * p)) + n * 4096 + ks * 2048, a1 = (vl1 ^ (64 * p)) + n * 4096 + ks * 2048;
        return lds_read_tr_pair((const char MLA_LDS*)(uintptr_t)a0, (const char MLA_LDS*)(uintptr_t)a1);
      };
      bf16x8 v0 = vfrag(0), v1 = vfrag(1);
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        bf16x8 v2;
        if (st + 2 < 16) v2 = vfrag(st + 2);
        const int mt = st & 7;
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, st < 8 ? pk0 : pk1, acc[mt], 0, 0, 0);
        v0 = v1;
        v1 = v2;
      }
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

hipError_t launch_decode_v2(const V2DecodeArgs& a, hipStream_t st) {
  decode_v2_bf16_kernel<<<a.n_items, kDecThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
