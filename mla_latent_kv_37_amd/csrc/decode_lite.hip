// MLA decode with few heads: DeepSeek-V2-Lite shapes on gfx950.
//
// V2-Lite keeps the V2 cache row (latent d_c = 512 plus a 64-wide RoPE key,
// 576 bf16 per token) but has 16 heads ([DeepSeek-V2 explainer] §3.1.1, the
// V2-Lite paragraph), so a token costs 2*16*576 + 2*16*512 = 34,816 flops for
// its 1,152 bytes: 30 flop/B, ten times below the MFMA/HBM ridge.  The kernel
// only has to keep enough cache bytes in flight; the matrix work is small.
//
// Work decomposition.  A work item is a list of (sequence, token range)
// segments (partition.h; ranges start on page boundaries).  One workgroup of
// 4 wavefronts (one per SIMD) serves an item; wavefront w takes quarter w
// (tokens 16w..16w+15) of every page of the range and keeps its own online
// softmax over them, so the tile loop has no barrier.  At the end of a segment
// the four (max, sum, output) partials are combined through LDS.
//
// Per 16-token tile, on the matrix cores (all heads of one wavefront):
//   S^T [16 tok x 16 heads] = K [16 x 576] . Q^T [576 x 16]   18 x v_mfma_f32_16x16x32_bf16
//   O^T [512 x 16 heads]   += V^T [512 x 16] . P^T [16 x 16]  32 x v_mfma_f32_16x16x16_bf16
// With tokens as the rows of S^T, lane l holds tokens 4(l>>4)..+3 of head l&15,
// which is the P^T operand layout of the second product as it is, and the
// output O^T keeps head l&15 in lane l, so each lane owns one head's softmax
// state.  V^T fragments come from transposing LDS reads (ds_read_b64_tr_b16).
//
// Data movement.  Each wavefront stages its tiles (16 rows x 1152 B = 18 KB) in
// two LDS buffers of its own with buffer loads that write LDS directly, one
// tile ahead of the one it computes on.  LDS tile layout: 1 KB blocks of 8 rows
// x 8 sixteen-byte chunks; chunk c of row t at (c>>3)*2048 + (t>>3)*1024 +
// (t&7)*128 + ((c&7) ^ f(t))*16, f(t) = (t&7 with bits 1 and 2 swapped) ^
// ((t>>3)&1).  One load instruction fills one block from 8 whole 128-byte row
// segments, and with 64 LDS banks the K reads (16 rows of one chunk per 16
// lanes) and the transposing V reads (4 rows x 32 B) are free of bank conflicts.
// The descriptor's size is the tile's valid bytes, so rows past the end of a
// sequence read as zeros (and their scores are masked).
//
// Softmax in the log2 domain, with the running max raised lazily (rescale only
// when it grows by more than 8), as in the 128-head kernel.
#include "kernels.h"

namespace mla {

namespace {

constexpr int kLHeads = 16, kLLat = 512, kLRope = 64, kLRow = 576, kLPage = 64;
constexpr int kLRowBytes = kLRow * 2;                 // 1152
constexpr int kLPageBytes = kLPage * kLRowBytes;      // 73728
constexpr int kLTileTok = 16;
constexpr int kLTileBytes = kLTileTok * kLRowBytes;   // 18432
constexpr int kLWaves = 4;
constexpr int kLThreads = 64 * kLWaves;
constexpr int kLArea = kLWaves * 2 * kLTileBytes;     // 147456: two tile buffers per wavefront
constexpr int kLLoads = 18;                           // one-KB loads per tile
constexpr float kLSlack = 8.0f;
constexpr uint32_t kLBufferFlags = 0x00020000u;

typedef int i32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int lswz(int t) {
  return ((t & 1) | ((t & 2) << 1) | ((t & 4) >> 1)) ^ ((t >> 3) & 1);
}
__host__ __device__ constexpr int lite_offset(int t, int c) {
  return (c >> 3) * 2048 + (t >> 3) * 1024 + (t & 7) * 128 + (((c & 7) ^ lswz(t)) * 16);
}

// The 18 loads of one tile: block (g, rb) = chunk group g (chunks 8g..8g+7) of
// rows 8rb..8rb+7.  Lane l reads row 8rb + (l>>3), chunk 8g + ((l&7) ^ f(row)),
// landing at LDS offset g*2048 + rb*1024 + 16*l.  Rows at or past `valid` read
// as zeros (descriptor size).  The loads carry the non-temporal hint: the cache
// is streamed once per step, and without the hint it evicts the data the step
// reuses (measured: decode 66.0 -> 58.9 us, merge + out-proj 10.4 -> 9.3 us).
__device__ __forceinline__ void lite_issue(const char* src, int valid, uint32_t buf) {
  int ln = threadIdx.x & 63;
  asm volatile("" : "+v"(ln));
  const int r0 = ln >> 3;
  const int voff0 = r0 * kLRowBytes + (((ln & 7) ^ lswz(r0)) * 16);
  const int voff1 = (8 + r0) * kLRowBytes + (((ln & 7) ^ lswz(8 + r0)) * 16);
  const uint64_t base = reinterpret_cast<uint64_t>(src);
  i32x4 rsrc;
  rsrc[0] = uniform(int(uint32_t(base)));
  rsrc[1] = uniform(int(uint32_t(base >> 32) & 0xFFFFu));
  rsrc[2] = uniform(valid * kLRowBytes);
  rsrc[3] = int(kLBufferFlags);
#pragma unroll
  for (int g = 0; g < 9; ++g) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int m0 = uniform(int(buf + uint32_t(g * 2048 + rb * 1024)));
      const int soff = uniform(g * 128);
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %1, %2, %3 offen nt lds"
          :
          : "s"(m0), "v"(rb ? voff1 : voff0), "s"(rsrc), "s"(soff)
          : "memory", "m0");
    }
  }
}

__device__ __forceinline__ bf16x8 lds_b128(uint32_t addr) {
  return *reinterpret_cast<const bf16x8 MLA_LDS*>((const char MLA_LDS*)(uintptr_t)addr);
}

__device__ __forceinline__ s16x4 lds_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 MLA_LDS*)(uintptr_t)addr);
}

// max / sum over the four 16-lane rows (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace

__global__ __launch_bounds__(kLThreads) void decode_lite_kernel(V2DecodeArgs a) {
  __shared__ __attribute__((aligned(4096))) char area_raw[kLArea];
  const int n_items = a.n_items;
  const int item = (n_items & 7) == 0 ? int(blockIdx.x & 7) * (n_items >> 3) + int(blockIdx.x >> 3) : int(blockIdx.x);
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int hd = lane & 15, g = lane >> 4;
  if (item >= n_items) return;
  const uint32_t area = uint32_t(reinterpret_cast<uintptr_t>(area_raw));
  const uint32_t buf0 = area + uint32_t(wave * 2 * kLTileBytes);
  // per-lane LDS bases: K chunk g of row hd (step s: ^ 64*(s&1), + (s>>1)*2048);
  // V^T rows 4g + ((lane&15)>>2), chunk ((lane>>1)&1), byte (lane&1)*8
  // (column tile n: ^ 32*(n&3), + (n>>2)*2048)
  const uint32_t kb = uint32_t(lite_offset(hd, g));
  const uint32_t vb = uint32_t(lite_offset(4 * g + (hd >> 2), (hd >> 1) & 1) + (hd & 1) * 8);

  SegmentIter it;
  it.init(a.pp, a.seq_lens, item, a.meta);
  Segment sg;
  while (it.next(sg)) {
    const int b = uniform(sg.b);
    const int t0 = uniform(sg.t0), t1 = uniform(sg.t1);
    const int32_t* bt = a.block_table + int64_t(b / a.bt_div) * a.max_pages + t0 / kLPage;
    const char* kv = static_cast<const char*>(a.kv);
    const int len = t1 - t0;
    const int npages = ceil_div(len, kLPage);
    // this wavefront's tiles: quarter `wave` of pages 0..ntl-1 (only the last
    // page can have an empty quarter)
    const int last_valid = len - (npages - 1) * kLPage - kLTileTok * wave;
    const int ntl = last_valid > 0 ? npages : npages - 1;
    // a page id outside [0, num_pages) reads as a page of zero rows (no
    // address outside the cache is formed)
    auto tile_valid = [&](int k) { return k < npages - 1 ? kLTileTok : min(kLTileTok, last_valid); };
    auto dma_valid = [&](int k) {   // rows the tile loads read (0: a zero tile)
      return unsigned(load_const(bt, k)) < unsigned(a.num_pages) ? tile_valid(k) : 0;
    };
    auto tile_src = [&](int k) {
      const int pid = load_const(bt, k);
      return kv + int64_t(unsigned(pid) < unsigned(a.num_pages) ? pid : 0) * kLPageBytes + wave * kLTileBytes;
    };
    auto tile_buf = [&](int k) { return buf0 + uint32_t((k & 1) * kLTileBytes); };

    // every wavefront is done with the previous segment's LDS use
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    raw_barrier();
    if (ntl > 0) lite_issue(tile_src(0), dma_valid(0), tile_buf(0));
    // Q^T fragments (B operand): head hd, dims 32s + 8g .. +7 of [q_lat | q_pe]
    bf16x8 qf[18];
    {
      const uint16_t* ql = a.q_lat + (int64_t(b) * kLHeads + hd) * kLLat + 8 * g;
      const uint16_t* qr = a.q_pe + (int64_t(b) * kLHeads + hd) * kLRope + 8 * g;
#pragma unroll
      for (int s = 0; s < 16; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(ql + 32 * s);
      qf[16] = *reinterpret_cast<const bf16x8*>(qr);
      qf[17] = *reinterpret_cast<const bf16x8*>(qr + 32);
    }
    // tile 0 and the query first; the explicit full wait also tells the compiler
    // that the query registers are ready, so it puts no wait for them inside the
    // tile loop (where it would drain the tile prefetch)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if (ntl > 1) lite_issue(tile_src(1), dma_valid(1), tile_buf(1));
    f32x4 acc[32];
#pragma unroll
    for (int n = 0; n < 32; ++n) acc[n] = f32x4{};
    float m_run = -INFINITY, lsum = 0.f;

    for (int k = 0; k < ntl; ++k) {
      // tile k complete (tile k+1's 18 loads may still be in flight)
      if (k + 1 < ntl) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLLoads));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      const uint32_t tb = tile_buf(k);
      // ---- S^T = K . Q^T: even and odd k-steps in two accumulators (two
      // independent MFMA chains), K fragments read two steps ahead
      f32x4 s;
      {
        auto kfrag = [&](int st) { return lds_b128(((tb + kb) ^ uint32_t(64 * (st & 1))) + uint32_t((st >> 1) * 2048)); };
        f32x4 se = {}, so = {};
        bf16x8 k0 = kfrag(0), k1 = kfrag(1);
#pragma unroll
        for (int st = 0; st < 18; ++st) {
          bf16x8 k2;
          if (st + 2 < 18) k2 = kfrag(st + 2);
          if (st & 1) so = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[st], so, 0, 0, 0);
          else se = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[st], se, 0, 0, 0);
          k0 = k1;
          k1 = k2;
        }
        s = se + so;
      }
      // ---- online softmax: lane holds tokens 4g..4g+3 of head hd
      const int valid = tile_valid(k);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = 4 * g + i < valid ? s[i] * a.scale_log2 : -INFINITY;
      const float mx = rows_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
      const float m_new = fmaxf(m_run, mx);
      if (__any(m_new > m_run + kLSlack)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int n = 0; n < 32; ++n) acc[n] *= alpha;
        lsum *= alpha;
        m_run = m_new;
      }
      s16x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[i] - m_run);
        lsum += p;
        pk[i] = __builtin_bit_cast(short, (__bf16)p);
      }
      // ---- O^T += V^T . P^T over the 32 column tiles
      {
        auto vfrag = [&](int n) { return lds_tr(((tb + vb) ^ uint32_t(32 * (n & 3))) + uint32_t((n >> 2) * 2048)); };
        s16x4 v0 = vfrag(0), v1 = vfrag(1);
#pragma unroll
        for (int n = 0; n < 32; ++n) {
          s16x4 v2;
          if (n + 2 < 32) v2 = vfrag(n + 2);
          acc[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, pk, acc[n], 0, 0, 0);
          v0 = v1;
          v1 = v2;
        }
      }
      // the buffer's reads are done before the next tile's loads overwrite it
      if (k + 2 < ntl) {
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
        lite_issue(tile_src(k + 2), dma_valid(k + 2), tb);
      }
    }

    // ---- combine the four wavefronts' partials through LDS
    const float ltot = rows_sum(lsum);
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    raw_barrier();   // every wavefront is done with its tile buffers
    // O^T partial of wavefront w: column quad q = 4n + g, head hd at
    // w*32768 + (q*16 + hd)*16 (16 lanes write 256 consecutive bytes)
    const uint32_t ow = area + uint32_t(wave * 32768);
#pragma unroll
    for (int n = 0; n < 32; ++n)
      *reinterpret_cast<f32x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(ow + uint32_t(((4 * n + g) * 16 + hd) * 16))) = acc[n];
    const uint32_t ml = area + uint32_t(kLWaves * 32768);
    if (g == 0) {
      *reinterpret_cast<float MLA_LDS*>((char MLA_LDS*)(uintptr_t)(ml + uint32_t((wave * 16 + hd) * 4))) = m_run;
      *reinterpret_cast<float MLA_LDS*>((char MLA_LDS*)(uintptr_t)(ml + uint32_t((64 + wave * 16 + hd) * 4))) = ltot;
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    raw_barrier();
    float mw[kLWaves], M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kLWaves; ++w) {
      mw[w] = *reinterpret_cast<const float MLA_LDS*>((const char MLA_LDS*)(uintptr_t)(ml + uint32_t((w * 16 + hd) * 4)));
      M = fmaxf(M, mw[w]);
    }
    float wt[kLWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kLWaves; ++w) {
      const float lw = *reinterpret_cast<const float MLA_LDS*>(
          (const char MLA_LDS*)(uintptr_t)(ml + uint32_t((64 + w * 16 + hd) * 4)));
      wt[w] = mw[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - M);
      L += wt[w] * lw;
    }
    const float inv = 1.f / L;
    // this wavefront writes column quads 32*wave + g + 4j (j = 0..7) of head hd
    void* const obase = sg.whole ? a.o_lat : a.o_part;
    const int64_t orow = (int64_t(sg.whole ? b : sg.slot) * kLHeads + hd) * kLLat;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = 32 * wave + g + 4 * j;
      f32x4 o = {};
#pragma unroll
      for (int w = 0; w < kLWaves; ++w) {
        const f32x4 v = *reinterpret_cast<const f32x4 MLA_LDS*>(
            (const char MLA_LDS*)(uintptr_t)(area + uint32_t(w * 32768 + (q * 16 + hd) * 16)));
        o += v * wt[w];
      }
      o *= inv;
      if (a.o_dt == MLA_BF16) {
        bf16x4 ob;
#pragma unroll
        for (int e = 0; e < 4; ++e) ob[e] = (__bf16)o[e];
        *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(obase) + orow + 4 * q) = ob;
      } else {
        *reinterpret_cast<f32x4*>(static_cast<float*>(obase) + orow + 4 * q) = o;
      }
    }
    if (wave == 0 && g == 0) {
      const float lse_nat = (M + __log2f(L)) * kLn2;
      if (!sg.whole) a.lse_part[int64_t(sg.slot) * kLHeads + hd] = lse_nat;
      else if (a.lse != nullptr) a.lse[int64_t(b) * kLHeads + hd] = lse_nat;
    }
  }
}

hipError_t launch_decode_lite(const V2DecodeArgs& a, hipStream_t st) {
  decode_lite_kernel<<<a.n_items, kLThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
