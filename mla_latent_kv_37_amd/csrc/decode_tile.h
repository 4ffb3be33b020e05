// Paged-cache tile staging of the 128-head decode kernel (V2 shapes:
// 576-wide rows [c^KV | k^R], 64-token pages, bf16): the LDS tile layout, the
// direct-to-LDS tile and query loads, and the LDS fragment reads.
//
// LDS tile layout: 1 KB blocks of 8 rows x 8 chunks (a chunk is 16 B = 8 bf16);
// chunk c of row t sits at (c>>3)*4096 + (t>>3)*1024 + (t&7)*128 +
// ((c&7) ^ f(t))*16 with f(t) = (t&7 with bits 1 and 2 swapped) ^ ((t>>3)&1).
// One load instruction fills one block from 8 whole 128-byte row segments
// (full cache lines), and with 64 LDS banks both the K-fragment reads (32 rows
// of one chunk) and the transposing V reads (4 rows x 32 B) are free of bank
// conflicts.  Every fragment address is a per-lane base plus an immediate, or
// the base XOR a constant: the chunk slot occupies address bits 4-6 and every
// buffer base is a multiple of 2048.
#pragma once

#include "kernels.h"

namespace mla {

constexpr int kV2Heads = 128, kV2Lat = 512, kV2Rope = 64, kV2Row = 576, kV2Page = 64;
constexpr int kRowBytes = kV2Row * 2;                 // 1152
constexpr int kPageBytes = kV2Page * kRowBytes;       // 73728
constexpr int kTileTok = 32;
constexpr int kTileBytes = kTileTok * kRowBytes;      // 36864
constexpr uint32_t kBufferFlags = 0x00020000u;        // raw buffer, 32-bit data format

typedef int i32x4 __attribute__((ext_vector_type(4)));

// chunk-slot swizzle of row t (see the layout note above)
__host__ __device__ constexpr int swz_f(int t) {
  return ((t & 1) | ((t & 2) << 1) | ((t & 4) >> 1)) ^ ((t >> 3) & 1);
}
__host__ __device__ constexpr int tile_offset(int t, int c) {
  return (c >> 3) * 4096 + (t >> 3) * 1024 + (t & 7) * 128 + (((c & 7) ^ swz_f(t)) * 16);
}

// Tile loads: block i = 4g + rb holds rows 8rb..8rb+7 of chunk group g (chunks
// 8g..8g+7); a tile is 36 one-block loads, row block rb of all 9 chunk groups
// being one wavefront's share.  Lane l of a block load
// reads row 8rb + (l>>3), logical chunk 8g + ((l&7) ^ f(row)), so that it lands
// at LDS offset i*1024 + 16*l; its byte offset in the tile is the per-lane
// `voff` (fixed per wavefront) plus g*128 (the scalar offset).
__device__ __forceinline__ int dma_voff(int wave, int lane) {
  const int row = 8 * (wave & 3) + (lane >> 3);
  return row * kRowBytes + (((lane & 7) ^ swz_f(row)) * 16);
}

// Tile loads.  With or without the scalar offset in the hardware range check,
// a row is in range exactly when it is below `valid`, so rows past the
// sequence end read as zeros.
// The loads carry the non-temporal hint: the cache is streamed once per step,
// and without the hint it pushes the step's reused data (the weights, the
// absorbed queries, the split partials) out of the caches (measured: 3.6 us
// less per step over absorb, decode and merge).
// The loads are inline assembly so that the compiler does not track them: they
// have no destination registers (data goes to LDS at M0 + 16*lane) and their
// completion is waited for explicitly (vmcnt) before the barrier that publishes
// a tile.  The compiler's own vmcnt waits for other loads stay correct, only
// possibly stricter, since these loads are not counted by it.
// TileRowLoad: the loads of one tile's row block rb (rows 8rb..8rb+7, all 9
// chunk groups), 9 one-block loads.  `init` sets up the buffer descriptor and the per-lane
// offset, `group` issues chunk group g, so that a caller can spread the 9
// issues over other work.
struct TileRowLoad {
  i32x4 rsrc;
  int voff;
  uint32_t buf;
  int rb;
  __device__ __forceinline__ void init(const char* src, int valid, uint32_t buf_, int rb_) {
    // per-lane offset, recomputed at each use from an opaque lane id instead of
    // being held in a register across the tile loop
    int ln = threadIdx.x & 63;
    asm volatile("" : "+v"(ln));
    voff = dma_voff(rb_, ln);
    const uint64_t base = reinterpret_cast<uint64_t>(src);
    rsrc[0] = uniform(int(uint32_t(base)));
    rsrc[1] = uniform(int(uint32_t(base >> 32) & 0xFFFFu));  // stride 0
    rsrc[2] = uniform(valid * kRowBytes);
    rsrc[3] = int(kBufferFlags);
    buf = buf_;
    rb = rb_;
  }
  __device__ __forceinline__ void group(int g) const {
    const int m0 = uniform(int(buf + uint32_t((4 * g + rb) * 1024)));
    const int soff = uniform(g * 128);
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds"
        :
        : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff)
        : "memory", "m0");
  }
};

// Query staging.  A wavefront's latent query (32 heads x 256 dims, 16 KB) is
// copied into LDS in two passes of 128 dims (8 KB: 32 rows of 256 B) by
// direct-to-LDS loads that each read four whole row pieces (full cache lines),
// then read back in the MFMA operand layout.  Register loads in that layout
// would touch every 128-byte line four times.  In the staging area chunk c
// (16 B) of row r sits at r*256 + ((c ^ (r & 15)) * 16): the operand reads (16
// rows of one chunk per 16 lanes) hit 16 distinct bank groups.  The loads are
// not tracked by the compiler (inline assembly), so their completion is waited
// for explicitly, which also lets the first tile be waited for without the
// second.
__device__ __forceinline__ void issue_query_pass(const uint16_t* src, uint32_t stage) {
  int ln = threadIdx.x & 63;
  asm volatile("" : "+v"(ln));
  const uint64_t base = reinterpret_cast<uint64_t>(src);
  i32x4 rsrc;
  rsrc[0] = uniform(int(uint32_t(base)));
  rsrc[1] = uniform(int(uint32_t(base >> 32) & 0xFFFFu));
  rsrc[2] = 31 * kV2Lat * 2 + 256;   // rows 0..31 at a 1024-byte stride, 256 B each
  rsrc[3] = int(kBufferFlags);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (ln >> 4), c = (ln & 15) ^ (r & 15);
    const int voff = r * (kV2Lat * 2) + c * 16;
    const int m0 = uniform(int(stage + uint32_t(i * 1024)));
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 : : "s"(m0), "v"(voff), "s"(rsrc) : "memory", "m0");
  }
}

// ---------------------------------------------------------------------------
// fp8 cache (OCP E4M3 codes, one fp32 scale per token per 128-channel group;
// the stored value is code * scale).  A tile's codes (32 rows x 576 B, one
// contiguous run inside a page) and scales (32 x 5 fp32) are copied into an LDS
// staging buffer, then dequantised once into the bf16 tile layout above, which
// the score and PV steps read unchanged.
constexpr int kF8TileBytes = kTileTok * kV2Row;       // 18432
constexpr int kF8Groups = 5;                          // scale groups per row
constexpr int kF8StageBytes = kF8TileBytes + 1024;    // codes, then scales (640 B used)

// Loads of one staged tile: 18 one-KB code blocks and one scale block, by
// wavefronts 0-3 (5 each for wavefronts 0-2, 4 for wavefront 3; load i: codes
// block i for i < 18, the scales for i = 18).  Rows past `valid` read as zeros
// (codes and scales).  Non-temporal, like the bf16 tile loads.
__device__ __forceinline__ int f8_first_load(int wave) { return 5 * (wave & 3); }
__device__ __forceinline__ int f8_num_loads(int wave) { return wave < 3 ? 5 : 4; }

__device__ __forceinline__ void issue_tile_f8(const char* codes, const float* scales, int valid, uint32_t stage,
                                              int wave) {
  int ln = threadIdx.x & 63;
  asm volatile("" : "+v"(ln));
  const int voff = ln * 16;
  const uint64_t cb = reinterpret_cast<uint64_t>(codes), sb = reinterpret_cast<uint64_t>(scales);
  i32x4 rc, rs;
  rc[0] = uniform(int(uint32_t(cb)));
  rc[1] = uniform(int(uint32_t(cb >> 32) & 0xFFFFu));
  rc[2] = uniform(valid * kV2Row);
  rc[3] = int(kBufferFlags);
  rs[0] = uniform(int(uint32_t(sb)));
  rs[1] = uniform(int(uint32_t(sb >> 32) & 0xFFFFu));
  // whole 16-byte lane loads: the last valid row's scales end mid-load when
  // valid % 4 != 0, so the range is rounded up (to at most the tile's 640
  // bytes, inside the page); the extra scales belong to rows >= valid, which
  // the dequantisation writes as zeros whatever they hold
  rs[2] = uniform((valid * kF8Groups * 4 + 15) & ~15);
  rs[3] = int(kBufferFlags);
  const int i0 = f8_first_load(wave), nl = f8_num_loads(wave);
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    if (j < nl) {
      const int i = i0 + j;
      const int m0 = uniform(int(stage + uint32_t(i * 1024)));
      if (i < 18) {
        const int soff = uniform(i * 1024);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                     : : "s"(m0), "v"(voff), "s"(rc), "s"(soff) : "memory", "m0");
      } else {
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                     : : "s"(m0), "v"(voff), "s"(rs) : "memory", "m0");
      }
    }
  }
}

// The LDS reads of one dequantisation item (one bf16 chunk of 8 values of one
// row): its 8 codes and its row's group scale.  Each value is code * scale in
// fp32, rounded to bf16; rows past the sequence end are written as zeros, not
// code * scale, since their staged scales may be anything.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
struct F8Item {
  u32x2 code;
  float sc;
};

__device__ __forceinline__ bf16x8 lds_read_b128(uint32_t addr) {
  return *reinterpret_cast<const bf16x8 MLA_LDS*>((const char MLA_LDS*)(uintptr_t)addr);
}

__device__ __forceinline__ bf16x8 lds_read_tr_pair(uint32_t a0, uint32_t a1) {
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 MLA_LDS*)(uintptr_t)a0);
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 MLA_LDS*)(uintptr_t)a1);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}


}  // namespace mla
