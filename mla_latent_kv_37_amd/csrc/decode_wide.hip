// MLA decode at DeepSeek-V2 shapes over a bf16 cache, one wavefront per SIMD.
//
// One workgroup per work item (partition.h); a segment of a split sequence
// writes its bf16 partial and lse, a whole sequence its final rows; tiles sit
// in LDS in the layout of decode_tile.h.  A workgroup has 4 wavefronts, one
// per SIMD, and wavefront w owns heads 32w..32w+31 entirely: all 576 dims of
// their scores and all 512 output columns.  Per 32-token tile it computes
//   S^T [32 tokens x 32 heads] = K [32 x 576] . Q^T [576 x 32]    (36 MFMAs)
//   O^T [512 x 32 heads]     += V^T [512 x 32] . P^T [32 x 32]    (32 MFMAs)
// on v_mfma_f32_32x32x16_bf16, with nothing exchanged between wavefronts but
// the tiles.  Alone on its SIMD, a wavefront has the whole 512-entry register
// file: the 256 accumulator registers hold O^T, the VGPRs the query of its
// heads (128 latent + 16 RoPE), the scores and the fragment reads issued
// several MFMAs ahead of their use.  Those reads are what hides the LDS latency: no second wavefront shares
// the SIMD to switch to.
//
// Software pipeline of tile k (per wavefront):
//   (first tile of a segment only: the max of S(k), which sets the reference)
//   phase A: the 36 score MFMAs of tile k+1, with the exponentials of S(k)
//            (each placed while a K fragment read is outstanding, the running
//            max taken from the same scores), the row sums and the bf16
//            packing of P(k) between them
//   phase B: the 32 PV MFMAs of tile k, with the 9 loads of this wavefront's
//            row block of tile k+3 between them
//   wait for this wavefront's loads of tile k+2, barrier (tile k+2 complete;
//     every wavefront is done with tile k, whose buffer takes tile k+4)
// Four tile buffers take 144 KB of the 160 KB of LDS.  (The RoPE query is held
// in registers rather than read from LDS every tile: 4 KB less LDS reading per
// wavefront and tile, the latent score steps' K reads being what the loop
// waits for.)
//
// Softmax without rescaling.  The accumulators are written by MFMAs only:
// multiplying them by a rescale factor anywhere in the segment loop makes the
// compiler move them through VGPRs, which do not have room for them.  Instead
// each head's reference max m_ref is fixed at the segment's first tile, and
// later tiles' probabilities exp2(s - m_ref) may exceed 1.  They are exact in
// floating point as long as nothing overflows, which the running true max
// m_seen guards: if any head's m_seen exceeds m_ref by more than kRefSlack
// (2^64 is far from the fp32 and bf16 limits, with room for the sums), the
// workgroup agrees at the segment's end and computes the segment again with
// m_ref = m_seen, the exact max, so that every probability is <= 1.
#include "decode_tile.h"

namespace mla {
namespace {

constexpr int kWideWaves = 4;
constexpr int kWideThreads = 64 * kWideWaves;
constexpr int kWideBufs = 4;
constexpr int kScoreSteps = 36;   // k-steps of 16 dims: 32 latent, 4 RoPE
constexpr int kPvSteps = 32;      // 16 column tiles x 2 token halves
constexpr int kKAhead = 8;        // K fragment reads in flight ahead of the score MFMAs
// V^T fragment reads in flight ahead of the PV MFMAs: 10 for the bf16 cache
// (1.1% faster than 8 on the ragged batch); 8 for fp8, where 10 spills
// registers inside the tile loop (10% slower)
template <bool kF8> constexpr int kVAhead = kF8 ? 8 : 10;
constexpr float kRefSlack = 64.f; // log2 units a head's max may exceed its reference
constexpr int kStageBytes = kWideWaves * 32768;   // epilogue staging (bf16 output)
constexpr int kFlagOffset = kStageBytes;          // redo flags, past the staging area
// fp8 cache: three bf16 tile buffers (tiles k, k+1 and k+2, which is written
// by the dequantisation during tile k's PV phase) and two staging buffers of
// codes and scales
constexpr int kWideF8Bufs = 3;
constexpr int kWideF8Area = kWideF8Bufs * kTileBytes + 2 * kF8StageBytes;
static_assert(kWideBufs * kTileBytes <= 160 * 1024, "LDS budget");
static_assert(kWideF8Area <= 160 * 1024, "LDS budget (fp8)");
static_assert(kFlagOffset + 16 <= kWideBufs * kTileBytes && kFlagOffset + 16 <= kWideF8Area,
              "flags inside the tile area");

__device__ __forceinline__ bf16x8 pack_half(const f32x16& p, int base) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[base + i];
  return r;
}

// One score MFMA with its accumulator in VGPRs.  Alone on its SIMD the kernel
// has 512 registers, so the compiler gives every MFMA the AGPR accumulator
// form; the 256 AGPRs hold O^T, and a score accumulator there would not fit.
// Written as inline assembly, the hazards the compiler would handle are
// covered here: the s_nop gives the 2 wait states an MFMA needs after a VALU
// write of its sources, a dependent MFMA that reads the previous one's result
// as its exactly overlapping accumulator needs none, and every VALU read of
// the result is at least 24 wait states after the last MFMA (score_settle, or
// the PV phase in between).
__device__ __forceinline__ void score_mfma(f32x16& acc, bf16x8 a, bf16x8 b, bool first) {
  if (first)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// fp8 dequantisation with 256 threads: item r*256 + tx (r = 0..8) of a staged
// tile is row t = 2((tx>>4)&15) + ((tx>>3)&1), chunk c = 8r + (tx&7) (a
// 16-lane group of the 16-byte LDS writes then hits 16 distinct bank quads), so a thread's row and chunk slot are the same for
// all 9 of its items and every address is a per-thread base plus an immediate:
// codes at t*576 + 8(tx&7) + 64r, the scale at 18432 + 20t + 4(r>>1), the bf16
// chunk at tile_offset(t, tx&7) + 4096r.
struct F8Thread {
  uint32_t code_off, scale_off, write_off;
  int row;
};
__device__ __forceinline__ F8Thread f8_thread(int tx) {
  F8Thread p;
  const int t = 2 * ((tx >> 4) & 15) + ((tx >> 3) & 1), x = tx & 7;
  p.row = t;
  p.code_off = uint32_t(t * kV2Row + 8 * x);
  p.scale_off = uint32_t(kF8TileBytes + t * kF8Groups * 4);
  p.write_off = uint32_t(tile_offset(t, x));
  return p;
}
__device__ __forceinline__ F8Item f8_read(uint32_t stage, const F8Thread& p, int r) {
  F8Item x;
  x.code = *reinterpret_cast<const u32x2 MLA_LDS*>((const char MLA_LDS*)(uintptr_t)(stage + p.code_off + uint32_t(64 * r)));
  x.sc = *reinterpret_cast<const float MLA_LDS*>(
      (const char MLA_LDS*)(uintptr_t)(stage + p.scale_off + uint32_t(4 * (r >> 1))));
  return x;
}
// code * scale in fp32, rounded to bf16; rows past the sequence end as zeros
// (their codes read as zero bytes, the staged range ending at the last row's
// codes, and their scale is taken as 0 here: the 16-byte rounding of the scale
// range can reach a real scale past the end)
__device__ __forceinline__ void f8_write(const F8Item& x, uint32_t buf, const F8Thread& p, bool row_ok, int r) {
  const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(int(x.code[0]), false);
  const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(int(x.code[0]), true);
  const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8(int(x.code[1]), false);
  const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8(int(x.code[1]), true);
  const float sc = row_ok ? x.sc : 0.f;
  bf16x8 v;
  v[0] = (__bf16)(f0[0] * sc); v[1] = (__bf16)(f0[1] * sc);
  v[2] = (__bf16)(f1[0] * sc); v[3] = (__bf16)(f1[1] * sc);
  v[4] = (__bf16)(f2[0] * sc); v[5] = (__bf16)(f2[1] * sc);
  v[6] = (__bf16)(f3[0] * sc); v[7] = (__bf16)(f3[1] * sc);
  *reinterpret_cast<bf16x8 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(buf + p.write_off + uint32_t(4096 * r))) = v;
}

// kF8: fp8 cache (tiles staged as codes and scales, dequantised once into the
// bf16 tile layout); else bf16 cache.
template <bool kF8>
__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_wide_kernel(V2DecodeArgs a) {
  constexpr int kTileArea = kF8 ? kWideF8Area : kWideBufs * kTileBytes;
  __shared__ __attribute__((aligned(2048))) char tiles_raw[kTileArea];
  // XCD-aware item order: block x runs on XCD x % 8
  const int n_items = a.n_items;
  const int item = (n_items & 7) == 0 ? int(blockIdx.x & 7) * (n_items >> 3) + int(blockIdx.x >> 3) : int(blockIdx.x);
  if (item >= n_items) return;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, h = lane >> 5;
  const uint32_t tiles_lds = uint32_t(reinterpret_cast<uintptr_t>(tiles_raw));
  // per-lane LDS bases are recomputed where they are used from an opaque copy
  // of the lane id, so that they hold no registers across the tile loop
  auto opaque_lane = [&]() { int ln = lane; asm volatile("" : "+v"(ln)); return ln; };
  // K fragment of latent k-step st (token lane&31, chunk 2st + (lane>>5)):
  //   (kb0 ^ 32*(st&3)) + (st>>2)*4096; RoPE k-step j: (kb0 + 32768) ^ 32j
  auto kb0_of = [](int ln) { return tile_offset(ln & 31, ln >> 5); };
  // V^T fragment (transposing reads) of column tile mt, token half ks: rows
  // 4h + (j>>2) and 8 + 4h + (j>>2) (j = lane & 15) of chunk 2((lane>>4)&1) +
  // ((j>>1)&1), byte (j&1)*8; the second row's address is the first's ^ 0x410;
  // then ^ 64*(mt&1) + (mt>>1)*4096 + ks*2048
  auto vb0_of = [](int ln) {
    return tile_offset(4 * (ln >> 5) + ((ln & 15) >> 2), 2 * ((ln >> 4) & 1) + ((ln >> 1) & 1)) + (ln & 1) * 8;
  };

  SegmentIter it;
  it.init(a.pp, a.seq_lens, item, a.meta);
  Segment sg;
  bool redo = false;          // compute the same segment again (with exact maxima)
  float m_preset = -INFINITY; // this lane's head's reference for that second pass
  while (redo || it.next(sg)) {
    const int b = uniform(sg.b);
    const int t0 = uniform(sg.t0), t1 = uniform(sg.t1);   // t0 is a multiple of the page size
    // (the divisor passes through an empty asm: the division's reciprocal is
    // then made here each segment instead of held, and spilled, across them)
    int bt_div = a.bt_div;
    asm volatile("" : "+s"(bt_div));
    const int32_t* bt = a.block_table + int64_t(b / bt_div) * a.max_pages + t0 / kV2Page;
    const char* kv = static_cast<const char*>(a.kv);
    const int ntiles = ceil_div(t1 - t0, kTileTok);
    auto tile_valid = [&](int k) { return min(kTileTok, t1 - t0 - k * kTileTok); };
    auto tile_buf = [&](int k) {
      return tiles_lds + uint32_t((kF8 ? k % kWideF8Bufs : k & (kWideBufs - 1)) * kTileBytes);
    };
    // fp8: staging buffer of tile k, and the issue of its loads (a page id
    // outside [0, num_pages) reads as zero codes and scales)
    auto stage_buf = [&](int k) { return tiles_lds + uint32_t(kWideF8Bufs * kTileBytes + (k & 1) * kF8StageBytes); };
    auto issue_f8 = [&](int k, int page_id) {
      const bool ok = unsigned(page_id) < unsigned(a.num_pages);
      const int64_t row0 = int64_t(ok ? page_id : 0) * kV2Page + (k & 1) * kTileTok;
      issue_tile_f8(kv + row0 * kV2Row, a.scales + row0 * kF8Groups, ok ? tile_valid(k) : 0, stage_buf(k), wave);
    };
    // this wavefront's row block of tile k; a page id outside [0, num_pages)
    // reads as a page of zero rows (page 0's address, empty range)
    auto start_tile = [&](TileRowLoad& ld, int k, int page_id) {
      const bool ok = unsigned(page_id) < unsigned(a.num_pages);
      const char* src = kv + int64_t(ok ? page_id : 0) * kPageBytes + (k & 1) * kTileBytes;
      ld.init(src, ok ? tile_valid(k) : 0, tile_buf(k), wave);
    };
    auto load_tile = [&](int k, int page_id) {
      TileRowLoad ld;
      start_tile(ld, k, page_id);
#pragma unroll
      for (int g = 0; g < 9; ++g) ld.group(g);
    };

    // every wavefront is done with the previous segment's LDS
    raw_barrier();
    const int page0 = load_const(bt, 0);
    const int page1 = ntiles > 2 ? load_const(bt, 1) : 0;
    // Query: this wavefront's 32 heads x 512 latent dims in four 128-dim passes
    // through a 16 KB staging area per wavefront (bf16: tile buffers 2-3, free
    // until tile 2 is issued; fp8: tile buffers 1-2, free until tile 1 is
    // dequantised), two passes at a time; the RoPE query of its heads straight
    // into registers.
    const uint32_t qstage = tiles_lds + uint32_t((kF8 ? 1 : 2) * kTileBytes + wave * 16384);
    const uint16_t* const qsrc = a.q_lat + (int64_t(b) * kV2Heads + wave * 32) * kV2Lat;
    const uint16_t* const qpe_src = a.q_pe + int64_t(b) * kV2Heads * kV2Rope;
    // latent query slices (MFMA B operand): qf[st] holds dims 16st + 8(lane>>5)
    // .. +8 of head 32w + (lane&31)
    bf16x8 qf[32];
    auto read_query = [&](int pass0) {
      const int ln = opaque_lane();
      const int r = ln & 31;
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int c = 2 * t + (ln >> 5);
          qf[8 * (pass0 + p) + t] = lds_read_b128(qstage + uint32_t(p * 8192 + r * 256 + ((c ^ (r & 15)) * 16)));
        }
    };
    // RoPE query slices of head 32w + (lane&31) (MFMA B operand of the last
    // four k-steps: dims 8(2j + (lane>>5)) .. +8)
    bf16x8 qpe_r[4];
    issue_query_pass(qsrc, qstage);
    issue_query_pass(qsrc + 128, qstage + 8192);
    {
      const int ln = opaque_lane();
      const uint16_t* const qp = qpe_src + (wave * 32 + (ln & 31)) * kV2Rope + 8 * (ln >> 5);
#pragma unroll
      for (int j = 0; j < 4; ++j) qpe_r[j] = *reinterpret_cast<const bf16x8*>(qp + 16 * j);
    }
    if constexpr (kF8) {
      issue_f8(0, page0);
      if (ntiles > 1) issue_f8(1, page0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    } else {
      load_tile(0, page0);
      if (ntiles > 1) {
        load_tile(1, page0);
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(18));   // query passes 0-1 and the RoPE query
      } else {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
      }
    }
    read_query(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));   // read before the area is refilled
    issue_query_pass(qsrc + 256, qstage);
    issue_query_pass(qsrc + 384, qstage + 8192);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    read_query(2);
    // an explicit wait tells the compiler that the query registers are ready,
    // so that it puts no waits for them inside the tile loop
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    raw_barrier();   // tiles 0-1 complete; staging areas free
    if constexpr (kF8) {
      // tiles 0-1 dequantised by all threads; then staging buffer 0 takes tile 2
      {
        const F8Thread p = f8_thread(wave * 64 + opaque_lane());
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          if (kt < ntiles) {
            const bool row_ok = p.row < tile_valid(kt);
            F8Item x[3];   // reads two items ahead of each conversion
            x[0] = f8_read(stage_buf(kt), p, 0);
            x[1] = f8_read(stage_buf(kt), p, 1);
#pragma unroll
            for (int r = 0; r < 9; ++r) {
              if (r + 2 < 9) x[(r + 2) % 3] = f8_read(stage_buf(kt), p, r + 2);
              f8_write(x[r % 3], tile_buf(kt), p, row_ok, r);
            }
          }
        }
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();
      if (ntiles > 2) issue_f8(2, page1);
    } else {
      if (ntiles > 2) load_tile(2, page1);
    }

    // ---- score MFMAs of tile kt into sn, k-steps in order; the K fragments are
    // read kKAhead steps ahead.  `before(st)` runs after step st's fragment read
    // is issued and before its MFMA (VALU work of the previous tile, done while
    // the wavefront would otherwise wait for the fragment), `between(st)` after
    // the MFMA (reads for the phase that follows).
    auto score_phase = [&](int kt, f32x16& sn, auto&& before, auto&& between) {
      const uint32_t tb = tile_buf(kt);
      const int ln = opaque_lane();
      const int kb0 = kb0_of(ln);
      const uint32_t kl = tb + uint32_t(kb0), krp = tb + uint32_t(32768 + kb0);
      auto kaddr = [&](int st) -> uint32_t {
        return st < 32 ? (kl ^ uint32_t(32 * (st & 3))) + uint32_t((st >> 2) * 4096) : krp ^ uint32_t(32 * (st - 32));
      };
      bf16x8 kr[kKAhead];
#pragma unroll
      for (int i = 0; i < kKAhead; ++i) kr[i] = lds_read_b128(kaddr(i));
#pragma unroll
      for (int st = 0; st < kScoreSteps; ++st) {
        const bf16x8 kc = kr[st % kKAhead];
        const int nx = st + kKAhead;
        if (nx < kScoreSteps) {
          kr[st % kKAhead] = lds_read_b128(kaddr(nx));
        }
        before(st);   // VALU work while this step's fragment read is outstanding
        __builtin_amdgcn_sched_barrier(0);
        score_mfma(sn, kc, st < 32 ? qf[st] : qpe_r[st - 32], st == 0);
        between(st);
        __builtin_amdgcn_sched_barrier(0);   // keep each step's order
      }
    };

    f32x16 s;
    score_phase(0, s, [](int) {}, [](int) {});
    score_settle();

    f32x16 acc[16];
    if constexpr (kF8) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = f32x16{};
    } else {
      // O^T from zero, written by MFMAs of zero operands made here (a zeroed
      // register tuple kept for the segment starts would be spilled)
      uint32_t z0, z1, z2, z3;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z0));
      asm volatile("v_mov_b32 %0, 0" : "=v"(z1));
      asm volatile("v_mov_b32 %0, 0" : "=v"(z2));
      asm volatile("v_mov_b32 %0, 0" : "=v"(z3));
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4_t{z0, z1, z2, z3});
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(z, z, f32x16{}, 0, 0, 0);
    }
    // Softmax of S(k): the lane holds head 32w + (lane&31) and 16 of the
    // tile's tokens (token 8(rr>>2) + 4h + (rr&3) in s[rr]); lane^32 the other
    // 16.  Scores are kept in the log2 domain (scale * log2 e folded into one
    // FMA); m_ref is the reference max.  The running true max of the lane's
    // raw scores, m_raw, is taken with the exponentials (the head's max, scaled,
    // at the segment's end); only the first tile's max is needed before them.
    float m_ref = m_preset, m_raw = -INFINITY, lsum = 0.f;
    int page3 = page1;   // page of tile k+3 (tiles 2j and 2j+1 share page j)

    for (int k = 0; k < ntiles; ++k) {
      {
        const int valid = tile_valid(k);
        if (valid < kTileTok) {
          const int hm = opaque_lane() >> 5;   // (not hoisted: 16 token ids would hold registers)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) {
            const int tok = 8 * (rr >> 2) + 4 * hm + (rr & 3);
            s[rr] = tok < valid ? s[rr] : -INFINITY;
          }
        }
        if (k == 0) {
          float mx = s[0];
#pragma unroll
          for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
          m_ref = fmaxf(m_ref, mx);
        }
      }
      const bool more = k + 1 < ntiles;
      const bool load3 = k + 3 < ntiles;
      // fp8: tile k+3's codes into the staging buffer that tile k+1's held
      // (dequantised in the previous tile's PV phase, before the barrier)
      if constexpr (kF8) {
        if (load3) issue_f8(k + 3, page3);
      }

      bf16x8 pk0, pk1;
      // pinned: the score passes through an empty asm where the step is placed,
      // which keeps the compiler from hoisting the exponential out of the loop
      auto softmax_step = [&](int st, bool pinned) {
        if (st < 16) {
          float x = s[st];
          if (pinned) asm volatile("" : "+v"(x));
          m_raw = fmaxf(m_raw, x);
          s[st] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, a.scale_log2, -m_ref));
        } else if (st == 16) {
          pk0 = pack_half(s, 0);
        } else if (st == 17) {
          pk1 = pack_half(s, 8);
        } else if (st == 18) {
          const float u0 = (s[0] + s[1]) + (s[2] + s[3]), u1 = (s[4] + s[5]) + (s[6] + s[7]);
          const float u2 = (s[8] + s[9]) + (s[10] + s[11]), u3 = (s[12] + s[13]) + (s[14] + s[15]);
          lsum += (u0 + u1) + (u2 + u3);
        }
      };

      // V^T fragments of tile k, read kVAhead<kF8> steps ahead (the first ones
      // during the last score steps)
      const uint32_t tb = tile_buf(k);
      uint32_t vl0 = 0;
      bf16x8 vr[kVAhead<kF8>];
      auto vfrag = [&](int st) -> bf16x8 {
        const int ks = st >> 4, mt = st & 15, p = mt & 1, n = mt >> 1;
        const uint32_t off = uint32_t(n * 4096 + ks * 2048);
        const uint32_t a0 = vl0 ^ uint32_t(64 * p);
        return lds_read_tr_pair(a0 + off, (a0 ^ 0x410u) + off);
      };
      auto v_start = [&]() { vl0 = tb + uint32_t(vb0_of(opaque_lane())); };

      // ======== phase A: scores of tile k+1 | softmax of tile k
      f32x16 sn;
      if (more) {
        score_phase(k + 1, sn, [&](int st) { softmax_step(st, true); }, [&](int st) {
          const int i = st - (kScoreSteps - kVAhead<kF8>);
          if (i == 0) v_start();
          if (i >= 0) vr[i] = vfrag(i);
        });
      } else {
#pragma unroll
        for (int st = 0; st < 19; ++st) softmax_step(st, false);
        v_start();
#pragma unroll
        for (int i = 0; i < kVAhead<kF8>; ++i) vr[i] = vfrag(i);
      }

      // ======== phase B: O^T += V^T . P^T of tile k | bf16: loads of tile k+3;
      // fp8: dequantisation of tile k+2 (9 items per thread)
      {
        const bool conv = kF8 && k + 2 < ntiles;
        if constexpr (kF8) {
          if (k == 0 && conv) {
            // tile 2's codes (issued before the loop; tile 3's stay in flight)
            if (!load3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            else if (wave < 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(5));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
            raw_barrier();
          }
        }
        TileRowLoad ld3;
        if (!kF8 && load3) start_tile(ld3, k + 3, page3);
        F8Item f8x[3];   // fp8: ring of the items whose reads are in flight
        // (computed whether or not this tile converts: a conditional definition
        // leaves the compiler carrying and spilling both versions)
        F8Thread f8p = f8_thread(wave * 64 + opaque_lane());   // (no register holds the thread id)
        const bool f8_row_ok = f8p.row < tile_valid(k + 2);
        const uint32_t f8_stage = stage_buf(k + 2), f8_buf = tile_buf(k + 2);
#pragma unroll
        for (int st = 0; st < kPvSteps; ++st) {
          const bf16x8 vc = vr[st % kVAhead<kF8>];
          if (st + kVAhead<kF8> < kPvSteps) vr[st % kVAhead<kF8>] = vfrag(st + kVAhead<kF8>);
          const int mt = st & 15;
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc, st < 16 ? pk0 : pk1, acc[mt], 0, 0, 0);
          if constexpr (kF8) {
            // item r's reads go out at step 3r - 5 (at least 0), its conversion
            // at step 3r + 1: two items' reads in flight ahead of each conversion
#pragma unroll
            for (int r = 0; r < 9; ++r) {
              if (conv && st == (3 * r - 5 < 0 ? 0 : 3 * r - 5)) f8x[r % 3] = f8_read(f8_stage, f8p, r);
            }
          }
          if (st % 3 == 1 && st / 3 < 9) {
            if constexpr (kF8) {
              if (conv) f8_write(f8x[(st / 3) % 3], f8_buf, f8p, f8_row_ok, st / 3);
            } else {
              if (load3) ld3.group(st / 3);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (more) s = sn;   // (read by VALU only after the PV phase: no settle needed)

      // ---- tile k+2 complete for every wavefront (this wavefront's loads of
      // tile k+3 stay in flight), and every wavefront done with tile k, whose
      // buffer takes tile k+4.  The page of tile k+4 is resolved before the
      // barrier: an outstanding scalar load would turn every LDS wait of the
      // next tile into a wait for all.
      page3 = k + 4 < ntiles ? load_const(bt, (k + 4) >> 1) : 0;
      if (k + 2 < ntiles) {
        if (!kF8 && load3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // fp8: tile k+3's codes
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      if (k + 2 < ntiles) raw_barrier();
    }

    // ---- epilogue.  First the workgroup's verdict on the references: every
    // wavefront is done with the tile buffers (no loads are in flight), and
    // each posts whether one of its heads' maxima outran its reference.
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    raw_barrier();
    float m_seen;
    {
      // the head's true max over the segment (the scale is positive)
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m_raw), __float_as_uint(m_raw), false, false);
      m_seen = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
      const bool bad = __any(m_seen > m_ref + kRefSlack);
      const uint32_t flags = tiles_lds + uint32_t(kFlagOffset);
      if (opaque_lane() == 0) *reinterpret_cast<int MLA_LDS*>((char MLA_LDS*)(uintptr_t)(flags + 4 * wave)) = bad;
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();
      const i32x4 f = *reinterpret_cast<const i32x4 MLA_LDS*>((const char MLA_LDS*)(uintptr_t)flags);
      redo = uniform((f[0] | f[1] | f[2] | f[3]) != 0);
    }
    if (redo) {
      m_preset = m_seen;   // the exact max of this lane's head over the segment
      continue;            // (the same segment again; that pass cannot fail)
    }
    m_preset = -INFINITY;

    // normalise, write o (final or partial) and lse
    float ltot;
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
      ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float inv = 1.f / ltot;
    const float lse_nat = (m_ref + __log2f(ltot)) * kLn2;
    const int lane_e = opaque_lane();
    const int hd_e = lane_e & 31;
    const int head_e = wave * 32 + hd_e;
    // final output of a sequence covered by this item alone, else a split
    // partial (normalised within the split); both in the output dtype
    void* const obase = sg.whole ? a.o_lat : a.o_part;
    const int64_t orow0 = int64_t(sg.whole ? b : sg.slot) * kV2Heads * kV2Lat;
    if (a.o_dt == MLA_BF16) {
      // Through LDS, so that the global stores are whole 1 KB rows: wavefront
      // w's 32 heads x 512 columns at w*32768, head hd's row at hd*1024, its
      // 16-byte chunk c (columns 8c..8c+7) at slot c ^ (hd & 15).
      uint16_t* const orows = static_cast<uint16_t*>(obase) + orow0 + int64_t(wave * 32) * kV2Lat;
      const uint32_t area = tiles_lds + uint32_t(wave * 32768);
      const uint32_t wbase = area + uint32_t(hd_e * 1024 + 8 * (lane_e >> 5));
#pragma unroll
      for (int mt = 0; mt < 16; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[mt][4 * q4 + e] * inv);
          const uint32_t ad = wbase + uint32_t((((4 * mt + q4) ^ (hd_e & 15)) * 16));
          *reinterpret_cast<bf16x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)ad) = v;
        }
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));   // own area: no barrier needed
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const bf16x8 v = lds_read_b128(area + uint32_t(j * 1024 + ((lane_e ^ (j & 15)) * 16)));
        *reinterpret_cast<bf16x8*>(orows + int64_t(j) * kV2Lat + lane_e * 8) = v;
      }
    } else {
      float* const o = static_cast<float*>(obase) + orow0 + int64_t(head_e) * kV2Lat + 4 * (lane_e >> 5);
#pragma unroll
      for (int mt = 0; mt < 16; ++mt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[mt][4 * q4 + e] * inv;
          *reinterpret_cast<f32x4*>(o + 32 * mt + 8 * q4) = v;
        }
    }
    if (h == 0) {
      if (!sg.whole) a.lse_part[int64_t(sg.slot) * kV2Heads + head_e] = lse_nat;
      else if (a.lse != nullptr) a.lse[int64_t(b) * kV2Heads + head_e] = lse_nat;
    }
  }
}

}  // namespace

hipError_t launch_decode_wide(const V2DecodeArgs& a, hipStream_t st) {
  if (a.kv_dt == MLA_FP8_E4M3) decode_wide_kernel<true><<<a.n_items, kWideThreads, 0, st>>>(a);
  else if (a.kv_dt == MLA_BF16) decode_wide_kernel<false><<<a.n_items, kWideThreads, 0, st>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace mla
