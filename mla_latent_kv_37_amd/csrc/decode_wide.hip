// MLA decode at DeepSeek-V2 shapes over a bf16 cache, one wavefront per SIMD.
//
// The operation, the work items (partition.h), the split partials and the LDS
// tile layout (decode_tile.h) are those of decode_v2.hip; what differs is the
// division of the work inside a workgroup.  A workgroup has 4 wavefronts, one
// per SIMD, and wavefront w owns heads 32w..32w+31 entirely: all 576 dims of
// their scores and all 512 output columns.  Per 32-token tile it computes
//   S^T [32 tokens x 32 heads] = K [32 x 576] . Q^T [576 x 32]    (36 MFMAs)
//   O^T [512 x 32 heads]     += V^T [512 x 32] . P^T [32 x 32]    (32 MFMAs)
// on v_mfma_f32_32x32x16_bf16, with nothing exchanged between wavefronts but
// the tiles.  Alone on its SIMD, a wavefront has the whole 512-entry register
// file: the 256 accumulator registers hold O^T, the VGPRs the latent query
// (128), the scores and the fragment reads issued several MFMAs ahead of their
// use.  Those reads are what hides the LDS latency: no second wavefront shares
// the SIMD to switch to.
//
// Software pipeline of tile k (per wavefront):
//   softmax max of S(k)
//   phase A: the 36 score MFMAs of tile k+1, with the exponentials, the row
//            sums and the bf16 packing of P(k) between them
//   phase B: the 32 PV MFMAs of tile k, with the 9 loads of this wavefront's
//            row block of tile k+3 between them
//   wait for this wavefront's loads of tile k+2, barrier (tile k+2 complete;
//     every wavefront is done with tile k, whose buffer takes tile k+4)
// Four tile buffers (144 KB) and the RoPE query of all heads (16 KB) fill the
// 160 KB of LDS.
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
constexpr int kVAhead = 8;        // V^T fragment reads in flight ahead of the PV MFMAs
constexpr float kRefSlack = 64.f; // log2 units a head's max may exceed its reference
constexpr int kStageBytes = kWideWaves * 32768;   // epilogue staging (bf16 output)
constexpr int kFlagOffset = kStageBytes;          // redo flags, past the staging area
static_assert(kWideBufs * kTileBytes + kQpeBytes <= 160 * 1024, "LDS budget");
static_assert(kFlagOffset + 16 <= kWideBufs * kTileBytes, "flags inside the tile area");

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

__global__ __launch_bounds__(kWideThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_wide_kernel(V2DecodeArgs a) {
  __shared__ __attribute__((aligned(2048))) char tiles_raw[kWideBufs * kTileBytes];
  __shared__ __attribute__((aligned(1024))) char qpe_raw[kQpeBytes];
  // XCD-aware item order (as in decode_v2.hip): block x runs on XCD x % 8
  const int n_items = a.n_items;
  const int item = (n_items & 7) == 0 ? int(blockIdx.x & 7) * (n_items >> 3) + int(blockIdx.x >> 3) : int(blockIdx.x);
  if (item >= n_items) return;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, h = lane >> 5;
  const uint32_t tiles_lds = uint32_t(reinterpret_cast<uintptr_t>(tiles_raw));
  const uint32_t qpe_lds = uint32_t(reinterpret_cast<uintptr_t>(qpe_raw));
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
    const int32_t* bt = a.block_table + int64_t(b / a.bt_div) * a.max_pages + t0 / kV2Page;
    const char* kv = static_cast<const char*>(a.kv);
    const int ntiles = ceil_div(t1 - t0, kTileTok);
    auto tile_valid = [&](int k) { return min(kTileTok, t1 - t0 - k * kTileTok); };
    auto tile_buf = [&](int k) { return tiles_lds + uint32_t((k & (kWideBufs - 1)) * kTileBytes); };
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
    // through a 16 KB staging area per wavefront in tile buffers 2-3 (free
    // until tile 2 is issued), two passes at a time; the RoPE query of all heads
    // into its own area (blocks 2w, 2w+1, 2w+8, 2w+9 by wavefront w).
    const uint32_t qstage = tiles_lds + uint32_t(2 * kTileBytes + wave * 16384);
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
    issue_query_pass(qsrc, qstage);
    issue_query_pass(qsrc + 128, qstage + 8192);
    issue_query_pe(qpe_src, qpe_lds, wave);
    issue_query_pe(qpe_src, qpe_lds, wave + 4);
    load_tile(0, page0);
    if (ntiles > 1) {
      load_tile(1, page0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(18));   // query passes 0-1 and RoPE query
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
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
    raw_barrier();   // tiles 0-1 and the RoPE query complete; staging areas free
    if (ntiles > 2) load_tile(2, page1);

    // ---- score MFMAs of tile kt into sn, k-steps in order; the K fragments
    // (and for the RoPE steps the query fragments) are read kKAhead steps ahead.
    // `between(st)` runs after the MFMA of step st (VALU work of the previous
    // tile) and may issue reads for the phase that follows.
    auto score_phase = [&](int kt, f32x16& sn, auto&& between) {
      const uint32_t tb = tile_buf(kt);
      const int ln = opaque_lane();
      const int kb0 = kb0_of(ln);
      const uint32_t kl = tb + uint32_t(kb0), krp = tb + uint32_t(32768 + kb0);
      const int hq = wave * 32 + (ln & 31);
      const uint32_t qpl = qpe_lds + uint32_t(hq * 128);
      auto kaddr = [&](int st) -> uint32_t {
        return st < 32 ? (kl ^ uint32_t(32 * (st & 3))) + uint32_t((st >> 2) * 4096) : krp ^ uint32_t(32 * (st - 32));
      };
      auto qaddr = [&](int j) -> uint32_t { return qpl + uint32_t(((2 * j + (ln >> 5)) ^ (hq & 7)) * 16); };
      bf16x8 kr[kKAhead], qr[4];
#pragma unroll
      for (int i = 0; i < kKAhead; ++i) kr[i] = lds_read_b128(kaddr(i));
#pragma unroll
      for (int st = 0; st < kScoreSteps; ++st) {
        const bf16x8 kc = kr[st % kKAhead];
        const int nx = st + kKAhead;
        if (nx < kScoreSteps) {
          kr[st % kKAhead] = lds_read_b128(kaddr(nx));
          if (nx >= 32) qr[nx - 32] = lds_read_b128(qaddr(nx - 32));
        }
        score_mfma(sn, kc, st < 32 ? qf[st] : qr[st - 32], st == 0);
        between(st);
        __builtin_amdgcn_sched_barrier(0);   // keep each step's order
      }
    };

    f32x16 s;
    score_phase(0, s, [](int) {});
    score_settle();

    f32x16 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x16{};
    // Softmax of S(k): the lane holds head 32w + (lane&31) and 16 of the
    // tile's tokens (token 8(rr>>2) + 4h + (rr&3) in s[rr]); lane^32 the other
    // 16.  Scores are kept in the log2 domain (scale * log2 e folded into one
    // FMA); m_ref is the reference max, m_seen the running true max.
    float m_ref = m_preset, m_seen = -INFINITY, lsum = 0.f;
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
        float mx = s[0];
#pragma unroll
        for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
        m_seen = fmaxf(m_seen, mx);
        if (k == 0) m_ref = fmaxf(m_ref, mx);
      }
      const bool more = k + 1 < ntiles;
      const bool load3 = k + 3 < ntiles;

      bf16x8 pk0, pk1;
      auto softmax_step = [&](int st) {
        if (st < 16) {
          s[st] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[st], a.scale_log2, -m_ref));
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

      // V^T fragments of tile k, read kVAhead steps ahead (the first ones
      // during the last score steps)
      const uint32_t tb = tile_buf(k);
      uint32_t vl0 = 0;
      bf16x8 vr[kVAhead];
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
        score_phase(k + 1, sn, [&](int st) {
          softmax_step(st);
          const int i = st - (kScoreSteps - kVAhead);
          if (i == 0) v_start();
          if (i >= 0) vr[i] = vfrag(i);
        });
      } else {
#pragma unroll
        for (int st = 0; st < 19; ++st) softmax_step(st);
        v_start();
#pragma unroll
        for (int i = 0; i < kVAhead; ++i) vr[i] = vfrag(i);
      }

      // ======== phase B: O^T += V^T . P^T of tile k | loads of tile k+3
      {
        TileRowLoad ld3;
        if (load3) start_tile(ld3, k + 3, page3);
#pragma unroll
        for (int st = 0; st < kPvSteps; ++st) {
          const bf16x8 vc = vr[st % kVAhead];
          if (st + kVAhead < kPvSteps) vr[st % kVAhead] = vfrag(st + kVAhead);
          const int mt = st & 15;
          acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc, st < 16 ? pk0 : pk1, acc[mt], 0, 0, 0);
          if (st % 3 == 1 && st / 3 < 9) {
            if (load3) ld3.group(st / 3);
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
        if (load3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(9));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      if (k + 2 < ntiles) raw_barrier();
    }

    // ---- epilogue.  First the workgroup's verdict on the references: every
    // wavefront is done with the tile buffers (no loads are in flight), and
    // each posts whether one of its heads' maxima outran its reference.
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    raw_barrier();
    {
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
  if (a.kv_dt != MLA_BF16) return hipErrorInvalidValue;
  decode_wide_kernel<<<a.n_items, kWideThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
