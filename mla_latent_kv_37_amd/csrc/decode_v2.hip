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
// segments (partition.h); one workgroup of 8 wavefronts serves one work item
// for all 128 heads.  Wavefronts w and w+4 run on the same SIMD.  Pair
// p = w >> 1 (wavefronts 2p, 2p+1) owns heads 32p..32p+31; member d = w & 1
// multiplies half of the 576 row dims for the scores (latent dims
// [256d, 256d+256) plus RoPE dims [32d, 32d+32)) and owns output columns
// [256d, 256d+256).  The pair adds its two fp32 partial score blocks through
// LDS, both members run the (identical) softmax, and each accumulates its 256
// columns.  Per wavefront that is 72 registers of query and 128 of
// accumulator, which fits two wavefronts per SIMD.
//
// Ping-pong schedule.  Wavefronts 0-3 (team X) and 4-7 (team Y) run the same
// per-tile program half a tile apart, so that on every SIMD one wavefront's
// score MFMAs overlap the other's softmax.  Time is cut into slots, each
// opened by a workgroup barrier.  For a segment of n tiles there are 2n+1
// slots; team X computes the partial scores of tile k in slot 2k and the
// softmax and PV product of tile k in slot 2k+1, team Y one slot later.  The
// barrier between the two slots of a tile also publishes the pair's partial
// scores.
//
// Data movement.  32-token tiles (36,864 B) are staged in LDS by buffer loads
// that write LDS directly (16 B per lane); three tile buffers.  Tile t reuses
// the buffer of tile t-3, whose last reader (team Y's PV) runs in slot 2t-4,
// so it is issued in slot 2t-3 (by team Y, once its score MFMAs are done) and
// must be complete at the barrier that opens slot 2t: about two and a half
// slots of latency cover.  The descriptor's
// size is the tile's valid bytes, so rows past the end of a sequence read as
// zeros (their scores are masked to -inf, and a zero value row keeps 0 * v
// finite even when the slot holds NaN).
// LDS tile layout: 1 KB blocks of 8 rows x 8 chunks (a chunk is 16 B = 8 bf16);
// chunk c of row t sits at (c>>3)*4096 + (t>>3)*1024 + (t&7)*128 +
// ((c&7) ^ f(t))*16 with f(t) = (t&7 with bits 1 and 2 swapped) ^ ((t>>3)&1).
// One load instruction fills one block from 8 whole 128-byte row segments
// (full cache lines), and with 64 LDS banks both the K-fragment reads (32 rows
// of one chunk) and the transposing V reads (4 rows x 32 B) are free of bank
// conflicts.  Every LDS address is a per-lane base plus an immediate.
//
// Softmax.  Scores are kept in the log2 domain (scale * log2 e folded into one
// FMA).  The running max is raised lazily: the accumulators are rescaled only
// when a head's max grows by more than 8 (a factor 256), which keeps every
// probability <= 256 in bf16 and fp32 and skips almost every rescale.
#include "decode_tile.h"

namespace mla {

constexpr int kF8NumBuf = 2;                          // bf16 tile buffers (and staging buffers)

// wait for this wavefront's staged loads of the tile before the newest
__device__ __forceinline__ void wait_tile_f8(int wave, bool newer_in_flight) {
  if (!newer_in_flight) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  else if (wave >= 4) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  else if (wave < 3) __builtin_amdgcn_s_waitcnt(waitcnt_vm(5));
  else __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
}

// Dequantise a staged fp8 tile into a bf16 tile buffer, by all 512 threads
// (items tx, tx + 512, ...; see convert_item_f8).
__device__ __forceinline__ void convert_tile_f8(uint32_t stage, uint32_t buf, int valid) {
  int tx = int(threadIdx.x);
  asm volatile("" : "+v"(tx));
#pragma unroll
  for (int r = 0; r < 5; ++r) {
    const int i = r * kDecThreads + tx;
    if (r < 4 || i < kF8Items) convert_item_f8(stage, buf, valid, i);
  }
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& p, int base) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[base + i];
  return r;
}

// kF8: fp8 cache (staged and dequantised per tile); else bf16 cache.
template <bool kF8>
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_v2_kernel(V2DecodeArgs a) {
  // bf16 tile buffers (3 for a bf16 cache; 2 plus 2 staging buffers for fp8)
  constexpr int kBufs = kF8 ? kF8NumBuf : kNumBuf;
  constexpr int kTileArea = kBufs * kTileBytes + (kF8 ? kF8NumBuf * kF8StageBytes : 0);
  // alignment: tile buffers at multiples of 2048 and the exchange area at a
  // multiple of 8192 keep the XOR address tricks below exact
  __shared__ __attribute__((aligned(2048))) char tiles_raw[kTileArea];
  __shared__ __attribute__((aligned(8192))) char xs_raw[kXsBytes];
  __shared__ __attribute__((aligned(1024))) char qpe_raw[kQpeBytes];
  // Work items w and w+1 usually share a sequence (and so its query).  Blocks
  // are dealt to the 8 XCDs round robin (block x runs on XCD x % 8), so when
  // the item count allows, XCD x gets the contiguous item range
  // [x*n/8, (x+1)*n/8) and repeated query reads hit its L2.
  const int n_items = a.n_items;
  const int item = (n_items & 7) == 0 ? int(blockIdx.x & 7) * (n_items >> 3) + int(blockIdx.x >> 3) : int(blockIdx.x);
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, h = lane >> 5;
  const int team = wave >> 2;                   // 0: wavefronts 0-3, 1: wavefronts 4-7
  const int pair = wave >> 1, dh = wave & 1;    // pair members 2p, 2p+1 are in one team
  const int head = pair * 32 + (lane & 31);
  if (item >= a.n_items) return;

  const uint32_t tiles_lds = uint32_t(reinterpret_cast<uintptr_t>(tiles_raw));
  const uint32_t xs_lds = uint32_t(reinterpret_cast<uintptr_t>(xs_raw));
  // Per-lane LDS offsets inside a tile, without the chunk-group part (a
  // wavefront-uniform 16384*dh for its latent half, 32768 for the RoPE group,
  // n*4096 for later groups), which is added as a scalar or an immediate.  The
  // chunk slot occupies address bits 4-6 and every base is a multiple of 1024,
  // so moving to chunk c ^ x within a group is an XOR of the address with 16*x.
  // K fragment of latent k-step 4n+m: token lane&31, chunk 32dh + 2m + h:
  //   kb0 ^ 32m (+ n*4096).  RoPE k-step j: chunk 64 + 4dh + 2j + h:
  //   kb0 ^ (64dh + 32j) in the RoPE group.
  auto kb0_of = [](int ln) { return tile_offset(ln & 31, ln >> 5); };
  // V^T fragment (transposing reads) of column tile 2n+p, token half ks: two
  // 8-byte reads at rows 4h + (j>>2) and 8 + 4h + (j>>2) (j = lane & 15) of
  // chunk 2(g&1) + ((j>>1)&1) (g = lane >> 4), byte (j&1)*8 of the chunk.  The
  // second row's address is the first's ^ 0x410 (next row block: +1024, which
  // flips bit 0 of the chunk swizzle: ^16); then ^ 64p + n*4096 + ks*2048.
  auto vb0_of = [](int ln) {
    return tile_offset(4 * (ln >> 5) + ((ln & 15) >> 2), 2 * ((ln >> 4) & 1) + ((ln >> 1) & 1)) + (ln & 1) * 8;
  };
  // exchange area: wavefront w writes [w*4096, w*4096 + 4096); its partner w^1
  // reads it (address ^ 4096)
  auto xs_of = [&](int ln) { return xs_lds + uint32_t(wave * 4096 + ln * 16); };
  // RoPE query of head hd, chunk c (dims 8c..8c+7) in LDS: hd*128 + ((c ^ (hd & 7)) * 16)
  const uint32_t qpe_lds = uint32_t(reinterpret_cast<uintptr_t>(qpe_raw));
  // The per-lane bases above are recomputed in every slot from an opaque copy
  // of the lane id: held across the tile loop they would cost registers that
  // two wavefronts per SIMD cannot spare.
  auto opaque_lane = [&]() { int ln = lane; asm volatile("" : "+v"(ln)); return ln; };

  SegmentIter it;
  it.init(a.pp, a.seq_lens, item, a.meta);
  Segment sg;
  while (it.next(sg)) {
    const int b = uniform(sg.b);
    const int t0 = uniform(sg.t0), t1 = uniform(sg.t1);   // t0 is a multiple of the page size
    const int32_t* bt = a.block_table + int64_t(b / a.bt_div) * a.max_pages + t0 / kV2Page;
    const char* kv = static_cast<const char*>(a.kv);
    const int ntiles = ceil_div(t1 - t0, kTileTok);
    auto tile_src = [&](int k, int page_id) -> const char* {
      return kv + int64_t(page_id) * kPageBytes + (k & 1) * kTileBytes;
    };
    auto tile_valid = [&](int k) { return min(kTileTok, t1 - t0 - k * kTileTok); };
    auto tile_buf = [&](int k) { return tiles_lds + uint32_t((k % kBufs) * kTileBytes); };
    // fp8: staging buffer of tile k, and the issue of its loads
    auto stage_buf = [&](int k) {
      return tiles_lds + uint32_t(kBufs * kTileBytes + (k % kF8NumBuf) * kF8StageBytes);
    };
    // A page id outside [0, num_pages) is read as a page of zero rows: the
    // loads then use page 0's address with an empty range.
    auto issue = [&](int k, int page_id) {
      const bool ok = unsigned(page_id) < unsigned(a.num_pages);
      const int pid = ok ? page_id : 0;
      const int dv = ok ? tile_valid(k) : 0;
      if constexpr (kF8) {
        const char* codes = kv + (int64_t(pid) * kV2Page + (k & 1) * kTileTok) * kV2Row;
        const float* sc = a.scales + (int64_t(pid) * kV2Page + (k & 1) * kTileTok) * kF8Groups;
        issue_tile_f8(codes, sc, dv, stage_buf(k), wave);
      } else {
        issue_tile(tile_src(k, pid), dv, tile_buf(k), wave);
      }
    };

    // every wavefront is done with the previous segment's tiles and scores
    raw_barrier();
    const int page_first = load_const(bt, 0);
    // query staging area of this wavefront (free until the loop's first
    // barrier): the tile buffer that no tile uses before slot 1 for wavefronts
    // 0-3, the exchange area for 4-7
    const uint32_t qstage = (wave < 4 ? tiles_lds + uint32_t((kF8 ? 1 : 2) * kTileBytes) : xs_lds) +
                            uint32_t((wave & 3) * 8192);
    const uint16_t* const qsrc = a.q_lat + (int64_t(b) * kV2Heads + pair * 32) * kV2Lat + 256 * dh;
    // query slices of head `head` (MFMA B operand: lane holds 8 consecutive dims):
    // latent dims 256*dh + 16*kk + 8*h .. +8, RoPE dims in LDS
    bf16x8 qf[16];
    auto read_query_pass = [&](int pass) {
      const int ln = opaque_lane();
      const int r = ln & 31;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int c = 2 * t + (ln >> 5);
        qf[8 * pass + t] = lds_read_b128(qstage + uint32_t(r * 256 + ((c ^ (r & 15)) * 16)));
      }
    };
    // pass 0 and the RoPE query, then tile 0; wait for the first two only
    issue_query_pass(qsrc, qstage);
    issue_query_pe(a.q_pe + int64_t(b) * kV2Heads * kV2Rope, qpe_lds, wave);
    issue(0, page_first);
    if constexpr (kF8) wait_tile_f8(wave, true);
    else wait_tile(wave, true);
    read_query_pass(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));   // read before the area is refilled
    issue_query_pass(qsrc + 128, qstage);
    // bf16: tile 1 goes out before the wait, so only pass 1 and tile 0 are waited for
    if (!kF8 && ntiles > 1) {
      issue(1, page_first);
      wait_tile(wave, true);
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    read_query_pass(1);
    // an explicit wait here tells the compiler that the query registers are
    // ready, so it puts no waits for them inside the tile loop
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    if constexpr (kF8) {
      // tile 0's staged codes visible to all, dequantised before slot 0
      raw_barrier();
      convert_tile_f8(stage_buf(0), tile_buf(0), tile_valid(0));
    }
    if (kF8 && ntiles > 1) issue(1, page_first);
    // page of the next tile to issue (tile 2); loaded a slot before its use
    int page_next = ntiles > 2 ? load_const(bt, 1) : 0;

    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
    float m_run = -INFINITY, lsum = 0.f;

    // Opening of slot j (the same in every wavefront): wait for this
    // wavefront's loads that the slot needs, barrier (fp8: then dequantise the
    // tile that slot j starts), and after the slot's work prefetch the page id
    // of the next tile to issue.
    // bf16: tile t is issued in slot 2t-3 (after team Y's score MFMAs) and read
    //       from slot 2t on.
    // fp8:  tile t is issued in slot 2t-4 (after team X's score MFMAs),
    //       dequantised in slot 2t-1 and read from slot 2t on (its bf16 buffer's
    //       previous tile, t-2, was last read in slot 2t-2; its staging
    //       buffer's, dequantised in slot 2t-5).
    auto open_slot = [&](int j) {
      if constexpr (kF8) {
        const int tc = (j + 1) >> 1;
        if ((j & 1) && tc < ntiles) wait_tile_f8(wave, tc + 1 < ntiles);
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
        raw_barrier();
        if ((j & 1) && tc < ntiles) {
          convert_tile_f8(stage_buf(tc), tile_buf(tc), tile_valid(tc));
        }
      } else {
        if ((j & 1) == 0 && j >= 2 && j / 2 < ntiles) wait_tile(wave, j / 2 + 1 < ntiles);
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
        raw_barrier();
      }
    };
    auto close_slot = [&](int j) {
      if constexpr (kF8) {
        if (j & 1) {
          const int tn = ((j + 1) >> 1) + 2;
          if (tn < ntiles) page_next = load_const(bt, tn >> 1);
        }
      } else {
        if ((j & 1) == 0) {
          const int tn = (j + 4) >> 1;
          if (tn < ntiles) page_next = load_const(bt, tn >> 1);
        }
      }
    };

    if (team == 1) {  // slot 0 belongs to team X alone (and issues no loads)
      open_slot(0);
      close_slot(0);
    }
    for (int k = 0; k < ntiles; ++k) {
      // ======== slot 2k + team: partial S^T of tile k over this wavefront's 288
      // row dims; fragment reads run two k-steps ahead of the (dependent) MFMA chain
      const int jq = 2 * k + team;
      open_slot(jq);
      // bf16: the score wavefront wins issue arbitration against its SIMD
      // partner during this slot (1.3-1.8% less decode time in interleaved A/B
      // runs; the fp8 kernel was 2% slower with it)
      if constexpr (!kF8) __builtin_amdgcn_s_setprio(1);
      const uint32_t tb = tile_buf(k);
      f32x16 s = {};
      {
        const int ln = opaque_lane();
        const int kb0 = kb0_of(ln);
        const uint32_t kl = tb + uint32_t(16384 * dh + kb0), krp = tb + uint32_t(32768 + kb0);
        const int hq = pair * 32 + (ln & 31);
        const uint32_t qpl = qpe_lds + uint32_t(hq * 128);
        auto kfrag = [&](int st) -> bf16x8 {
          return lds_read_b128(st < 16 ? (kl ^ uint32_t(32 * (st & 3))) + uint32_t((st >> 2) * 4096)
                                       : krp ^ uint32_t(64 * dh + 32 * (st - 16)));
        };
        // RoPE query fragment j: chunk 4dh + 2j + h of head hq
        auto qfrag = [&](int j) -> bf16x8 {
          return lds_read_b128(qpl + uint32_t(((4 * dh + 2 * j + (ln >> 5)) ^ (hq & 7)) * 16));
        };
        bf16x8 k0 = kfrag(0), k1 = kfrag(1);
#pragma unroll
        for (int st = 0; st < 18; ++st) {
          bf16x8 k2;
          if (st + 2 < 18) k2 = kfrag(st + 2);
          if (st < 16) {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[st], s, 0, 0, 0);
          } else {
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qfrag(st - 16), s, 0, 0, 0);
          }
          k0 = k1;
          k1 = k2;
          __builtin_amdgcn_sched_barrier(0);  // keep the reads two steps ahead
        }
      }
      // tile k + 2 goes out here, after the score MFMAs: from team Y (odd
      // slots) for bf16, from team X (even slots) for fp8
      if constexpr (!kF8) {
        if ((jq & 1) && k + 2 < ntiles) issue(k + 2, page_next);
      } else {
        if (!(jq & 1) && k + 2 < ntiles) issue(k + 2, page_next);
      }
      // publish it for the pair partner (read after the next barrier)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v = {s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
        *reinterpret_cast<f32x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(xs_of(opaque_lane()) + q4 * 1024)) = v;
      }
      if constexpr (!kF8) __builtin_amdgcn_s_setprio(0);
      close_slot(jq);

      // ======== slot 2k + team + 1: softmax and O^T += V^T . P^T of tile k
      open_slot(jq + 1);
      // V^T fragments of this wavefront's column half (transposing reads)
      const int lnp = opaque_lane();
      const uint32_t vl0 = tb + uint32_t(16384 * dh + vb0_of(lnp)), vl1 = vl0 ^ 0x410u;
      const uint32_t xs_peer = xs_of(lnp) ^ 4096u;
      auto vfrag = [&](int st) -> bf16x8 {
        const int ks = st >> 3, mt = st & 7, p = mt & 1, n = mt >> 1;
        const uint32_t off = uint32_t(n * 4096 + ks * 2048);
        return lds_read_tr_pair((vl0 ^ uint32_t(64 * p)) + off, (vl1 ^ uint32_t(64 * p)) + off);
      };
      // the partner's partial scores first (a wavefront's LDS reads return in
      // order), then the first V fragments, which do not depend on the softmax
      f32x4 pv[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        pv[q4] = *reinterpret_cast<const f32x4 MLA_LDS*>((const char MLA_LDS*)(uintptr_t)(xs_peer + q4 * 1024));
      bf16x8 v0 = vfrag(0), v1 = vfrag(1);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * q4 + e] += pv[q4][e];
      // online softmax (lane: head `head`, 16 of the tile's tokens; lane^32 the other 16)
      const int valid = tile_valid(k);
      if (valid < kTileTok) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int tok = 8 * (rr >> 2) + 4 * h + (rr & 3);
          s[rr] = tok < valid ? s[rr] : -INFINITY;
        }
      }
      float mx = s[0];
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
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
      // Rows 0-7 of the lane (tokens 0-15 of the tile) first; the MFMAs of that
      // token half overlap the exponentials of rows 8-15 (tokens 16-31).
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) s[rr] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rr], a.scale_log2, -m_run));
      const bf16x8 pk0 = pack8(s, 0);
      bf16x8 pk1;
#pragma unroll
      for (int st = 0; st < 16; ++st) {
        bf16x8 v2;
        if (st + 2 < 16) v2 = vfrag(st + 2);
        if (st == 8) pk1 = pack8(s, 8);
        const int mt = st & 7;
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, st < 8 ? pk0 : pk1, acc[mt], 0, 0, 0);
        if (st < 8) s[8 + st] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 + st], a.scale_log2, -m_run));
        v0 = v1;
        v1 = v2;
        __builtin_amdgcn_sched_barrier(0);  // keep this step's order: read ahead, MFMA, exponential
      }
      {
        float u0 = (s[0] + s[1]) + (s[2] + s[3]), u1 = (s[4] + s[5]) + (s[6] + s[7]);
        float u2 = (s[8] + s[9]) + (s[10] + s[11]), u3 = (s[12] + s[13]) + (s[14] + s[15]);
        lsum += (u0 + u1) + (u2 + u3);
      }
      close_slot(jq + 1);
    }
    if (team == 0) {  // the last slot belongs to team Y alone (and issues no loads)
      open_slot(2 * ntiles);
      close_slot(2 * ntiles);
    }

    // ---- epilogue: normalise, write o (final or partial) and lse
    // lane pair sum across the two row halves (a lane swap: no lane-id register)
    float ltot;
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
      ltot = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    const float inv = 1.f / ltot;
    const float lse_nat = (m_run + __log2f(ltot)) * kLn2;
    // the lane's head from an opaque lane id: output addresses built from
    // `head` itself are hoisted out of the segment loop, and the register pair
    // they hold through the tile loop is one more than the loop can spare
    const int lane_e = opaque_lane();
    const int head_e = pair * 32 + (lane_e & 31);
    const int colbase = 256 * dh + 4 * (lane_e >> 5);
    // final output of a sequence covered by this item alone, else a split
    // partial (normalised within the split); both in the output dtype
    void* const obase = sg.whole ? a.o_lat : a.o_part;
    const int64_t orow = (int64_t(sg.whole ? b : sg.slot) * kV2Heads + head_e) * kV2Lat + colbase;
    if (a.o_dt == MLA_BF16) {
      // Through LDS, so that the global stores are whole 256-byte row pieces:
      // a lane's direct stores would put 16 bytes into each of 32 rows per
      // instruction.  Two rounds, one 128-column quarter of each wavefront's
      // 256 columns per round: head hd's quarter of column half d sits at
      // d*32768 + hd*256, its 16-byte chunk c at slot c ^ (hd & 15).
      uint16_t* const orows = static_cast<uint16_t*>(obase) + int64_t(sg.whole ? b : sg.slot) * kV2Heads * kV2Lat;
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();   // every wavefront is done with the tile buffers
      // per-thread addresses from an opaque thread id, so that they are computed
      // here and not hoisted out of the segment loop (where they would hold
      // registers through the tile loop)
      int tx = int(threadIdx.x);
      asm volatile("" : "+v"(tx));
      const int hw = 32 * (tx >> 7) + (tx & 31), hh = (tx >> 5) & 1;   // head and half of this lane
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const uint32_t wbase = tiles_lds + uint32_t(dh * 32768 + hw * 256 + 8 * hh);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[4 * r + m][4 * q4 + e] * inv);
            const uint32_t ad = wbase + uint32_t((((4 * m + q4) ^ (hw & 15)) * 16));
            *reinterpret_cast<bf16x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)ad) = v;
          }
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
        raw_barrier();
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int pc = tx + kDecThreads * j;
          const int dhp = pc >> 11, hd = (pc >> 4) & 127, c = pc & 15;
          const bf16x8 v = lds_read_b128(tiles_lds + uint32_t(dhp * 32768 + hd * 256 + ((c ^ (hd & 15)) * 16)));
          *reinterpret_cast<bf16x8*>(orows + int64_t(hd) * kV2Lat + dhp * 256 + 128 * r + c * 8) = v;
        }
        if (r == 0) {
          __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
          raw_barrier();
        }
      }
    } else {
      float* o = static_cast<float*>(obase) + orow;
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
    if (h == 0 && dh == 0) {
      if (!sg.whole) a.lse_part[int64_t(sg.slot) * kV2Heads + head_e] = lse_nat;
      else if (a.lse != nullptr) a.lse[int64_t(b) * kV2Heads + head_e] = lse_nat;
    }
  }
}

hipError_t launch_decode_v2(const V2DecodeArgs& a, hipStream_t st) {
  if (a.kv_dt == MLA_FP8_E4M3) decode_v2_kernel<true><<<a.n_items, kDecThreads, 0, st>>>(a);
  else decode_v2_kernel<false><<<a.n_items, kDecThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
