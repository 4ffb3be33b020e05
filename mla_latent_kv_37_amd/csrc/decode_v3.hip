// MLA decode at DeepSeek-V2 shapes on gfx950 matrix cores, bf16 cache:
// 64-head teams, dimension-quarter score blocks and a reduce-scatter softmax.
//
// Shapes: n_h = 128 heads, latent d_c = 512, RoPE key d_h^R = 64: every cached
// token is one 576-wide row [c^KV | k^R] ([DeepSeek-V2 explainer] §2.2.2,
// §3.1.1).  With W^UK absorbed into the query, all heads score against the same
// row and the values are its first 512 columns, so per sequence the decode is
// two dense contractions, both on v_mfma_f32_32x32x16_bf16:
//   S^T [tokens x heads] = K [tokens x 576] . Q^T [576 x heads]
//   O^T [512 x heads]   += V^T [512 x tokens] . P^T [tokens x heads]
//
// Work decomposition.  One workgroup of 8 wavefronts serves one work item (a
// list of (sequence, token range) segments, partition.h) for all 128 heads;
// wavefronts w and w+4 share a SIMD.  Team T (wavefronts 4T..4T+3) owns heads
// 64T..64T+63 as two 32-head blocks; wavefront q = w & 3 of a team
//   - multiplies dimension quarter q of the row (latent dims 128q..128q+127 and
//     RoPE dims 16q..16q+15: 9 k-steps) for all 64 of its team's heads, so each
//     K fragment read from LDS feeds two MFMAs (18 per tile);
//   - owns, after a reduce-scatter of those partial scores through LDS, the
//     softmax of 16 heads (32(q>>1) + 16(q&1) .. +15 of its team);
//   - accumulates output columns 128q..128q+127 of all 64 team heads (16 MFMAs
//     per tile, each V fragment feeding two of them, P read from LDS).
// Per wavefront: 64 registers of latent query, 128 of output accumulator.
//
// Schedule.  Time is cut into slots opened by workgroup barriers.  Each team
// alternates an MFMA slot (PV of tile k-1, then the scores of tile k and the
// scatter of their partial sums) and a VALU slot (sum of the four partials,
// online softmax, P and rescale factors to LDS).  Team Y runs one slot behind
// team X, so on every SIMD one wavefront's MFMAs overlap the other's softmax:
//   team X: slot 2k   MFMA  (PV k-1, scores k)     slot 2k+1  VALU (softmax k)
//   team Y: slot 2k+1 MFMA  (PV k-1, scores k)     slot 2k+2  VALU (softmax k)
// A segment of n tiles takes 2n + 2 slots.
//
// Tiles.  32-token tiles (36,864 B) in three LDS buffers (decode_tile.h
// layout), filled by direct-to-LDS loads.  Tile k is read in slots 2k .. 2k+3
// (K by X then Y, V by X then Y), so tile k+2 can go into tile k-1's buffer
// from slot 2k+2 on; team Y issues it at the start of that slot (its VALU
// slot) and it is waited for before the barrier that opens slot 2k+4: two
// slots of latency cover.  Rows past the sequence end read as zeros.
//
// Partial-score exchange.  After the score MFMAs of a tile, a wavefront holds
// its dimension quarter's partial S^T for 2 x 32 heads; v_permlane16_swap
// regroups each 32-head block into two 16-head halves, the half the wavefront
// owns stays in registers and the other three go to LDS (2 KB each).  Both
// teams share one exchange area: a team writes its partials only after the
// other team has read its own, which a per-team LDS counter records (the
// reads come first in the same slot, so the wait is almost never taken).
//
// Softmax.  Log2 domain, running max raised lazily (rescale only when a
// head's max grows by more than 8, i.e. a factor 256).  The owner publishes a
// rescale factor per head and tile (exactly 1 when nothing changed); the PV
// wavefronts multiply their accumulators only when a factor differs from 1.
#include "decode_tile.h"

namespace mla {
namespace {

constexpr int kTeamHeads = 64;
// LDS map (bytes from the start of the workgroup's area)
constexpr int kOffXch = kNumBuf * kTileBytes;              // 110592: partial-score exchange
constexpr int kXchBlock = 2048;                              // one 16-head x 32-token fp32 partial
constexpr int kXchBytes = 4 * 3 * kXchBlock;                 // [owner q][source slot 0..2]
constexpr int kOffP = kOffXch + kXchBytes;                   // 135168: P, [team][64 heads][32 tok] bf16
constexpr int kPTeam = kTeamHeads * kTileTok * 2;            // 4096
constexpr int kOffQpe = kOffP + 2 * kPTeam;                  // 143360: RoPE query of the 128 heads
constexpr int kOffAlpha = kOffQpe + kQpeBytes;               // 159744: rescale factors [team][64] fp32
constexpr int kOffInvL = kOffAlpha + 2 * kTeamHeads * 4;     // 160256: 1 / softmax sum [team][64]
constexpr int kOffCnt = kOffInvL + 2 * kTeamHeads * 4;       // 160768: exchange read counters [team]
constexpr int kLdsBytes = kOffCnt + 16;
constexpr int kOffQStage = 2 * kTileBytes;                   // query staging, 8 KB per wavefront
constexpr int kOutStage = kV2Heads * kV2Lat * 2;             // bf16 output rows staged in LDS
static_assert(kOffQStage + kWaves * 8192 <= kOffQpe, "query staging overlaps the RoPE query");
static_assert(kOutStage <= kOffP, "output staging overlaps P");
static_assert(kLdsBytes <= 163840, "LDS budget");

// P of team-local head hd in LDS: 64 B per head, four 16-byte chunks, each two
// 4-token halves.  The token order follows the V^T fragments' k order (the
// transposing reads of decode_tile.h give lane half h of a 16-token step the
// tokens 4h..4h+3 and 8+4h..8+4h+3): chunk 2ks + h, half r holds tokens
// 16ks + 8r + 4h .. +3, so one 16-byte read is a P^T fragment.
__device__ __forceinline__ uint32_t p_off(int hd, int c, int hf) {
  return uint32_t(hd * 64 + ((c ^ ((hd >> 2) & 3)) * 16) + hf * 8);
}

__device__ __forceinline__ float lds_f32(uint32_t addr) {
  return *reinterpret_cast<const float MLA_LDS*>((const char MLA_LDS*)(uintptr_t)addr);
}
__device__ __forceinline__ f32x4 lds_f32x4(uint32_t addr) {
  return *reinterpret_cast<const f32x4 MLA_LDS*>((const char MLA_LDS*)(uintptr_t)addr);
}
__device__ __forceinline__ void lds_store(uint32_t addr, f32x4 v) {
  *reinterpret_cast<f32x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)addr) = v;
}

// max / sum over the four 16-lane rows (lanes l, l^16, l^32, l^48)
__device__ __forceinline__ float rows4_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace

__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_v3_kernel(V2DecodeArgs a) {
  __shared__ __attribute__((aligned(8192))) char lds_raw[kLdsBytes];
  // Work items w and w+1 usually share a sequence (and so its query).  Blocks
  // are dealt to the 8 XCDs round robin (block x runs on XCD x % 8), so when
  // the item count allows, XCD x gets the contiguous item range
  // [x*n/8, (x+1)*n/8) and repeated query reads hit its L2.
  const int n_items = a.n_items;
  const int item = (n_items & 7) == 0 ? int(blockIdx.x & 7) * (n_items >> 3) + int(blockIdx.x >> 3) : int(blockIdx.x);
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int team = wave >> 2, q = wave & 3;
  if (item >= n_items) return;

  // Arguments used only at the start or the end of a segment are read from the
  // kernel-argument segment where they are used (through a pointer the compiler
  // cannot see through), not held in scalar registers through the tile loop:
  // the loop needs every scalar register it has.
  const V2DecodeArgs MLA_CONST* const kargs = (const V2DecodeArgs MLA_CONST*)__builtin_amdgcn_kernarg_segment_ptr();
  auto K = [&]() {
    const V2DecodeArgs MLA_CONST* p = kargs;
    asm volatile("" : "+s"(p));
    return p;
  };
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(lds_raw));
  const uint32_t xch = lds + kOffXch, p_team = lds + kOffP + uint32_t(team * kPTeam);
  const uint32_t alpha_team = lds + kOffAlpha + uint32_t(team * kTeamHeads * 4);
  const uint32_t invl_team = lds + kOffInvL + uint32_t(team * kTeamHeads * 4);
  int MLA_LDS* const cnt = (int MLA_LDS*)(uintptr_t)(lds + kOffCnt);
  // per-lane values are recomputed from an opaque copy of the lane id where
  // they are used: held across the tile loop they would cost registers that
  // two wavefronts per SIMD cannot spare
  auto opaque_lane = [&]() { int ln = lane; asm volatile("" : "+v"(ln)); return ln; };

  SegmentIter it;
  it.init(a.pp, a.seq_lens, item, a.meta);
  Segment sg;
  while (it.next(sg)) {
    const int b = uniform(sg.b);
    const int t0 = uniform(sg.t0), t1 = uniform(sg.t1);   // t0 is a multiple of the page size
    const int32_t* bt = a.block_table + int64_t(b) * a.max_pages + t0 / kV2Page;
    const char* kv = static_cast<const char*>(a.kv);
    const int ntiles = ceil_div(t1 - t0, kTileTok);
    auto tile_valid = [&](int k) { return min(kTileTok, t1 - t0 - k * kTileTok); };
    auto tile_buf = [&](int k) { return lds + uint32_t((k % kNumBuf) * kTileBytes); };
    // A page id outside [0, num_pages) is read as a page of zero rows: the
    // loads then use page 0's address with an empty range.
    auto issue = [&](int k, int page_id) {
      const bool ok = unsigned(page_id) < unsigned(a.num_pages);
      issue_tile(kv + int64_t(ok ? page_id : 0) * kPageBytes + (k & 1) * kTileBytes, ok ? tile_valid(k) : 0,
                 tile_buf(k), wave);
    };

    // every wavefront is done with the previous segment's LDS use
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    raw_barrier();
    if (wave == 0) {
      const int ln = opaque_lane();
      if (ln < 2) cnt[ln] = 0;
    }
    const int page_first = load_const(bt, 0);
    // Query staging (the area of tile buffer 2 and beyond, free until slot 0):
    // pass hb copies this wavefront's 32 x 128 latent dims of head block hb
    // (rows 64T + 32hb + j, dims 128q..128q+127) by whole-line loads, then reads
    // them back in the MFMA operand layout: qf[8hb + ks] = dims 128q + 16ks +
    // 8(lane>>5) .. +7 of head 64T + 32hb + (lane&31).
    const uint32_t qstage = lds + uint32_t(kOffQStage + wave * 8192);
    const uint16_t* const qsrc = K()->q_lat + (int64_t(b) * kV2Heads + team * kTeamHeads) * kV2Lat + 128 * q;
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
    issue_query_pass(qsrc, qstage);
    issue_query_pe(K()->q_pe + int64_t(b) * kV2Heads * kV2Rope, lds + kOffQpe, wave);
    issue(0, page_first);
    wait_tile(wave, true);                          // query pass 0 and the RoPE query (tile 0 may fly)
    read_query_pass(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));    // read before the area is refilled
    issue_query_pass(qsrc + 32 * kV2Lat, qstage);
    if (ntiles > 1) {
      issue(1, page_first);
      wait_tile(wave, true);                        // pass 1 and tile 0
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    read_query_pass(1);
    // an explicit wait tells the compiler the query registers are ready, so it
    // puts no waits for them inside the tile loop
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    int page_next = ntiles > 2 ? load_const(bt, 1) : 0;   // page of the next tile to issue (tile 2)

    f32x16 acc[2][4];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[hb][cb] = f32x16{};
    f32x4 own[2];                 // this wavefront's own quarter of the tile's partial scores
    float m_run = -INFINITY, lsum = 0.f;

    const int nslots = 2 * ntiles + 2;
    for (int j = 0; j < nslots; ++j) {
      // barrier opening slot j: team Y's loads of tile j/2 (issued in slot j-2)
      // are complete before team X reads it in slot j
      if (team == 1 && (j & 1) == 0 && j >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();
      const int u = j - team;
      if (u < 0 || u > 2 * ntiles) continue;
      const int k = u >> 1;
      if ((u & 1) == 0) {
        // ================= MFMA slot: scores of tile k, then PV of tile k-1 with the
        // scatter of the scores' partial sums interleaved
        f32x16 s0 = {}, s1 = {};
        const bool has_scores = k < ntiles, has_pv = k >= 1;
        if (has_scores) {
          const uint32_t tb = tile_buf(k);
          const int ln = opaque_lane();
          const int kb0 = tile_offset(ln & 31, ln >> 5);
          const uint32_t kl = tb + uint32_t(kb0 + 2 * q * 4096), krp = tb + uint32_t(32768 + kb0);
          // K fragment of latent k-step ks (chunks 16q + 2ks + (lane>>5)) or,
          // for ks = 8, of RoPE chunks 64 + 2q + (lane>>5); read two steps ahead
          auto kfrag = [&](int ks) -> bf16x8 {
            return lds_read_b128(ks < 8 ? (kl ^ uint32_t(32 * (ks & 3))) + uint32_t((ks >> 2) * 4096)
                                        : krp ^ uint32_t(32 * q));
          };
          // RoPE query fragment of head block hb: head 64T + 32hb + (lane&31), chunk 2q + (lane>>5)
          auto qpefrag = [&](int hb) -> bf16x8 {
            const int hd = team * kTeamHeads + 32 * hb + (ln & 31);
            return lds_read_b128(lds + uint32_t(kOffQpe + hd * 128 + (((2 * q + (ln >> 5)) ^ (hd & 7)) * 16)));
          };
          bf16x8 k0 = kfrag(0), k1 = kfrag(1);
#pragma unroll
          for (int ks = 0; ks < 9; ++ks) {
            bf16x8 k2;
            if (ks + 2 < 9) k2 = kfrag(ks + 2);
            if (ks < 8) {
              s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[ks], s0, 0, 0, 0);
              s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[8 + ks], s1, 0, 0, 0);
            } else {
              s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qpefrag(0), s0, 0, 0, 0);
              s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qpefrag(1), s1, 0, 0, 0);
            }
            k0 = k1;
            k1 = k2;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // Scatter of head block hb's partial scores, in place: permlane16_swap of
        // registers e and e+8 leaves in all 64 lanes heads (lane&15) of the
        // block's first half in register e and of its second half in register
        // e+8 (e = 0..7), lane row rho = lane>>4 holding tokens 8(e>>2) + (e&3) +
        // 16(rho&1) + 4(rho>>1).  Half u of block hb belongs to wavefront 2hb + u
        // of the team: the wavefront keeps its own half and writes the others
        // to their owners' exchange blocks (source slot ((q - owner) & 3) - 1).
        auto permute = [&](f32x16& sv) __attribute__((always_inline)) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(sv[e]), __float_as_uint(sv[e + 8]),
                                                             false, false);
            sv[e] = __uint_as_float(sw[0]);
            sv[e + 8] = __uint_as_float(sw[1]);
          }
        };
        auto half = [](const f32x16& sv, int u, int r) {
          return f32x4{sv[8 * u + 4 * r], sv[8 * u + 4 * r + 1], sv[8 * u + 4 * r + 2], sv[8 * u + 4 * r + 3]};
        };
        auto write_part = [&](int o, f32x4 v0, f32x4 v1) __attribute__((always_inline)) {
          const int ln = opaque_lane();
          const uint32_t blk = xch + uint32_t((o * 3 + (((q - o) & 3) - 1)) * kXchBlock);
          lds_store(blk + uint32_t(ln * 16), v0);
          lds_store(blk + uint32_t(1024 + ln * 16), v1);
        };
        // the halves this wavefront does not own go to their owners
        auto deliver = [&](const f32x16& sv, int hb) __attribute__((always_inline)) {
          if ((q >> 1) == hb) {
            if (q & 1) write_part(2 * hb, half(sv, 0, 0), half(sv, 0, 1));
            else write_part(2 * hb + 1, half(sv, 1, 0), half(sv, 1, 1));
          } else {
            write_part(2 * hb, half(sv, 0, 0), half(sv, 0, 1));
            write_part(2 * hb + 1, half(sv, 1, 0), half(sv, 1, 1));
          }
        };
        // the other team must have read its previous partials from the shared
        // area: team X writing tile k waits for team Y's reads of tiles
        // 0..k-1, team Y for team X's reads of tiles 0..k
        auto wait_area = [&]() __attribute__((always_inline)) {
          const int target = 4 * (k + team);
          while (__atomic_load_n((volatile int MLA_LDS*)(cnt + (1 - team)), __ATOMIC_RELAXED) < target)
            __builtin_amdgcn_s_sleep(1);
        };
        // PV of tile k-1
        const uint32_t tbv = tile_buf(k - 1);
        const int lnv = opaque_lane();
        // V^T fragment of column block C = 4q + cb, token half ks (transposing reads)
        const uint32_t vl0 = tbv + uint32_t(tile_offset(4 * (lnv >> 5) + ((lnv & 15) >> 2),
                                                        2 * ((lnv >> 4) & 1) + ((lnv >> 1) & 1)) +
                                            (lnv & 1) * 8);
        const uint32_t vl1 = vl0 ^ 0x410u;
        auto vfrag = [&](int st) __attribute__((always_inline)) -> bf16x8 {
          const int ks = st >> 2, C = 4 * q + (st & 3);
          const uint32_t off = uint32_t((C >> 1) * 4096 + ks * 2048);
          const uint32_t x = uint32_t(64 * (C & 1));
          return lds_read_tr_pair((vl0 ^ x) + off, (vl1 ^ x) + off);
        };
        // P^T fragment of head block hb, token half ks: head 32hb + (lane&31),
        // tokens 16ks + 4(lane>>5) + {0..3, 8..11}
        auto pfrag = [&](int hb, int ks) __attribute__((always_inline)) -> bf16x8 {
          const int hd = 32 * hb + (lnv & 31);
          return lds_read_b128(p_team + p_off(hd, 2 * ks + (lnv >> 5), 0));
        };
        if (has_scores) {
          // the own half is selected unconditionally (so that the previous
          // tile's is dead during the score MFMAs), block 0's before block 1
          // is permuted, so that block 0's registers are free by then
          permute(s0);
          wait_area();
          deliver(s0, 0);
          f32x4 c0[2];
#pragma unroll
          for (int r = 0; r < 2; ++r) c0[r] = (q & 1) ? half(s0, 1, r) : half(s0, 0, r);
          permute(s1);
          deliver(s1, 1);
#pragma unroll
          for (int r = 0; r < 2; ++r) own[r] = (q >> 1) ? ((q & 1) ? half(s1, 1, r) : half(s1, 0, r)) : c0[r];
        } else {
          own[0] = own[1] = f32x4{};   // no softmax follows this slot
        }
        if (has_pv) {
          bf16x8 p0 = pfrag(0, 0), p1 = pfrag(1, 0);
          bf16x8 v0 = vfrag(0), v1 = vfrag(1);
          // rescale factors of tile k-1's softmax for this lane's head in each block
          const float al0 = lds_f32(alpha_team + uint32_t((lnv & 31) * 4));
          const float al1 = lds_f32(alpha_team + uint32_t(128 + (lnv & 31) * 4));
          if (__any(al0 != 1.f || al1 != 1.f)) {
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
              acc[0][cb] *= al0;
              acc[1][cb] *= al1;
            }
          }
#pragma unroll
          for (int st = 0; st < 8; ++st) {
            bf16x8 v2;
            if (st + 2 < 8) v2 = vfrag(st + 2);
            bf16x8 pn0, pn1;
            if (st == 2) {
              pn0 = pfrag(0, 1);
              pn1 = pfrag(1, 1);
            }
            const int cb = st & 3;
            acc[0][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, p0, acc[0][cb], 0, 0, 0);
            acc[1][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, p1, acc[1][cb], 0, 0, 0);
            if (st == 3) {
              p0 = pn0;
              p1 = pn1;
            }
            v0 = v1;
            v1 = v2;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
        // ================= VALU slot: softmax of tile k (team Y first issues tile k+2)
        if (team == 1 && k + 2 < ntiles) issue(k + 2, page_next);
        const int ln = opaque_lane();
        f32x4 part[3][2];
#pragma unroll
        for (int s = 0; s < 3; ++s) {
          const uint32_t blk = xch + uint32_t((q * 3 + s) * kXchBlock);
          part[s][0] = lds_f32x4(blk + uint32_t(ln * 16));
          part[s][1] = lds_f32x4(blk + uint32_t(1024 + ln * 16));
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
        if (ln == 0) __atomic_fetch_add(cnt + team, 1, __ATOMIC_RELAXED);
        // the four quarters summed in a fixed order: own, then source slots 0, 1, 2
        // (slot s holds wavefront (q + s + 1) & 3); one wavefront owns a head, so
        // every head's sum has one order
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[e] = ((own[e >> 2][e & 3] + part[0][e >> 2][e & 3]) + part[1][e >> 2][e & 3]) + part[2][e >> 2][e & 3];
        const int rho = ln >> 4;
        const int tbase = 16 * (rho & 1) + 4 * (rho >> 1);   // token of register 0
        const int valid = tile_valid(k);
        if (valid < kTileTok) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (tbase + 8 * (e >> 2) + (e & 3)) < valid ? x[e] : -INFINITY;
        }
        float mx = x[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
        mx = rows4_max(mx);
        const float m_new = fmaxf(m_run, mx * a.scale_log2);
        float alpha = 1.f;
        if (__any(m_new > m_run + kRescaleSlack)) {
          alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          lsum *= alpha;
          m_run = m_new;
        }
        const int hd = 16 * q + (ln & 15);   // team-local head of this lane
        if (ln < 16) *reinterpret_cast<float MLA_LDS*>((char MLA_LDS*)(uintptr_t)(alpha_team + uint32_t(hd * 4))) = alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], a.scale_log2, -m_run));
        lsum += ((x[0] + x[1]) + (x[2] + x[3])) + ((x[4] + x[5]) + (x[6] + x[7]));
        // run r of this lane (tokens 16(rho&1) + 8r + 4(rho>>1) .. +3) is half r of
        // chunk 2(rho&1) + (rho>>1)
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          bf16x4 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = (__bf16)x[4 * run + e];
          *reinterpret_cast<bf16x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(
              p_team + p_off(hd, 2 * (rho & 1) + (rho >> 1), run))) = pv;
        }
        if (k == ntiles - 1) {
          // last tile: 1/l for the output scaling, lse of this segment
          const float ltot = rows4_sum(lsum);
          const float lse_nat = (m_run + __log2f(ltot)) * kLn2;
          if (ln < 16) {
            *reinterpret_cast<float MLA_LDS*>((char MLA_LDS*)(uintptr_t)(invl_team + uint32_t(hd * 4))) = 1.f / ltot;
            const int head = team * kTeamHeads + hd;
            float* const lse_out = sg.whole ? K()->lse : K()->lse_part;
            if (lse_out != nullptr) lse_out[int64_t(sg.whole ? b : sg.slot) * kV2Heads + head] = lse_nat;
          }
        }
        // page of the tile that the next VALU slot issues (tile k+3)
        if (k + 3 < ntiles) page_next = load_const(bt, (k + 3) >> 1);
      }
    }

    // ---- epilogue: normalise and write o (final output, or this split's partial)
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
    raw_barrier();   // every wavefront is done with the tiles; 1/l of every head is in LDS
    const int lane_e = opaque_lane();
    const float inv0 = lds_f32(invl_team + uint32_t((lane_e & 31) * 4));
    const float inv1 = lds_f32(invl_team + uint32_t(128 + (lane_e & 31) * 4));
    const int64_t orow = int64_t(sg.whole ? b : sg.slot) * kV2Heads;   // first output row of the segment
    void* const obase = sg.whole ? K()->o_lat : K()->o_part;
    if (K()->o_dt == MLA_BF16) {
      // Through LDS, so that the global stores are whole 1 KB rows: head hd's row
      // at hd*1024, its 16-byte chunk c at slot c ^ (hd & 63).
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int hd = team * kTeamHeads + 32 * hb + (lane_e & 31);
        const float inv = hb ? inv1 : inv0;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[hb][cb][4 * g + e] * inv);
            const int c = 16 * q + 4 * cb + g;   // column chunk: cols 8c + 4(lane>>5) .. +3
            *reinterpret_cast<bf16x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(
                lds + uint32_t(hd * 1024 + ((c ^ (hd & 63)) * 16) + (lane_e >> 5) * 8))) = v;
          }
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();
      int tx = int(threadIdx.x);
      asm volatile("" : "+v"(tx));
      uint16_t* const orows = static_cast<uint16_t*>(obase) + orow * kV2Lat;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pc = tx + kDecThreads * i;
        const int hd = pc >> 6, c = pc & 63;
        const bf16x8 v = lds_read_b128(lds + uint32_t(hd * 1024 + ((c ^ (hd & 63)) * 16)));
        *reinterpret_cast<bf16x8*>(orows + int64_t(hd) * kV2Lat + c * 8) = v;
      }
    } else {
      float* const o = static_cast<float*>(obase) + orow * kV2Lat;
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int hd = team * kTeamHeads + 32 * hb + (lane_e & 31);
        const float inv = hb ? inv1 : inv0;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[hb][cb][4 * g + e] * inv;
            const int col = 128 * q + 32 * cb + 8 * g + 4 * (lane_e >> 5);
            *reinterpret_cast<f32x4*>(o + int64_t(hd) * kV2Lat + col) = v;
          }
      }
    }
  }
}

hipError_t launch_decode_v3(const V2DecodeArgs& a, hipStream_t st) {
  decode_v3_kernel<<<a.n_items, kDecThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace mla
