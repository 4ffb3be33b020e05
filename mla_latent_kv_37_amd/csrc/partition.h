// Enumeration of the (sequence, token range) segments a work item processes.
//
// Three partitions (mla_partition_t):
//   whole:    item b = sequence b.
//   fixed:    item b*S + s = tokens [s*L, min((s+1)*L, T_b)) of sequence b.
//   balanced: the cost stream of mla_common.h (the pages of all sequences in
//             sequence order, kSegCost units between consecutive non-empty
//             sequences; C units) is cut into W = min(num_parts, total pages)
//             contiguous parts; item w takes units [floor(w*C/W),
//             floor((w+1)*C/W)), i.e. the pages inside that range, and may span
//             sequences.  Item w's share of sequence b uses slot w + b (unique
//             because both w and b grow along the stream).  The item holding a
//             sequence's first page records w in meta[b]; the one holding its
//             last page records w in meta[B + b], so the merge knows the slots;
//             every item in between holds at least one page of that sequence
//             (parts are at least one unit long).
#pragma once

#include "mla_common.h"

namespace mla {

// Sums and scans over one wavefront (64 lanes), without LDS or barriers.
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Iterates over the segments of one work item, in order:
//   SegmentIter it; it.init(pp, seq_lens, item, meta);
//   Segment sg; while (it.next(sg)) { ... }
// Every wavefront computes the (uniform) results on its own with wavefront
// scans over the sequences, 64 at a time; all threads of the block must call
// init() and next() together.
struct SegmentIter {
  PartParams pp;
  const int32_t* seq_lens;
  int32_t* meta;
  int item;
  int b;          // next sequence to look at
  int64_t S;      // its first unit in the cost stream (balanced)
  int64_t p0, p1; // the item's unit range (balanced)
  bool done;

  __device__ __forceinline__ void init(const PartParams& pp_, const int32_t* __restrict__ seq_lens_, int item_,
                                       int32_t* meta_) {
    pp = pp_; seq_lens = seq_lens_; meta = meta_; item = item_;
    done = false; b = 0; S = 0; p0 = p1 = 0;
    if (pp.mode != PART_BALANCED) return;
    const int B = pp.batch, page = pp.page_size;
    const int lane = threadIdx.x & 63;
    auto pages_of = [&](int i) { return i < B ? ceil_div(seq_len_of(seq_lens[seq_len_index(i, pp)], i, pp), page) : 0; };
    // total pages P and non-empty sequences m of the batch
    int P = 0, m = 0;
    for (int base = 0; base < B; base += 64) {
      const int np = pages_of(base + lane);
      P += wave_sum(np);
      m += wave_sum(np > 0 ? 1 : 0);
    }
    P = __builtin_amdgcn_readfirstlane(P);
    m = __builtin_amdgcn_readfirstlane(m);
    const int W = min(pp.num_parts, P);
    if (P == 0 || item >= W) { done = true; return; }
    const int64_t C = cost_units(P, m);
    p0 = part_start(item, C, W);
    p1 = part_start(item + 1, C, W);
    // the sequence whose pages and following extra units [u_b, u_b + n_b +
    // kSegCost) hold unit p0
    int fb = -1, fS = 0, offset = 0;
    for (int base = 0; base < B; base += 64) {
      const int np = pages_of(base + lane);
      const int cu = np > 0 ? np + kSegCost : 0;
      const int incl = wave_inclusive_scan(cu), excl = incl - cu;
      const bool hit = np > 0 && offset + excl <= p0 && p0 < offset + incl;
      const unsigned long long m = __ballot(hit);
      if (m != 0ull) {
        const int l = __ffsll(m) - 1;
        fb = base + l;
        fS = offset + __shfl(excl, l, 64);
        break;
      }
      offset += __shfl(incl, 63, 64);
    }
    b = __builtin_amdgcn_readfirstlane(fb);
    S = __builtin_amdgcn_readfirstlane(fS);
    if (b < 0) done = true;
  }

  __device__ __forceinline__ bool next(Segment& sg) {
    if (done) return false;
    const int B = pp.batch, page = pp.page_size;
    if (pp.mode == PART_WHOLE) {
      done = true;
      if (item >= B) return false;
      const int T = seq_len_of(load_const(seq_lens, seq_len_index(item, pp)), item, pp);
      if (T <= 0) return false;
      sg = Segment{item, 0, T, -1, true};
      return true;
    }
    if (pp.mode == PART_FIXED) {
      done = true;
      const int bb = item / pp.fixed_slots, sp = item % pp.fixed_slots;
      if (bb >= B) return false;
      const int T = seq_len_of(load_const(seq_lens, seq_len_index(bb, pp)), bb, pp);
      const int n = ceil_div(T, pp.split_tokens);
      if (sp >= n) return false;
      sg = Segment{bb, sp * pp.split_tokens, min(T, (sp + 1) * pp.split_tokens), item, n == 1};
      return true;
    }
    while (b < B && S < p1) {
      const int T = seq_len_of(load_const(seq_lens, seq_len_index(b, pp)), b, pp);
      const int np = ceil_div(T, page);
      const int64_t Sb = S;
      const int bb = b;
      ++b;
      if (np == 0) continue;
      S += np + kSegCost;
      const int64_t lo = Sb > p0 ? Sb : p0, hi = Sb + np < p1 ? Sb + np : p1;
      if (hi <= lo) continue;   // p0 lies in the extra units after this sequence
      sg.b = bb;
      sg.t0 = int(lo - Sb) * page;
      sg.t1 = min(T, int(hi - Sb) * page);
      sg.slot = item + bb;
      sg.whole = (Sb >= p0) && (Sb + np <= p1);
      if (meta != nullptr && threadIdx.x == 0) {
        // the stored value is moved to a vector register here, not before the
        // caller's loop (where that register would be held, or spilled, throughout)
        int w = item;
        asm volatile("" : "+s"(w));
        // (and so is the store's vector offset, which the compiler would
        // otherwise make once and hold across the caller's loop)
        int off0, off1;
        asm volatile("v_mov_b32 %0, %1" : "=v"(off0) : "s"(bb * 4));
        asm volatile("v_mov_b32 %0, %1" : "=v"(off1) : "s"((B + bb) * 4));
        if (Sb >= p0) *reinterpret_cast<int32_t*>(reinterpret_cast<char*>(meta) + off0) = w;
        if (Sb + np <= p1) *reinterpret_cast<int32_t*>(reinterpret_cast<char*>(meta) + off1) = w;
      }
      return true;
    }
    done = true;
    return false;
  }
};

}  // namespace mla
