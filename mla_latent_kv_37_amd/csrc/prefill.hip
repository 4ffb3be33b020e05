// MLA prefill: attention of a batch of new prompt tokens over their sequences'
// paged latent cache, in the non-absorbed form.
//
// For a long run of new tokens the absorbed form (scores against the 576-wide
// cached rows, outputs in the 512-wide latent space) costs 2 x 1088 flops per
// (query, cached token, head); up-projecting the keys and values once,
//   k^C_{j,i} = W^UK_i c^KV_j,  v_{j,i} = W^UV_i c^KV_j   (DeepSeek-V2 explainer
//   (一文通透DeepSeek-V2) §2.2.1, the per-head keys and values of the latent),
// costs 2 x 2 x 512 x 128 flops per (cached token, head) once, and the
// attention itself 2 x (192 + 128) per (query, cached token, head) with
//   s = [q^C_i; q^R_i] . [k^C_{j,i}; k^R_j] / sqrt(d_h + d_h^R)
// (deepseek(2)——deepseek 關鍵技術 §1; a new token at position p attends to the
// cached positions 0..p).  Past a few hundred new tokens per sequence the
// up-projection is the cheaper route (the V2 technical report describes
// prompt processing in this form; the absorbed form is the decode's).
//
// Four launches, in stream order, all on one workspace (api.hip lays it out):
//   scan:    cu[b] = sum of the clamped lengths of sequences < b (int32).
//   gather:  C[g] = the cached row [c^KV | k^R] of global token g (sequence b,
//            position g - cu[b]) in bf16, dequantised for an fp8 cache; rows
//            past the batch's tokens and rows of a page id outside the cache
//            are zeros.  C is dense, so the two kernels after it need no
//            block table.
//   kv:      KV[s][g] = W_s . c^KV_g for the 2 n_h slabs s of 128 output
//            features (slab i < n_h: W^UK_i, slab n_h + i: W^UV_i), a dense
//            product [2 n_h 128 x 512] x [512 x rows] on MFMA.
//   attn:    per (head, block of 256 new tokens of one sequence), causal
//            attention over the keys [KV[i][g] | C[g][512:576]] and values
//            KV[n_h + i][g] with an online softmax, on MFMA.
#include "decode_tile.h"

namespace mla {
namespace {

constexpr int kPfHead = 128, kPfLat = 512, kPfRope = 64, kPfRow = 576, kPfPage = 64;
constexpr int kPfRowBytes = kPfRow * 2;   // 1152: one gathered row of C

// ---------------------------------------------------------------------------
// scan: one workgroup of 256 threads walks the batch 256 sequences at a time.
__global__ __launch_bounds__(256) void prefill_scan_kernel(PrefillArgs a) {
  __shared__ int part[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int64_t run = 0;
  for (int base = 0; base < a.batch; base += 256) {
    const int b = base + int(threadIdx.x);
    int T = b < a.batch ? a.seq_lens[b] : 0;
    T = T < 0 ? 0 : (T > a.max_tokens ? a.max_tokens : T);
    // inclusive scan within the wavefront, then across the 4 wavefronts
    int v = T;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      if (lane >= off) v += t;
    }
    if (lane == 63) part[wave] = v;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += part[w];
    const int64_t excl = run + before + v - T;
    if (b < a.batch) a.cu[b] = int(excl < a.total_kv ? excl : a.total_kv);
    run += part[0] + part[1] + part[2] + part[3];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.cu[a.batch] = int(run < a.total_kv ? run : a.total_kv);
}

// ---------------------------------------------------------------------------
// gather: workgroup x fills rows 32x..32x+31 of C (72 chunks of 8 values each).
__global__ __launch_bounds__(256) void prefill_gather_kernel(PrefillArgs a) {
  __shared__ int64_t src_row[32];   // cache row (page * page_size + slot), -1: zeros
  const int g0 = blockIdx.x * 32;
  if (threadIdx.x < 32) {
    const int g = g0 + int(threadIdx.x);
    int64_t row = -1;
    if (g < a.cu[a.batch]) {
      // the sequence holding global token g: the last b with cu[b] <= g
      int lo = 0, hi = a.batch;   // cu[lo] <= g < cu[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.cu[mid] <= g) lo = mid;
        else hi = mid;
      }
      const int j = g - a.cu[lo];
      const int page = a.block_table[int64_t(lo) * a.max_pages + j / kPfPage];
      if (unsigned(page) < unsigned(a.num_pages)) row = int64_t(page) * kPfPage + (j % kPfPage);
    }
    src_row[threadIdx.x] = row;
  }
  __syncthreads();
  uint16_t* out = a.c_rows + int64_t(g0) * kPfRow;
  for (int e = threadIdx.x; e < 32 * 72; e += 256) {
    const int t = e / 72, c = e % 72;
    const int64_t row = src_row[t];
    bf16x8 v = bf16x8{};
    if (row >= 0) {
      if (a.kv_dt == MLA_BF16) {
        v = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(a.kv) + row * kPfRow + c * 8);
      } else {
        // fp8: code * scale of the token's 128-channel group, in fp32, rounded to bf16
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 code = *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(a.kv) + row * kPfRow + c * 8);
        const float sc = a.scales[row * 5 + (c >> 4)];
        const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8(int(code[0]), false);
        const auto f1 = __builtin_amdgcn_cvt_pk_f32_fp8(int(code[0]), true);
        const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8(int(code[1]), false);
        const auto f3 = __builtin_amdgcn_cvt_pk_f32_fp8(int(code[1]), true);
        v[0] = (__bf16)(f0[0] * sc); v[1] = (__bf16)(f0[1] * sc);
        v[2] = (__bf16)(f1[0] * sc); v[3] = (__bf16)(f1[1] * sc);
        v[4] = (__bf16)(f2[0] * sc); v[5] = (__bf16)(f2[1] * sc);
        v[6] = (__bf16)(f3[0] * sc); v[7] = (__bf16)(f3[1] * sc);
      }
    }
    *reinterpret_cast<bf16x8*>(out + t * kPfRow + c * 8) = v;
  }
}

// Output staging.  An MFMA accumulator tile holds, in lane (r, h) = (lane&31,
// lane>>5), row r's columns 8j + 4h .. +3 in registers 4j .. 4j+3 of each
// 32-column block: stored as they are, every global write would be 8 bytes
// scattered over 32 rows.  Instead a wavefront writes its rows (256 B each,
// bf16) into its own LDS area, chunk c (16 B) of row r at r*256 + ((c ^ (r&15))
// * 16), and then writes them out 4 whole rows per instruction.
__device__ __forceinline__ void stage_block(uint32_t area, int row, int h, int blk, const f32x16& v, float mul) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bf16x4 x;
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (__bf16)(v[4 * j + e] * mul);
    const int c = 4 * blk + j;
    *reinterpret_cast<bf16x4 MLA_LDS*>((char MLA_LDS*)(uintptr_t)(area + uint32_t(row * 256 + ((c ^ (row & 15)) * 16) + 8 * h))) = x;
  }
}
// row r of the staged rows (4 per call, lane l: row 4i + (l>>4), chunk l&15)
__device__ __forceinline__ bf16x8 staged_chunk(uint32_t area, int row, int c) {
  return lds_read_b128(area + uint32_t(row * 256 + ((c ^ (row & 15)) * 16)));
}

// ---------------------------------------------------------------------------
// kv: KV^T tile [256 features x 256 rows] per workgroup, K = 512 in 16 chunks of
// 32.  8 wavefronts (2 per SIMD): wavefront w computes features 128(w&1) ..+127
// x rows 64(w>>1) ..+63 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16 (A = weight
// rows, B = C rows, so a lane's accumulator holds one row's runs of 4
// consecutive features).  Each chunk's operands (256 weight rows and 256 C
// rows, 64 B of each) sit in one of 4 LDS stages, 3 chunks ahead of use; row r's
// 16-byte piece p at r*64 + ((p ^ ((r>>2)&3)) * 16), so that the fragment
// reads (16 rows of one piece per 16 lanes) hit distinct banks.
constexpr int kKvTile = 256, kKvChunk = 32, kKvChunks = kPfLat / kKvChunk, kKvStages = 4;
constexpr int kKvHalf = kKvTile * kKvChunk * 2;   // 16 KB: one operand of a stage
constexpr int kKvStage = 2 * kKvHalf;

__global__ __launch_bounds__(512) void prefill_kv_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds_raw[kKvStages * kKvStage];
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(lds_raw));
  // Row tiles vary fastest: block x runs on XCD x % 8, so an XCD holds the
  // same few row tiles of C (256 KB each) for the whole launch, from its L2,
  // while the weight tiles stream past once per XCD.
  const int ft = int(blockIdx.y);
  const int f0 = ft * kKvTile, g0 = int(blockIdx.x) * kKvTile;
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, h = lane >> 5;
  const int nk = a.n_heads * kPfHead;

  // loads: wavefront w fills 16-row blocks 2w and 2w+1 of both operands; lane
  // l reads row 16i + (l>>2), logical piece (l&3) ^ ((l>>4)&3)
  const int lp = (lane & 3) ^ ((lane >> 4) & 3);
  const char* asrc[2];
  const char* bsrc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 16 * (2 * wave + j) + (lane >> 2);
    const int f = f0 + r;
    const uint16_t* w = f < nk ? a.w_uk + int64_t(f) * kPfLat : a.w_uv + int64_t(f - nk) * kPfLat;
    asrc[j] = reinterpret_cast<const char*>(w) + lp * 16;
    bsrc[j] = reinterpret_cast<const char*>(a.c_rows + int64_t(g0 + r) * kPfRow) + lp * 16;
  }
  auto issue = [&](int c) {
    const uint32_t sb = lds + uint32_t((c % kKvStages) * kKvStage);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      dma16(asrc[j] + c * 64, sb + uint32_t((2 * wave + j) * 1024));
      dma16(bsrc[j] + c * 64, sb + uint32_t(kKvHalf + (2 * wave + j) * 1024));
    }
  };

  const int fw = wave & 1, tw = wave >> 1;
  const int sw = (lane >> 2) & 3;
  const uint32_t a_row = uint32_t((128 * fw + (lane & 31)) * 64);
  const uint32_t b_row = uint32_t(kKvHalf + (64 * tw + (lane & 31)) * 64);
  f32x16 acc[4][2];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n) acc[m][n] = f32x16{};

  // fragments of one chunk: k-step s, 4 weight and 2 row fragments
  struct Frags {
    bf16x8 a[2][4], b[2][2];
  };
  auto read_step = [&](Frags& f, int c, int s) {
    const uint32_t sb = lds + uint32_t((c % kKvStages) * kKvStage);
    const uint32_t pofs = uint32_t(((2 * s + h) ^ sw) * 16);
#pragma unroll
    for (int m = 0; m < 4; ++m) f.a[s][m] = lds_read_b128(sb + a_row + uint32_t(m * 2048) + pofs);
#pragma unroll
    for (int n = 0; n < 2; ++n) f.b[s][n] = lds_read_b128(sb + b_row + uint32_t(n * 2048) + pofs);
  };

  // Chunk c's fragments are read into registers during chunk c-1's MFMAs, so
  // the MFMAs never wait for LDS; the barrier at the top of iteration c
  // publishes chunk c+1 and tells that every wavefront holds chunk c in
  // registers, so chunk c+4 may overwrite its stage.
#pragma unroll
  for (int c = 0; c < kKvStages; ++c) issue(c);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * (kKvStages - 1)));
  raw_barrier();
  Frags cur;
  read_step(cur, 0, 0);
  read_step(cur, 0, 1);
#pragma unroll
  for (int c = 0; c < kKvChunks; ++c) {
    Frags nxt;
    if (c + 1 < kKvChunks) {
      const int later = min(c + kKvStages - 1, kKvChunks - 1) - (c + 1);   // chunks issued after c+1
      if (later == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(8));
      else if (later == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
      raw_barrier();
      if (c + kKvStages < kKvChunks) issue(c + kKvStages);
      read_step(nxt, c + 1, 0);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur.a[s][m], cur.b[s][n], acc[m][n], 0, 0, 0);
      if (s == 0 && c + 1 < kKvChunks) read_step(nxt, c + 1, 1);
    }
    if (c + 1 < kKvChunks) cur = nxt;
  }

  // stores: the wavefront's 64 rows x 128 features of slab 2 ft + fw are one
  // contiguous 16 KB block (rows g0 + 64 tw ..), staged through the LDS area
  // of the (finished) operand stages
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  raw_barrier();
  const uint32_t area = lds + uint32_t(wave * 16384);
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m) stage_block(area, 32 * n + (lane & 31), h, m, acc[m][n], 1.f);
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  uint16_t* dst = a.kv_up + (int64_t(2 * ft + fw) * a.cap_rows + g0 + 64 * tw) * kPfHead;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = 4 * i + (lane >> 4), c = lane & 15;
    // non-temporal: the 64 KB per token of keys and values stream past the
    // caches (measured: 6% less time than plain stores)
    __builtin_nontemporal_store(__builtin_bit_cast(i32x4, staged_chunk(area, row, c)),
                                reinterpret_cast<i32x4*>(dst + row * kPfHead + c * 8));
  }
}

// ---------------------------------------------------------------------------
// attn: workgroup (head i, block of 256 new tokens of sequence b), 8 wavefronts
// of 32 new tokens each.  Per 32-token tile of cached positions, wavefront w
//   S^T [32 positions x 32 tokens] = K [32 x 192] . Q^T [192 x 32]   (12 MFMAs)
//   O^T [128 x 32 tokens]        += V^T [128 x 32] . P^T [32 x 32]   (8 MFMAs)
// with Q^T in registers and K, V from LDS (the tile layout of decode_tile.h:
// K = 24 chunks, 16 of k^C then 8 of k^R; V = 16 chunks).  A lane holds one new
// token (column lane&31) and 16 of the tile's positions (8(r>>2) + 4h + (r&3)
// in register r), so a token's softmax is a reduction over its lane pair.
// Online softmax in the log2 domain with a lazy rescale: a token's reference
// max moves (and its O^T and row sum are rescaled) only when the tile's max
// exceeds it by more than kPfSlack, so probabilities stay below 2^kPfSlack.
// (4 wavefronts per workgroup, two workgroups per compute unit with 4 buffers
// each, measured 54% slower: twice the tile loads per token, and no gain from
// the independent barriers)
constexpr int kPaWaves = 8, kPaQ = 32 * kPaWaves, kPaTok = 32;
// tile buffers: tiles k and k+1 are read while tiles k+2 .. k+kPaBufs-1 load
constexpr int kPaBufs = 6, kPaLead = kPaBufs - 1;
constexpr int kPaKBytes = 3 * 4096, kPaVBytes = 2 * 4096, kPaTileBytes = kPaKBytes + kPaVBytes;
constexpr float kPfSlack = 8.f;
constexpr int kPaKAhead = 6;   // K fragment reads in flight ahead of the score MFMAs

__global__ __launch_bounds__(64 * kPaWaves) void prefill_attn_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(2048))) char lds_raw[kPaBufs * kPaTileBytes];
  const uint32_t lds = uint32_t(reinterpret_cast<uintptr_t>(lds_raw));
  // Order: block x runs on XCD x % 8.  Each XCD takes its heads (x % 8,
  // x % 8 + 8, ...) two at a time, and a pair's token blocks longest first
  // (the blocks of both heads and of every sequence at one block index, then
  // the next lower index), so that the workgroups resident on an XCD read the
  // keys and values of two heads, which its L2 then serves, and the last
  // blocks to start are short ones.
  const int per_head = a.batch * a.n_qblk;
  int head, b, qb;
  if ((a.n_heads & 15) == 0) {
    const int j = int(blockIdx.x) >> 3;
    const int grp = j / (2 * per_head), idx = j % (2 * per_head);
    const int rest = idx % (2 * a.batch);
    head = int(blockIdx.x & 7) + 8 * (2 * grp + (rest & 1));
    b = rest >> 1;
    qb = a.n_qblk - 1 - idx / (2 * a.batch);
  } else {
    head = int(blockIdx.x) / per_head;
    const int r = int(blockIdx.x) % per_head;
    b = r % a.batch;
    qb = a.n_qblk - 1 - r / a.batch;
  }
  const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63, h = lane >> 5;

  int T0 = load_const(a.seq_lens, b);
  T0 = T0 < 0 ? 0 : (T0 > a.max_tokens ? a.max_tokens : T0);
  const int cu = load_const(a.cu, b);
  const int T = min(T0, load_const(a.cu, b + 1) - cu);   // rows the scan placed (capacity)
  int qo = load_const(a.q_off, b), qn = load_const(a.q_off, b + 1) - qo;
  qo = max(qo, 0);
  qn = max(0, min(qn, a.total_q - qo));
  if (kPaQ * qb >= qn) return;
  const int p0 = T0 - qn;   // position of new token 0
  // last visible position of the workgroup, of this wavefront and of this lane
  const int tq_last = min(qn, kPaQ * (qb + 1)) - 1;
  const int p_last = min(p0 + tq_last, T - 1);
  const int ntiles = p_last >= 0 ? p_last / kPaTok + 1 : 0;
  const int t_base = kPaQ * qb + 32 * wave;
  const int w_last = t_base < qn ? min(p0 + min(qn - 1, t_base + 31), T - 1) : -1;
  const int w_tiles = w_last >= 0 ? w_last / kPaTok + 1 : 0;
  const int w_first = min(p0 + t_base, T - 1);   // first token's last visible position
  const int t = t_base + (lane & 31);
  const bool q_ok = t < qn;
  const int lim = min(p0 + t, T - 1);            // this token sees positions 0..lim

  // Q^T fragments: k-step st holds dims 16st + 8h .. +7 of token t (q^C for
  // st < 8, q^R for st >= 8)
  bf16x8 qf[12];
  {
    const int64_t qrow = int64_t(qo + (q_ok ? t : 0)) * a.n_heads + head;
    const uint16_t* qc = a.q_nope + qrow * kPfHead + 8 * h;
    const uint16_t* qr = a.q_pe + qrow * kPfRope + 8 * h;
#pragma unroll
    for (int st = 0; st < 12; ++st) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(st < 8 ? qc + 16 * st : qr + 16 * (st - 8));
      qf[st] = q_ok ? v : bf16x8{};
    }
  }

  // tile loads: 20 one-KB blocks (block 4g + rb: rows 8rb..8rb+7 of chunk
  // group g; groups 0-1 k^C, 2 k^R, 3-4 V); wavefront w issues blocks w, w+8
  // and (w < 4) w+16.  Lane l reads row 8rb + (l>>3), logical chunk
  // 8g' + ((l&7) ^ f(row)) of its source row.
  const int n_my = (20 - wave + kPaWaves - 1) / kPaWaves;   // blocks wave, wave + kPaWaves, ..
  const uint16_t* kc_base = a.kv_up + (int64_t(head) * a.cap_rows + cu) * kPfHead;
  const uint16_t* v_base = a.kv_up + (int64_t(a.n_heads + head) * a.cap_rows + cu) * kPfHead;
  const uint16_t* kr_base = a.c_rows + int64_t(cu) * kPfRow + kPfLat;
  // per block j of this wavefront: the source of tile 0, the step from tile to
  // tile (uniform) and the LDS offset in a tile buffer, computed once (1.4%
  // less attention time than computing each address at its issue)
  constexpr int kMaxMy = (20 + kPaWaves - 1) / kPaWaves;
  const char* src0[kMaxMy];
  int64_t step[kMaxMy];
  uint32_t doff[kMaxMy];
#pragma unroll
  for (int j = 0; j < kMaxMy; ++j) {
    const int i = min(wave + kPaWaves * j, 19);
    const int g = i >> 2, rb = i & 3;
    const int row = 8 * rb + (lane >> 3);
    const int ch = (lane & 7) ^ swz_f(row);
    if (g < 2) {
      src0[j] = reinterpret_cast<const char*>(kc_base + int64_t(row) * kPfHead + 8 * (8 * g + ch));
      step[j] = int64_t(kPaTok) * kPfHead * 2;
      doff[j] = uint32_t(i * 1024);
    } else if (g == 2) {
      src0[j] = reinterpret_cast<const char*>(kr_base + int64_t(row) * kPfRow + 8 * ch);
      step[j] = int64_t(kPaTok) * kPfRow * 2;
      doff[j] = uint32_t(i * 1024);
    } else {
      src0[j] = reinterpret_cast<const char*>(v_base + int64_t(row) * kPfHead + 8 * (8 * (g - 3) + ch));
      step[j] = int64_t(kPaTok) * kPfHead * 2;
      doff[j] = uint32_t(kPaKBytes + (i - 12) * 1024);
    }
  }
  auto issue_block = [&](int k, int j) {   // block wave + kPaWaves j of tile k
    dma16(src0[j] + k * step[j], lds + uint32_t((k % kPaBufs) * kPaTileBytes) + doff[j]);
  };
  auto issue = [&](int k) {
#pragma unroll
    for (int j = 0; j < (20 + kPaWaves - 1) / kPaWaves; ++j)
      if (j < n_my) issue_block(k, j);
  };

  const int kb0 = tile_offset(lane & 31, h);
  // V^T fragment (transposing reads) of column tile mt, token half ks: rows
  // 4h + (j>>2) and 8 + 4h + (j>>2) (j = lane & 15) of chunk 2((lane>>4)&1) +
  // ((j>>1)&1), byte (j&1)*8; the second row's address is the first's ^ 0x410;
  // then ^ 64*(mt&1) + (mt>>1)*4096 + ks*2048
  const int vb0 = tile_offset(4 * h + ((lane & 15) >> 2), 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1)) + (lane & 1) * 8;
  auto tile_buf = [&](int k) { return lds + uint32_t((k % kPaBufs) * kPaTileBytes); };
  auto kfrag = [&](uint32_t tb, int st) {
    return lds_read_b128(((tb + uint32_t(kb0)) ^ uint32_t(32 * (st & 3))) + uint32_t((st >> 2) * 4096));
  };
  auto vfrag = [&](uint32_t tb, int st) {   // PV step st: token half st >> 2, column tile st & 3
    const int ks = st >> 2, mt = st & 3;
    const uint32_t a0 = ((tb + uint32_t(kPaKBytes + vb0)) ^ uint32_t(64 * (mt & 1))) + uint32_t((mt >> 1) * 4096 + ks * 2048);
    return lds_read_tr_pair(a0, a0 ^ 0x410u);
  };

  f32x16 acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = f32x16{};
  float m_run = -INFINITY, lsum = 0.f;

  // Software pipeline of tile k (per wavefront; the workgroup's tiles go on
  // past a wavefront's own range, where it only loads and waits):
  //   mask and max of S(k), lazy rescale of O^T
  //   phase A: the 12 score MFMAs of tile k+1, with the exponentials, the bf16
  //            packing and the row sums of P(k) between them and the first V^T
  //            reads of tile k during the last ones
  //   phase B: the 8 PV MFMAs of tile k, with this wavefront's loads of tile
  //            k+5 between them (into the buffer of tile k-1)
  //   wait for this wavefront's loads of tile k+2, barrier (tile k+2 complete;
  //     every wavefront is done with tile k, whose buffer takes tile k+6)
  for (int k = 0; k < min(ntiles, kPaLead); ++k) issue(k);
  // tiles 0 and 1 complete (the loads of the later ones stay in flight)
  wait_vm(n_my * max(0, min(ntiles, kPaLead) - 2));
  raw_barrier();
  f32x16 s = f32x16{};
  if (w_tiles > 0) {
    const uint32_t tb = tile_buf(0);
#pragma unroll
    for (int st = 0; st < 12; ++st) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(tb, st), qf[st], s, 0, 0, 0);
  }

  for (int k = 0; k < ntiles; ++k) {
    const bool load3 = k + kPaLead < ntiles;   // tile k+kPaLead, into tile k-1's buffer
    if (k < w_tiles) {
      const uint32_t tb = tile_buf(k);
      // causal mask (only where the tile reaches past the wavefront's first
      // token's last position) and the tile max
      const int j0 = k * kPaTok;
      if (j0 + kPaTok - 1 > w_first) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[r] = (j0 + 8 * (r >> 2) + 4 * h + (r & 3) > lim) ? -INFINITY : s[r];
      }
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      {
        const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1])) * a.scale_log2;
      }
      const bool need = mx > m_run + kPfSlack;   // (false while mx is -inf)
      if (__any(need)) {
        const float m_new = need ? mx : m_run;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;   // exp2(-inf) = 0
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[m][r] *= alpha;
        lsum *= alpha;
        m_run = m_new;
      }
      const float mref = m_run == -INFINITY ? 0.f : m_run;

      // ======== phase A: scores of tile k+1 (computed also past the
      // wavefront's range, where they are not used: no branch inside the
      // pipeline), softmax of tile k in 11 pieces between them
      bf16x8 pk[2];
      bf16x8 vr[4];
      f32x16 sn;
      {
        const uint32_t tn = tile_buf(k + 1);
        bf16x8 kr[kPaKAhead];
#pragma unroll
        for (int i = 0; i < kPaKAhead; ++i) kr[i] = kfrag(tn, i);
#pragma unroll
        for (int st = 0; st < 12; ++st) {
          const bf16x8 kc = kr[st % kPaKAhead];
          if (st + kPaKAhead < 12) kr[st % kPaKAhead] = kfrag(tn, st + kPaKAhead);
          sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kc, qf[st], st == 0 ? f32x16{} : sn, 0, 0, 0);
          // (each piece is pinned where it is written: left alone, the
          // compiler sinks the exponentials next to their use in phase B)
          if (st < 8) {
            s[2 * st] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * st], a.scale_log2, -mref));
            s[2 * st + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * st + 1], a.scale_log2, -mref));
            asm volatile("" : "+v"(s[2 * st]), "+v"(s[2 * st + 1]));
          } else if (st < 10) {
            const int ks = st - 8;
#pragma unroll
            for (int e = 0; e < 8; ++e) pk[ks][e] = (__bf16)s[8 * ks + e];
            asm volatile("" : "+v"(pk[ks]));
          } else if (st == 10) {
            const float u0 = (s[0] + s[1]) + (s[2] + s[3]), u1 = (s[4] + s[5]) + (s[6] + s[7]);
            const float u2 = (s[8] + s[9]) + (s[10] + s[11]), u3 = (s[12] + s[13]) + (s[14] + s[15]);
            lsum += (u0 + u1) + (u2 + u3);
          }
          if (st >= 8) vr[st - 8] = vfrag(tb, st - 8);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // ======== phase B: O^T += V^T . P^T of tile k | loads of tile k+5
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 vc = vr[st % 4];
        if (st + 4 < 8) vr[st % 4] = vfrag(tb, st + 4);
        acc[st & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vc, pk[st >> 2], acc[st & 3], 0, 0, 0);
        if (load3 && st < n_my) issue_block(k + kPaLead, st);
        __builtin_amdgcn_sched_barrier(0);
      }
      s = sn;
    } else if (load3) {
      issue(k + kPaLead);
    }

    // ---- tile k+2 complete for every wavefront (the later tiles' loads stay in flight)
    if (k + 2 < ntiles) {
      wait_vm(n_my * (min(ntiles - 1, k + kPaLead) - (k + 2)));
      raw_barrier();
    }
  }

  // epilogue: the token's row sum over both lanes of its pair; o = O / sum,
  // lse = ln(sum) + m (natural log); a token that sees no position gets zeros
  // and -inf
  {
    const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
  }
  const bool any = lsum > 0.f;
  const float inv = any ? 1.f / lsum : 0.f;
  if (q_ok && a.lse != nullptr && h == 0)
    a.lse[int64_t(qo + t) * a.n_heads + head] = any ? (m_run + __log2f(lsum)) * kLn2 : -INFINITY;
  // outputs: the wavefront's 32 token rows (256 B each) staged through its 8 KB
  // of LDS, then written 4 whole rows per instruction (the tile buffers are
  // free once every wavefront has left the loop)
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
  raw_barrier();              // (no tile loads are in flight after the loop)
  if (t_base >= qn) return;   // (wave-uniform: no token of this wavefront is valid)
  const uint32_t area = lds + uint32_t(wave * 8192);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) stage_block(area, lane & 31, h, mt, acc[mt], inv);
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm(0));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 4 * i + (lane >> 4), c = lane & 15;
    if (t_base + row < qn)
      *reinterpret_cast<bf16x8*>(a.out + (int64_t(qo + t_base + row) * a.n_heads + head) * kPfHead + c * 8) =
          staged_chunk(area, row, c);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  prefill_scan_kernel<<<1, 256, 0, st>>>(a);
  prefill_gather_kernel<<<a.cap_rows / 32, 256, 0, st>>>(a);
  prefill_kv_kernel<<<dim3(a.cap_rows / kKvTile, 2 * a.n_heads * kPfHead / kKvTile), 512, 0, st>>>(a);
  PrefillArgs b = a;
  b.n_qblk = (a.max_q_len + kPaQ - 1) / kPaQ;
  if (b.batch > 0 && b.n_qblk > 0) prefill_attn_kernel<<<b.n_heads * b.batch * b.n_qblk, 64 * kPaWaves, 0, st>>>(b);
  return hipGetLastError();
}

}  // namespace mla
