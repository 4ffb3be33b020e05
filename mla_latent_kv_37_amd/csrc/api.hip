// C ABI of libmla (include/mla.h): argument validation, partition resolution,
// dtype/shape dispatch and kernel launches.  Nothing here allocates device
// memory; every check runs before the first launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "api_internal.h"

namespace mla {

// Plan of the weight-streaming product (gemm.hip): the MFMA kernel for bf16
// operands on whole 64 x 64 tiles, with k slices until tiles x slices fill the
// chip about twice (two workgroups per compute unit).
int gemm_ws_slices(int N, int K, int batch, int max_slices) {
  if (N % kGemmTile != 0 || K % kGemmChunk != 0) return 1;
  const int tiles = (N / kGemmTile) * ceil_div(batch > 1 ? batch : 1, kGemmTile);
  for (int sl : {16, 8, 4, 2})
    if (sl <= max_slices && K % (kGemmChunk * sl) == 0 && tiles * sl <= 512) return sl;
  return 1;
}

void gemm_ws_plan(GemmArgs& a, int max_slices) {
  a.use_mfma = a.x_dt == MLA_BF16 && a.w_dt == MLA_BF16 && a.N % kGemmTile == 0 && a.K % kGemmChunk == 0;
  a.slices = a.use_mfma ? gemm_ws_slices(a.N, a.K, a.batch, max_slices) : 1;
}

}  // namespace mla

namespace {

using namespace mla;

constexpr int kGenMaxLatent = 1024;
constexpr int kGenMaxRow = 1280;
constexpr int kGenMaxHead = 1024;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

bool is_v2(const mla_dims_t* d) {
  return d->n_heads == 128 && d->d_latent == 512 && d->d_rope == 64;
}

mla_status_t check_dims(const mla_dims_t* d) {
  if (d == nullptr) return MLA_ERR_INVALID_ARG;
  if (d->n_heads < 1 || d->d_head < 1 || d->d_rope < 0 || d->d_latent < 1) return MLA_ERR_INVALID_ARG;
  return MLA_OK;
}

bool valid_dtype(mla_dtype_t t) { return t == MLA_F32 || t == MLA_BF16 || t == MLA_FP8_E4M3; }

// Resolve a partition into kernel parameters, item and slot counts.
mla_status_t resolve(const mla_dims_t* /*dims*/, int32_t batch, int32_t max_pages, int32_t page_size,
                     const mla_partition_t* part, PartParams* pp, int* n_items, int* n_slots) {
  if (batch < 0 || max_pages < 1 || page_size < 1) return MLA_ERR_INVALID_ARG;
  PartParams p{};
  p.page_size = page_size;
  p.batch = batch;
  {
    const int64_t mt = int64_t(max_pages) * page_size;
    p.max_tokens = mt > INT32_MAX ? INT32_MAX : int(mt);
  }
  const int split = part ? part->split_tokens : 0;
  const int parts = part ? part->num_parts : 0;
  if (split < 0) return MLA_ERR_INVALID_ARG;
  if (split > 0) {
    if (split % page_size != 0) return MLA_ERR_INVALID_ARG;
    const int64_t max_tokens = int64_t(max_pages) * page_size;
    p.mode = PART_FIXED;
    p.split_tokens = split;
    p.fixed_slots = int((max_tokens + split - 1) / split);
    *n_items = batch * p.fixed_slots;
    *n_slots = *n_items;
  } else if (parts == 0) {
    p.mode = PART_WHOLE;
    *n_items = batch;
    *n_slots = 0;
  } else {
    int w = parts;
    if (w < 0) {
      // library default: fill the device once (one workgroup per compute unit)
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
      if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MLA_ERR_HIP;
      if (cus < 1) return MLA_ERR_HIP;
      w = cus;
    }
    p.mode = PART_BALANCED;
    p.num_parts = w;
    *n_items = w;
    *n_slots = w + batch;
  }
  *pp = p;
  return MLA_OK;
}

struct WsLayout {
  size_t o_part, lse_part, meta, total;
};

// o_elem: bytes per partial element.  The public workspace is sized for fp32
// (sizeof(float)) so that one size serves either output dtype; the
// no-allocation entry point packs partials at the output dtype's own size.
WsLayout ws_layout(const mla_dims_t* d, int n_slots, int batch, bool balanced, size_t o_elem = sizeof(float)) {
  WsLayout L{};
  if (n_slots == 0) return L;
  L.o_part = 0;
  L.lse_part = align256(size_t(n_slots) * d->n_heads * d->d_latent * o_elem);
  L.meta = L.lse_part + align256(size_t(n_slots) * d->n_heads * sizeof(float));
  L.total = L.meta + (balanced ? align256(size_t(2) * batch * sizeof(int32_t)) : 0);
  return L;
}

// RoPE parameters of an mla_rope_t (NULL: invalid) or a plain base
mla_status_t rope_params(const mla_rope_t* r, RopeParams* out) {
  if (r == nullptr) return MLA_ERR_INVALID_ARG;
  if (!(r->base >= 0.f) || !(r->base < 1e30f)) return MLA_ERR_INVALID_ARG;
  if (!(r->yarn_scale >= 1.f) || !(r->yarn_scale < 1e30f)) return MLA_ERR_INVALID_ARG;
  RopeParams p{r->base, 1.f, 0.f, 0.f, 0.f};
  if (r->yarn_scale > 1.f) {
    if (!(r->yarn_beta > r->yarn_alpha) || !(r->yarn_alpha >= 0.f) || !(r->yarn_beta < 1e30f) ||
        r->yarn_orig_ctx < 1)
      return MLA_ERR_INVALID_ARG;
    p = RopeParams{r->base, r->yarn_scale, r->yarn_alpha, r->yarn_beta, float(r->yarn_orig_ctx)};
  }
  *out = p;
  return MLA_OK;
}

// checks shared by the cache-store entry points; fills the store arguments
mla_status_t store_args(const mla_dims_t* dims, int32_t batch, const void* rows, mla_dtype_t rows_dt,
                        const int32_t* positions, const mla_rope_t* rope, const mla_paged_cache_t* cache,
                        CacheStoreArgs* a) {
  if (mla_status_t s = check_dims(dims)) return s;
  if (batch < 0 || cache == nullptr) return MLA_ERR_INVALID_ARG;
  RopeParams rp;
  if (mla_status_t s = rope_params(rope, &rp)) return s;
  if (rows_dt != MLA_F32 && rows_dt != MLA_BF16) return valid_dtype(rows_dt) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!valid_dtype(cache->dtype)) return MLA_ERR_INVALID_ARG;
  const int W = dims->d_latent + dims->d_rope;
  if ((dims->d_latent & 1) || (dims->d_rope & 1)) return MLA_ERR_UNSUPPORTED;   // columns go in pairs
  if (W > kGenMaxRow) return MLA_ERR_UNSUPPORTED;
  if (cache->page_size < 1 || cache->max_pages_per_seq < 1 || cache->num_pages < 1) return MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!rows || !positions || !cache->kv || !cache->block_table) return MLA_ERR_INVALID_ARG;
  if (cache->dtype == MLA_FP8_E4M3 && !cache->scales) return MLA_ERR_INVALID_ARG;
  if (!aligned16(rows) || !aligned16(cache->kv)) return MLA_ERR_ALIGNMENT;
  a->rows = rows;
  a->rows_dt = rows_dt;
  a->positions = positions;
  a->rope = rp;
  a->kv = const_cast<void*>(cache->kv);
  a->scales = const_cast<float*>(cache->scales);
  a->kv_dt = cache->dtype;
  a->block_table = cache->block_table;
  a->max_pages = cache->max_pages_per_seq;
  a->page_size = cache->page_size;
  a->num_pages = cache->num_pages;
  a->d_latent = dims->d_latent;
  a->d_rope = dims->d_rope;
  return MLA_OK;
}

// mla_query_prep scratch: stage-1 k slices (at most kQueryMaxSlices: d_model is
// not an argument of the size query), c^Q (in the weights' dtype; its area is
// sized for fp32), stage-2 k slices (as many as the bf16 plan for
// [n_h (d_h + d_rope)] x d_qlatent uses; every other plan uses one), and the
// query epilogue's RoPE table (batch x d_rope/2 pairs of doubles).  One size
// serves every dtype.
struct QueryScratch { size_t s1, cq, s2, tab, total; };
// d_qlatent = 0 (no query compression): no stage 1, and the single product's
// k slices are sized for the largest plan (d_model is not an argument either).
QueryScratch query_scratch(const mla_dims_t* d, int32_t d_qlatent, int32_t batch) {
  QueryScratch q{};
  const size_t B = size_t(batch > 0 ? batch : 0);
  const int n2 = d->n_heads * (d->d_head + d->d_rope);
  q.s1 = 0;
  q.cq = align256(kQueryMaxSlices * B * d_qlatent * sizeof(float));
  q.s2 = q.cq + align256(B * d_qlatent * sizeof(float));
  const size_t slices2 = d_qlatent > 0 ? size_t(gemm_ws_slices(n2, d_qlatent, int(B), kQueryMaxSlices)) : kQueryMaxSlices;
  q.tab = q.s2 + align256(slices2 * B * n2 * sizeof(float));
  q.total = q.tab + align256(B * size_t(d->d_rope / 2) * 2 * sizeof(double));
  return q;
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG: null pointer, bad size or inconsistent arguments";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: dtype combination or size not implemented";
    case MLA_ERR_ALIGNMENT: return "MLA_ERR_ALIGNMENT: tensor pointer not 16-byte aligned";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
  }
  return "unknown mla_status_t";
}

const char* mla_build_info(void) {
  return "libmla gfx950: absorb(v2 mfma, generic), decode(v2 bf16 / fp8-dequant one-wavefront-per-SIMD mfma, "
         "16-head bf16 mfma, "
         "generic f32/bf16/fp8), "
         "cache store (f32/bf16/fp8 1x128), cache append and query prep (weight-streaming mfma / generic "
         "products), "
         "merge, out_proj(v2 mfma, generic)";
}

mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t batch, const void* q_nope, mla_dtype_t q_dt,
                          const void* w_uk, mla_dtype_t w_dt, void* q_lat, mla_dtype_t out_dt, void* stream) {
  if (mla_status_t s = check_dims(dims)) return s;
  if (batch < 0) return MLA_ERR_INVALID_ARG;
  if (!q_nope || !w_uk || !q_lat) return MLA_ERR_INVALID_ARG;
  for (mla_dtype_t t : {q_dt, w_dt, out_dt})
    if (t != MLA_F32 && t != MLA_BF16) return valid_dtype(t) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_lat)) return MLA_ERR_ALIGNMENT;
  if (batch == 0) return MLA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dims->d_head == 128 && dims->d_latent == 512 && q_dt == MLA_BF16 && w_dt == MLA_BF16 && out_dt == MLA_BF16) {
    e = launch_absorb_v2(q_nope, w_uk, q_lat, batch, dims->n_heads, st);
  } else {
    if (dims->d_head > kGenMaxHead) return MLA_ERR_UNSUPPORTED;
    e = launch_absorb_generic(q_nope, q_dt, w_uk, w_dt, q_lat, out_dt, batch, dims->n_heads, dims->d_head,
                              dims->d_latent, st);
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_decode_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t max_pages_per_seq,
                                       int32_t page_size, const mla_partition_t* part, size_t* bytes,
                                       int32_t* num_slots) {
  if (mla_status_t s = check_dims(dims)) return s;
  if (!bytes) return MLA_ERR_INVALID_ARG;
  PartParams pp;
  int n_items = 0, n_slots = 0;
  if (mla_status_t s = resolve(dims, batch, max_pages_per_seq, page_size, part, &pp, &n_items, &n_slots)) return s;
  *bytes = ws_layout(dims, n_slots, batch, pp.mode == PART_BALANCED).total;
  if (num_slots) *num_slots = n_slots;
  return MLA_OK;
}

size_t mla_lse_part_offset(const mla_dims_t* dims, int32_t num_slots) {
  if (dims == nullptr || num_slots <= 0) return 0;
  return align256(size_t(num_slots) * dims->n_heads * dims->d_latent * sizeof(float));
}

}  // extern "C"

namespace mla {

// mla_decode's checks and launch; with dry = true only the checks.
mla_status_t decode_impl(const mla_dims_t* dims, int32_t batch, const void* q_lat, const void* q_pe,
                         mla_dtype_t q_dt, const mla_paged_cache_t* cache, float softmax_scale,
                         const mla_partition_t* part, void* workspace, size_t workspace_bytes, void* o_lat,
                         mla_dtype_t o_dt, float* lse, void* stream, bool dry, size_t o_elem, int bt_div) {
  if (mla_status_t s = check_dims(dims)) return s;
  if (!cache || !q_lat || !o_lat || (dims->d_rope > 0 && !q_pe)) return MLA_ERR_INVALID_ARG;
  if (!cache->kv || !cache->block_table || !cache->seq_lens) return MLA_ERR_INVALID_ARG;
  if (!valid_dtype(q_dt) || !valid_dtype(o_dt) || !valid_dtype(cache->dtype)) return MLA_ERR_INVALID_ARG;
  if (cache->num_pages < 1 || cache->page_size < 1 || cache->max_pages_per_seq < 1) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || softmax_scale == INFINITY) return MLA_ERR_INVALID_ARG;
  if (cache->dtype == MLA_FP8_E4M3 && !cache->scales) return MLA_ERR_INVALID_ARG;
  if (cache->dtype == MLA_FP8_E4M3 && !aligned16(cache->scales)) return MLA_ERR_ALIGNMENT;
  // supported combinations: f32 cache with f32 queries; bf16/fp8 cache with bf16 queries
  if (cache->dtype == MLA_F32 ? q_dt != MLA_F32 : q_dt != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (o_dt == MLA_FP8_E4M3) return MLA_ERR_UNSUPPORTED;
  if (!aligned16(q_lat) || (q_pe && !aligned16(q_pe)) || !aligned16(cache->kv) || !aligned16(o_lat))
    return MLA_ERR_ALIGNMENT;
  PartParams pp;
  int n_items = 0, n_slots = 0;
  if (mla_status_t s = resolve(dims, batch, cache->max_pages_per_seq, cache->page_size, part, &pp, &n_items, &n_slots))
    return s;
  pp.q_len = bt_div;   // (a multi-token decode's virtual lengths come from seq_lens)
  const WsLayout L = ws_layout(dims, n_slots, batch, pp.mode == PART_BALANCED, o_elem);
  if (L.total > 0 && (workspace == nullptr || workspace_bytes < L.total)) return MLA_ERR_WORKSPACE;
  if (L.total > 0 && !aligned16(workspace)) return MLA_ERR_ALIGNMENT;
  const bool fast = is_v2(dims) && cache->page_size == 64 && q_dt == MLA_BF16 &&
                    (cache->dtype == MLA_BF16 || cache->dtype == MLA_FP8_E4M3);
  const bool lite = dims->n_heads == 16 && dims->d_latent == 512 && dims->d_rope == 64 && cache->page_size == 64 &&
                    q_dt == MLA_BF16 && cache->dtype == MLA_BF16;
  if (!fast && !lite && (dims->d_latent > kGenMaxLatent || dims->d_latent + dims->d_rope > kGenMaxRow))
    return MLA_ERR_UNSUPPORTED;
  if (dry || batch == 0 || n_items == 0) return MLA_OK;
  char* ws = static_cast<char*>(workspace);
  void* o_part = L.total ? static_cast<void*>(ws + L.o_part) : nullptr;
  float* lse_part = L.total ? reinterpret_cast<float*>(ws + L.lse_part) : nullptr;
  int32_t* meta = (L.total && pp.mode == PART_BALANCED) ? reinterpret_cast<int32_t*>(ws + L.meta) : nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (fast || lite) {
    V2DecodeArgs a{};
    a.q_lat = static_cast<const uint16_t*>(q_lat);
    a.q_pe = static_cast<const uint16_t*>(q_pe);
    a.kv = cache->kv;
    a.scales = cache->dtype == MLA_FP8_E4M3 ? cache->scales : nullptr;
    a.kv_dt = cache->dtype;
    a.block_table = cache->block_table;
    a.seq_lens = cache->seq_lens;
    a.max_pages = cache->max_pages_per_seq;
    a.num_pages = cache->num_pages;
    a.bt_div = bt_div;
    a.n_items = n_items;
    a.scale_log2 = softmax_scale * kLog2e;
    a.pp = pp;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.meta = meta;
    a.o_lat = o_lat;
    a.o_dt = o_dt;
    a.lse = lse;
    if (!fast) e = launch_decode_lite(a, st);
    else e = launch_decode_wide(a, st);   // bf16 and fp8 caches
  } else {
    GenericDecodeArgs a{};
    a.q_lat = q_lat;
    a.q_pe = q_pe;
    a.q_dt = q_dt;
    a.kv = cache->kv;
    a.scales = cache->scales;
    a.kv_dt = cache->dtype;
    a.block_table = cache->block_table;
    a.seq_lens = cache->seq_lens;
    a.max_pages = cache->max_pages_per_seq;
    a.num_pages = cache->num_pages;
    a.bt_div = bt_div;
    a.n_heads = dims->n_heads;
    a.d_rope = dims->d_rope;
    a.d_latent = dims->d_latent;
    a.scale = softmax_scale;
    a.pp = pp;
    a.o_part = o_part;
    a.lse_part = lse_part;
    a.meta = meta;
    a.o_lat = o_lat;
    a.o_dt = o_dt;
    a.lse = lse;
    e = launch_decode_generic(a, n_items, st);
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

// mla_merge_splits' checks and launch (o_elem as for decode_impl).
mla_status_t merge_impl(const mla_dims_t* dims, int32_t batch, const int32_t* seq_lens, int32_t page_size,
                        int32_t max_pages_per_seq, const mla_partition_t* part, const void* workspace,
                        size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse, void* stream,
                        size_t o_elem, int q_len) {
  if (mla_status_t s = check_dims(dims)) return s;
  if (!seq_lens || !o_lat) return MLA_ERR_INVALID_ARG;
  if (o_dt != MLA_F32 && o_dt != MLA_BF16) return valid_dtype(o_dt) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!aligned16(o_lat)) return MLA_ERR_ALIGNMENT;
  PartParams pp;
  int n_items = 0, n_slots = 0;
  if (mla_status_t s = resolve(dims, batch, max_pages_per_seq, page_size, part, &pp, &n_items, &n_slots)) return s;
  pp.q_len = q_len;
  const WsLayout L = ws_layout(dims, n_slots, batch, pp.mode == PART_BALANCED, o_elem);
  if (L.total > 0 && (workspace == nullptr || workspace_bytes < L.total)) return MLA_ERR_WORKSPACE;
  if (batch == 0) return MLA_OK;
  const char* ws = static_cast<const char*>(workspace);
  MergeArgs a{};
  a.seq_lens = seq_lens;
  a.pp = pp;
  a.n_heads = dims->n_heads;
  a.d_latent = dims->d_latent;
  a.o_part = L.total ? static_cast<const void*>(ws + L.o_part) : nullptr;
  a.lse_part = L.total ? reinterpret_cast<const float*>(ws + L.lse_part) : nullptr;
  a.meta = (L.total && pp.mode == PART_BALANCED) ? reinterpret_cast<const int32_t*>(ws + L.meta) : nullptr;
  a.o_lat = o_lat;
  a.o_dt = o_dt;
  a.lse = lse;
  const hipError_t e = launch_merge(a, batch, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t decode_workspace_layout(const mla_dims_t* dims, int32_t batch, int32_t max_pages_per_seq,
                                     int32_t page_size, const mla_partition_t* part, size_t o_elem, size_t* bytes) {
  if (mla_status_t s = check_dims(dims)) return s;
  PartParams pp;
  int n_items = 0, n_slots = 0;
  if (mla_status_t s = resolve(dims, batch, max_pages_per_seq, page_size, part, &pp, &n_items, &n_slots)) return s;
  *bytes = ws_layout(dims, n_slots, batch, pp.mode == PART_BALANCED, o_elem).total;
  return MLA_OK;
}

}  // namespace mla

namespace {

// mla_decode_multi workspace: the workspace of the decode over batch * q_len
// virtual sequences (whose lengths the kernels derive from seq_lens).
struct MultiLayout {
  size_t dec, dec_bytes, total;
};

mla_status_t multi_layout(const mla_dims_t* dims, int32_t batch, int32_t q_len, int32_t max_pages,
                          int32_t page_size, const mla_partition_t* part, MultiLayout* M, int* n_slots) {
  if (mla_status_t s = check_dims(dims)) return s;
  if (batch < 0 || q_len < 1 || max_pages < 1) return MLA_ERR_INVALID_ARG;
  const int64_t vb = int64_t(batch) * q_len;
  if (vb > (int64_t(1) << 30) / max_pages) return MLA_ERR_INVALID_ARG;
  PartParams pp;
  int n_items = 0;
  if (mla_status_t s = resolve(dims, int(vb), max_pages, page_size, part, &pp, &n_items, n_slots)) return s;
  MultiLayout m{};
  m.dec = 0;
  m.dec_bytes = ws_layout(dims, *n_slots, int(vb), pp.mode == PART_BALANCED).total;
  m.total = m.dec + m.dec_bytes;
  *M = m;
  return MLA_OK;
}

}  // namespace

extern "C" {

mla_status_t mla_decode(const mla_dims_t* dims, int32_t batch, const void* q_lat, const void* q_pe,
                        mla_dtype_t q_dt, const mla_paged_cache_t* cache, float softmax_scale,
                        const mla_partition_t* part, void* workspace, size_t workspace_bytes, void* o_lat,
                        mla_dtype_t o_dt, float* lse, void* stream) {
  return decode_impl(dims, batch, q_lat, q_pe, q_dt, cache, softmax_scale, part, workspace, workspace_bytes, o_lat,
                     o_dt, lse, stream, false, sizeof(float), 1);
}

mla_status_t mla_merge_splits(const mla_dims_t* dims, int32_t batch, const int32_t* seq_lens, int32_t page_size,
                              int32_t max_pages_per_seq, const mla_partition_t* part, const void* workspace,
                              size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse, void* stream) {
  return merge_impl(dims, batch, seq_lens, page_size, max_pages_per_seq, part, workspace, workspace_bytes, o_lat,
                    o_dt, lse, stream, sizeof(float));
}

mla_status_t mla_decode_multi_workspace_size(const mla_dims_t* dims, int32_t batch, int32_t q_len,
                                             int32_t max_pages_per_seq, int32_t page_size,
                                             const mla_partition_t* part, size_t* bytes, int32_t* num_slots) {
  if (!bytes) return MLA_ERR_INVALID_ARG;
  MultiLayout M;
  int n_slots = 0;
  if (mla_status_t s = multi_layout(dims, batch, q_len, max_pages_per_seq, page_size, part, &M, &n_slots)) return s;
  *bytes = M.total;
  if (num_slots) *num_slots = n_slots;
  return MLA_OK;
}

namespace {

// Arguments of the W^UV projection checked before anything is enqueued (the
// fused call validates them too, but only after the decode has been launched).
mla_status_t check_out_proj_args(const mla_dims_t* dims, mla_dtype_t o_dt, const void* w_uv, mla_dtype_t w_dt,
                                 const void* o_heads, mla_dtype_t out_dt) {
  if (!w_uv || !o_heads) return MLA_ERR_INVALID_ARG;
  for (mla_dtype_t t : {o_dt, w_dt, out_dt})
    if (t != MLA_F32 && t != MLA_BF16) return valid_dtype(t) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!aligned16(w_uv) || !aligned16(o_heads)) return MLA_ERR_ALIGNMENT;
  const bool v2 = dims->d_head == 128 && dims->d_latent == 512 && w_dt == MLA_BF16 && out_dt == MLA_BF16;
  if (!v2 && dims->d_latent > kGenMaxLatent) return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// Decode over the batch * q_len virtual sequences, then the merge (w_uv ==
// nullptr) or the merge + W^UV projection (as mla_merge_out_proj).  Virtual
// sequence b' = b*q_len + t is new token t of sequence b: the kernels read its
// length from seq_lens[b] (seq_len_of in mla_common.h: the tokens up to its own
// position, [deepseek(2) 關鍵技術] §1) and its pages from block-table row
// b' / q_len, sequence b's row, in place.  A workgroup cannot hold more than
// one token's 128 heads (their fp32 accumulators fill half a CU's register
// file), so every virtual sequence streams the pages itself; the copies of one
// sequence are adjacent in the work-item order, which puts them on the same XCD
// at about the same time, so the repeated page reads are served from L2 and the
// Infinity Cache rather than from HBM.
mla_status_t decode_multi_impl(const mla_dims_t* dims, int32_t batch, int32_t q_len, const void* q_lat,
                               const void* q_pe, mla_dtype_t q_dt, const mla_paged_cache_t* cache,
                               float softmax_scale, const mla_partition_t* part, void* workspace,
                               size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse, const void* w_uv,
                               mla_dtype_t w_dt, void* o_heads, mla_dtype_t out_dt, void* stream) {
  if (!cache) return MLA_ERR_INVALID_ARG;
  MultiLayout M;
  int n_slots = 0;
  if (mla_status_t s = multi_layout(dims, batch, q_len, cache->max_pages_per_seq, cache->page_size, part, &M, &n_slots))
    return s;
  if (!cache->block_table || !cache->seq_lens) return MLA_ERR_INVALID_ARG;
  if (M.total > 0 && (!workspace || workspace_bytes < M.total)) return MLA_ERR_WORKSPACE;
  if (M.total > 0 && !aligned16(workspace)) return MLA_ERR_ALIGNMENT;
  if (o_dt != MLA_F32 && o_dt != MLA_BF16) return valid_dtype(o_dt) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (w_uv || o_heads)
    if (mla_status_t s = check_out_proj_args(dims, o_dt, w_uv, w_dt, o_heads, out_dt)) return s;
  char* ws = static_cast<char*>(workspace);
  const int vb = batch * q_len;
  void* dec_ws = M.dec_bytes ? static_cast<void*>(ws + M.dec) : nullptr;
  if (mla_status_t s = decode_impl(dims, vb, q_lat, q_pe, q_dt, cache, softmax_scale, part, dec_ws, M.dec_bytes,
                                   o_lat, o_dt, lse, stream, true, sizeof(float), q_len))
    return s;
  if (batch == 0) return MLA_OK;
  if (mla_status_t s = decode_impl(dims, vb, q_lat, q_pe, q_dt, cache, softmax_scale, part, dec_ws, M.dec_bytes,
                                   o_lat, o_dt, lse, stream, false, sizeof(float), q_len))
    return s;
  if (!w_uv)
    return merge_impl(dims, vb, cache->seq_lens, cache->page_size, cache->max_pages_per_seq, part, dec_ws,
                      M.dec_bytes, o_lat, o_dt, lse, stream, sizeof(float), q_len);
  return merge_out_proj_impl(dims, vb, cache->seq_lens, cache->page_size, cache->max_pages_per_seq, part, dec_ws,
                             M.dec_bytes, o_lat, o_dt, lse, w_uv, w_dt, o_heads, out_dt, stream, q_len);
}

// mla_prefill workspace: sequence offsets, gathered rows, up-projected keys
// and values (see PrefillArgs)
struct PrefillLayout {
  size_t cu, rows, kv, total;
  int cap_rows;
};

constexpr int64_t kPrefillMaxKv = (int64_t(1) << 24) - 1;

mla_status_t prefill_layout(const mla_dims_t* dims, int32_t batch, int64_t total_kv, PrefillLayout* L) {
  if (mla_status_t s = check_dims(dims)) return s;
  if (batch < 0 || total_kv < 0) return MLA_ERR_INVALID_ARG;
  if (dims->d_head != 128 || dims->d_latent != 512 || dims->d_rope != 64) return MLA_ERR_UNSUPPORTED;
  if (total_kv > kPrefillMaxKv || dims->n_heads > 32768) return MLA_ERR_UNSUPPORTED;
  PrefillLayout l{};
  // rows: every position a 32-row tile of a sequence can touch (up to 31 past
  // the last row), in whole 256-row tiles of the up-projection
  l.cap_rows = int(((total_kv + 32 + 255) / 256) * 256);
  l.cu = 0;
  l.rows = align256(size_t(batch + 1) * sizeof(int32_t));
  l.kv = l.rows + align256(size_t(l.cap_rows) * 576 * 2);
  l.total = l.kv + size_t(2) * dims->n_heads * size_t(l.cap_rows) * 128 * 2;
  *L = l;
  return MLA_OK;
}

}  // namespace

mla_status_t mla_decode_multi(const mla_dims_t* dims, int32_t batch, int32_t q_len, const void* q_lat,
                              const void* q_pe, mla_dtype_t q_dt, const mla_paged_cache_t* cache,
                              float softmax_scale, const mla_partition_t* part, void* workspace,
                              size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse, void* stream) {
  return decode_multi_impl(dims, batch, q_len, q_lat, q_pe, q_dt, cache, softmax_scale, part, workspace,
                           workspace_bytes, o_lat, o_dt, lse, nullptr, MLA_BF16, nullptr, MLA_BF16, stream);
}

mla_status_t mla_decode_multi_out_proj(const mla_dims_t* dims, int32_t batch, int32_t q_len, const void* q_lat,
                                       const void* q_pe, mla_dtype_t q_dt, const mla_paged_cache_t* cache,
                                       float softmax_scale, const mla_partition_t* part, void* workspace,
                                       size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse,
                                       const void* w_uv, mla_dtype_t w_dt, void* o_heads, mla_dtype_t out_dt,
                                       void* stream) {
  if (!w_uv || !o_heads) return MLA_ERR_INVALID_ARG;
  return decode_multi_impl(dims, batch, q_len, q_lat, q_pe, q_dt, cache, softmax_scale, part, workspace,
                           workspace_bytes, o_lat, o_dt, lse, w_uv, w_dt, o_heads, out_dt, stream);
}

mla_status_t mla_out_proj(const mla_dims_t* dims, int32_t batch, const void* o_lat, mla_dtype_t o_dt, const void* w_uv,
                          mla_dtype_t w_dt, void* o_heads, mla_dtype_t out_dt, void* stream) {
  if (mla_status_t s = check_dims(dims)) return s;
  if (batch < 0 || !o_lat || !w_uv || !o_heads) return MLA_ERR_INVALID_ARG;
  for (mla_dtype_t t : {o_dt, w_dt, out_dt})
    if (t != MLA_F32 && t != MLA_BF16) return valid_dtype(t) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(o_heads)) return MLA_ERR_ALIGNMENT;
  if (batch == 0) return MLA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (dims->d_head == 128 && dims->d_latent == 512 && w_dt == MLA_BF16 && out_dt == MLA_BF16) {
    e = launch_outproj_v2(o_lat, o_dt == MLA_F32, w_uv, o_heads, batch, dims->n_heads, st);
  } else {
    if (dims->d_latent > kGenMaxLatent) return MLA_ERR_UNSUPPORTED;
    e = launch_outproj_generic(o_lat, o_dt, w_uv, w_dt, o_heads, out_dt, batch, dims->n_heads, dims->d_head,
                               dims->d_latent, st);
  }
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_merge_out_proj(const mla_dims_t* dims, int32_t batch, const int32_t* seq_lens, int32_t page_size,
                                int32_t max_pages_per_seq, const mla_partition_t* part, const void* workspace,
                                size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse, const void* w_uv,
                                mla_dtype_t w_dt, void* o_heads, mla_dtype_t out_dt, void* stream) {
  return merge_out_proj_impl(dims, batch, seq_lens, page_size, max_pages_per_seq, part, workspace, workspace_bytes,
                             o_lat, o_dt, lse, w_uv, w_dt, o_heads, out_dt, stream, 1);
}

}  // extern "C"

namespace mla {

mla_status_t merge_out_proj_impl(const mla_dims_t* dims, int32_t batch, const int32_t* seq_lens, int32_t page_size,
                                 int32_t max_pages_per_seq, const mla_partition_t* part, const void* workspace,
                                 size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse, const void* w_uv,
                                 mla_dtype_t w_dt, void* o_heads, mla_dtype_t out_dt, void* stream, int q_len) {
  // validation of both calls before anything is enqueued
  if (mla_status_t s = check_dims(dims)) return s;
  if (batch < 0 || !seq_lens || !o_lat || !w_uv || !o_heads) return MLA_ERR_INVALID_ARG;
  for (mla_dtype_t t : {o_dt, w_dt, out_dt})
    if (t != MLA_F32 && t != MLA_BF16) return valid_dtype(t) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (!aligned16(o_lat) || !aligned16(w_uv) || !aligned16(o_heads)) return MLA_ERR_ALIGNMENT;
  PartParams pp;
  int n_items = 0, n_slots = 0;
  if (mla_status_t s = resolve(dims, batch, max_pages_per_seq, page_size, part, &pp, &n_items, &n_slots)) return s;
  pp.q_len = q_len;
  const WsLayout L = ws_layout(dims, n_slots, batch, pp.mode == PART_BALANCED);
  if (L.total > 0 && (workspace == nullptr || workspace_bytes < L.total)) return MLA_ERR_WORKSPACE;
  const bool fused = dims->d_head == 128 && dims->d_latent == 512 && o_dt == MLA_BF16 && w_dt == MLA_BF16 &&
                     out_dt == MLA_BF16;
  if (!fused && dims->d_latent > kGenMaxLatent &&
      !(dims->d_head == 128 && dims->d_latent == 512 && w_dt == MLA_BF16 && out_dt == MLA_BF16))
    return MLA_ERR_UNSUPPORTED;
  if (batch == 0) return MLA_OK;
  if (!fused) {
    if (mla_status_t s = merge_impl(dims, batch, seq_lens, page_size, max_pages_per_seq, part, workspace,
                                    workspace_bytes, o_lat, o_dt, lse, stream, sizeof(float), q_len))
      return s;
    return mla_out_proj(dims, batch, o_lat, o_dt, w_uv, w_dt, o_heads, out_dt, stream);
  }
  const char* ws = static_cast<const char*>(workspace);
  MergeArgs a{};
  a.seq_lens = seq_lens;
  a.pp = pp;
  a.n_heads = dims->n_heads;
  a.d_latent = dims->d_latent;
  a.o_part = L.total ? static_cast<const void*>(ws + L.o_part) : nullptr;
  a.lse_part = L.total ? reinterpret_cast<const float*>(ws + L.lse_part) : nullptr;
  a.meta = (L.total && pp.mode == PART_BALANCED) ? reinterpret_cast<const int32_t*>(ws + L.meta) : nullptr;
  a.o_lat = o_lat;
  a.o_dt = o_dt;
  a.lse = lse;
  const hipError_t e = launch_merge_proj(a, w_uv, o_heads, batch, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // namespace mla

extern "C" {

mla_status_t mla_cache_store(const mla_dims_t* dims, int32_t batch, const void* rows, mla_dtype_t rows_dt,
                             const int32_t* positions, float rope_base, const mla_paged_cache_t* cache,
                             void* stream) {
  const mla_rope_t r{rope_base, 1.f, 0.f, 0.f, 0};
  return mla_cache_store_rope(dims, batch, rows, rows_dt, positions, &r, cache, stream);
}

mla_status_t mla_cache_store_rope(const mla_dims_t* dims, int32_t batch, const void* rows, mla_dtype_t rows_dt,
                                  const int32_t* positions, const mla_rope_t* rope, const mla_paged_cache_t* cache,
                                  void* stream) {
  CacheStoreArgs a{};
  if (mla_status_t s = store_args(dims, batch, rows, rows_dt, positions, rope, cache, &a)) return s;
  if (batch == 0) return MLA_OK;
  a.batch = batch;
  a.n_partials = 1;
  const hipError_t e = launch_cache_store(a, batch, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_cache_append(const mla_dims_t* dims, int32_t d_model, int32_t batch, const void* h,
                              mla_dtype_t h_dt, const void* w_dkv, const void* w_kr, mla_dtype_t w_dt, float* rows,
                              const int32_t* positions, float rope_base, const mla_paged_cache_t* cache,
                              void* stream) {
  const mla_rope_t r{rope_base, 1.f, 0.f, 0.f, 0};
  return mla_cache_append_rope(dims, d_model, batch, h, h_dt, w_dkv, w_kr, w_dt, rows, positions, &r, cache, stream);
}

mla_status_t mla_cache_append_rope(const mla_dims_t* dims, int32_t d_model, int32_t batch, const void* h,
                                   mla_dtype_t h_dt, const void* w_dkv, const void* w_kr, mla_dtype_t w_dt,
                                   float* rows, const int32_t* positions, const mla_rope_t* rope,
                                   const mla_paged_cache_t* cache, void* stream) {
  CacheStoreArgs a{};
  if (mla_status_t s = store_args(dims, batch, rows, MLA_F32, positions, rope, cache, &a)) return s;
  if (d_model < 1) return MLA_ERR_INVALID_ARG;
  if ((h_dt != MLA_F32 && h_dt != MLA_BF16) || (w_dt != MLA_F32 && w_dt != MLA_BF16))
    return valid_dtype(h_dt) && valid_dtype(w_dt) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if (batch == 0) return MLA_OK;
  if (!h || !w_dkv || (dims->d_rope > 0 && !w_kr)) return MLA_ERR_INVALID_ARG;
  if (!aligned16(h) || !aligned16(w_dkv) || (w_kr && !aligned16(w_kr))) return MLA_ERR_ALIGNMENT;
  GemmArgs g{};
  g.x = h;
  g.x_dt = h_dt;
  g.w0 = w_dkv;
  g.w1 = w_kr;
  g.w_dt = w_dt;
  g.out = rows;
  g.batch = batch;
  g.K = d_model;
  g.N = dims->d_latent + dims->d_rope;
  g.n0 = dims->d_latent;
  gemm_ws_plan(g, kGemmMaxSlices);
  a.batch = batch;
  a.n_partials = g.slices;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_gemm_ws(g, st);
  if (e == hipSuccess) e = launch_cache_store(a, batch, st);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

size_t mla_query_prep_scratch_size(const mla_dims_t* dims, int32_t d_qlatent, int32_t batch) {
  if (check_dims(dims) != MLA_OK || d_qlatent < 0 || batch < 0) return 0;
  return query_scratch(dims, d_qlatent, batch).total;
}

mla_status_t mla_query_prep(const mla_dims_t* dims, int32_t d_model, int32_t d_qlatent, int32_t batch,
                            const void* h, mla_dtype_t h_dt, const void* w_dq, const void* w_uq, const void* w_qr,
                            mla_dtype_t w_dt, const int32_t* positions, float rope_base, void* q_nope, void* q_pe,
                            mla_dtype_t out_dt, void* scratch, size_t scratch_bytes, void* stream) {
  const mla_rope_t r{rope_base, 1.f, 0.f, 0.f, 0};
  return mla_query_prep_rope(dims, d_model, d_qlatent, batch, h, h_dt, w_dq, w_uq, w_qr, w_dt, positions, &r, q_nope,
                             q_pe, out_dt, scratch, scratch_bytes, stream);
}

float mla_yarn_attention_factor(float yarn_scale) {
  if (!(yarn_scale > 1.f)) return 1.f;
  const double f = 0.0707 * std::log(double(yarn_scale)) + 1.0;
  return float(f * f);
}

mla_status_t mla_query_prep_rope(const mla_dims_t* dims, int32_t d_model, int32_t d_qlatent, int32_t batch,
                                 const void* h, mla_dtype_t h_dt, const void* w_dq, const void* w_uq,
                                 const void* w_qr, mla_dtype_t w_dt, const int32_t* positions,
                                 const mla_rope_t* rope, void* q_nope, void* q_pe, mla_dtype_t out_dt, void* scratch,
                                 size_t scratch_bytes, void* stream) {
  if (mla_status_t s = check_dims(dims)) return s;
  RopeParams rp;
  if (mla_status_t s = rope_params(rope, &rp)) return s;
  if (batch < 0 || d_model < 1 || d_qlatent < 0) return MLA_ERR_INVALID_ARG;
  const bool compressed = d_qlatent > 0;
  for (mla_dtype_t t : {h_dt, w_dt, out_dt})
    if (t != MLA_F32 && t != MLA_BF16) return valid_dtype(t) ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  if ((dims->d_head & 1) || (dims->d_rope & 1)) return MLA_ERR_UNSUPPORTED;
  const QueryScratch L = query_scratch(dims, d_qlatent, batch);
  if (batch == 0) return MLA_OK;
  if (!h || (compressed && !w_dq) || !w_uq || !q_nope || (dims->d_rope > 0 && (!w_qr || !q_pe || !positions)))
    return MLA_ERR_INVALID_ARG;
  if (!scratch || scratch_bytes < L.total) return MLA_ERR_WORKSPACE;
  if (!aligned16(h) || (compressed && !aligned16(w_dq)) || !aligned16(w_uq) || (w_qr && !aligned16(w_qr)) ||
      !aligned16(scratch))
    return MLA_ERR_ALIGNMENT;
  char* ws = static_cast<char*>(scratch);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // stage 2's plan first: with one k slice (the V2 shapes) its epilogue writes
  // q^C and the rotated q^R itself, from a RoPE table that stage 1's reduction
  // launch computes
  const int nc = dims->n_heads * dims->d_head;
  GemmArgs g2{};
  g2.x = compressed ? static_cast<const void*>(ws + L.cq) : h;
  g2.x_dt = compressed ? w_dt : h_dt;
  g2.w0 = w_uq;
  g2.w1 = w_qr;
  g2.w_dt = w_dt;
  g2.out = reinterpret_cast<float*>(ws + L.s2);
  g2.batch = batch;
  g2.K = compressed ? d_qlatent : d_model;
  g2.N = dims->n_heads * (dims->d_head + dims->d_rope);
  g2.n0 = nc;
  gemm_ws_plan(g2, kQueryMaxSlices);
  const bool fused = compressed && g2.use_mfma && g2.slices == 1 && nc % 4 == 0 && dims->d_rope % 4 == 0 &&
                     aligned16(q_nope) && (dims->d_rope == 0 || aligned16(q_pe));
  RopeTableArgs tab{positions, rp, batch, dims->d_rope, nullptr};
  if (fused) {
    g2.fin_nope = q_nope;
    g2.fin_pe = q_pe;
    g2.fin_dt = out_dt;
    g2.fin_drope = dims->d_rope;
    if (dims->d_rope > 0 && rp.base > 0.f) {
      tab.table = reinterpret_cast<double*>(ws + L.tab);
      g2.fin_rope = tab.table;
    }
  }
  if (compressed) {
  // stage 1: c^Q = W^DQ h
  GemmArgs g1{};
  g1.x = h;
  g1.x_dt = h_dt;
  g1.w0 = w_dq;
  g1.w1 = nullptr;
  g1.w_dt = w_dt;
  g1.out = reinterpret_cast<float*>(ws + L.s1);
  g1.batch = batch;
  g1.K = d_model;
  g1.N = d_qlatent;
  g1.n0 = d_qlatent;
  gemm_ws_plan(g1, kQueryMaxSlices);
  e = launch_gemm_ws(g1, st);
  if (e == hipSuccess)
    e = launch_reduce_cast(g1.out, g1.slices, int64_t(batch) * d_qlatent, ws + L.cq, w_dt, tab, st);
  }
  // stage 2: [q^C ; q^R before rotation] = [W^UQ ; W^QR] c^Q (or h when the
  // query is not compressed), then rotate and write
  if (e == hipSuccess) e = launch_gemm_ws(g2, st);
  if (fused) return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
  QueryFinishArgs f{};
  f.slices = g2.out;
  f.n_slices = g2.slices;
  f.batch = batch;
  f.n_heads = dims->n_heads;
  f.d_head = dims->d_head;
  f.d_rope = dims->d_rope;
  f.positions = positions;
  f.rope = rp;
  f.q_nope = q_nope;
  f.q_pe = q_pe;
  f.out_dt = out_dt;
  if (e == hipSuccess) e = launch_query_finish(f, st);
  return e == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_validate_cache_host(const int32_t* block_table_host, const int32_t* seq_lens_host, int32_t batch,
                                     int32_t max_pages_per_seq, int32_t page_size, int32_t num_pages,
                                     int32_t* bad_seq) {
  if (bad_seq) *bad_seq = -1;
  if (batch < 0 || max_pages_per_seq < 1 || page_size < 1 || num_pages < 1) return MLA_ERR_INVALID_ARG;
  if (batch > 0 && (!block_table_host || !seq_lens_host)) return MLA_ERR_INVALID_ARG;
  const int64_t max_tokens = int64_t(max_pages_per_seq) * page_size;
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t T = seq_lens_host[b];
    bool ok = T >= 0 && int64_t(T) <= max_tokens;
    const int64_t np = ok ? (int64_t(T) + page_size - 1) / page_size : 0;
    const int32_t* row = block_table_host + int64_t(b) * max_pages_per_seq;
    for (int64_t p = 0; ok && p < np; ++p) ok = row[p] >= 0 && row[p] < num_pages;
    if (!ok) {
      if (bad_seq) *bad_seq = b;
      return MLA_ERR_INVALID_ARG;
    }
  }
  return MLA_OK;
}

mla_status_t mla_partition_host(const int32_t* seq_lens_host, int32_t batch, int32_t page_size,
                                int32_t max_pages_per_seq, const mla_partition_t* part, int32_t* part_first,
                                int32_t* part_count) {
  if (batch < 0 || (batch > 0 && (!seq_lens_host || !part_first || !part_count))) return MLA_ERR_INVALID_ARG;
  if (part && part->num_parts < 0 && part->split_tokens == 0) return MLA_ERR_INVALID_ARG;
  mla_dims_t d{1, 1, 0, 1};
  PartParams pp;
  int n_items = 0, n_slots = 0;
  if (mla_status_t s = resolve(&d, batch, max_pages_per_seq, page_size, part, &pp, &n_items, &n_slots)) return s;
  int64_t P = 0, m = 0;
  for (int b = 0; b < batch; ++b) {
    if (seq_lens_host[b] < 0 || int64_t(seq_lens_host[b]) > int64_t(max_pages_per_seq) * page_size)
      return MLA_ERR_INVALID_ARG;
    P += ceil_div(seq_lens_host[b], page_size);
    m += seq_lens_host[b] > 0 ? 1 : 0;
  }
  const int64_t W = pp.mode == PART_BALANCED ? (pp.num_parts < P ? pp.num_parts : P) : 0;
  const int64_t C = cost_units(P, m);
  int64_t S = 0;   // first cost unit of sequence b (balanced)
  for (int b = 0; b < batch; ++b) {
    const int T = seq_lens_host[b];
    const int np = ceil_div(T, page_size);
    if (T == 0) {
      part_first[b] = -1;
      part_count[b] = 0;
    } else if (pp.mode == PART_WHOLE) {
      part_first[b] = -1;
      part_count[b] = 1;
    } else if (pp.mode == PART_FIXED) {
      part_first[b] = b * pp.fixed_slots;
      part_count[b] = ceil_div(T, pp.split_tokens);
    } else {
      const int wf = part_of_unit(S, C, W), wl = part_of_unit(S + np - 1, C, W);
      part_first[b] = wf + b;
      part_count[b] = wl - wf + 1;
    }
    if (np > 0) S += np + kSegCost;
  }
  return MLA_OK;
}

mla_status_t mla_prefill_workspace_size(const mla_dims_t* dims, int32_t batch, int64_t total_kv, size_t* bytes) {
  if (!bytes) return MLA_ERR_INVALID_ARG;
  PrefillLayout L;
  if (mla_status_t s = prefill_layout(dims, batch, total_kv, &L)) return s;
  *bytes = L.total;
  return MLA_OK;
}

mla_status_t mla_prefill(const mla_dims_t* dims, int32_t batch, const int32_t* q_offsets, int32_t total_q,
                         int32_t max_q_len, const void* q_nope, const void* q_pe, mla_dtype_t q_dt,
                         const mla_paged_cache_t* cache, int64_t total_kv, const void* w_uk, const void* w_uv,
                         mla_dtype_t w_dt, float softmax_scale, void* workspace, size_t workspace_bytes,
                         void* o_heads, mla_dtype_t out_dt, float* lse, void* stream) {
  PrefillLayout L;
  if (mla_status_t s = prefill_layout(dims, batch, total_kv, &L)) return s;
  if (total_q < 0 || max_q_len < 0 || cache == nullptr || !q_offsets) return MLA_ERR_INVALID_ARG;
  if (!q_nope || !q_pe || !w_uk || !w_uv || !o_heads) return MLA_ERR_INVALID_ARG;
  if (!cache->kv || !cache->block_table || !cache->seq_lens) return MLA_ERR_INVALID_ARG;
  if (cache->page_size < 1 || cache->max_pages_per_seq < 1 || cache->num_pages < 1) return MLA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !(softmax_scale < 1e30f)) return MLA_ERR_INVALID_ARG;
  for (mla_dtype_t t : {q_dt, w_dt, out_dt, cache->dtype})
    if (!valid_dtype(t)) return MLA_ERR_INVALID_ARG;
  if (q_dt != MLA_BF16 || w_dt != MLA_BF16 || out_dt != MLA_BF16) return MLA_ERR_UNSUPPORTED;
  if (cache->dtype == MLA_F32 || cache->page_size != 64) return MLA_ERR_UNSUPPORTED;
  if (cache->dtype == MLA_FP8_E4M3 && !cache->scales) return MLA_ERR_INVALID_ARG;
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(o_heads) ||
      !aligned16(cache->kv))
    return MLA_ERR_ALIGNMENT;
  if (!workspace || workspace_bytes < L.total) return MLA_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MLA_ERR_ALIGNMENT;
  const int64_t n_qblk = (int64_t(max_q_len) + 127) / 128;   // (blocks of at least 128 new tokens)
  if (int64_t(batch) * n_qblk * dims->n_heads > INT32_MAX) return MLA_ERR_UNSUPPORTED;
  if (batch == 0 || total_q == 0) return MLA_OK;

  PrefillArgs a{};
  a.batch = batch;
  a.n_heads = dims->n_heads;
  {
    const int64_t mt = int64_t(cache->max_pages_per_seq) * cache->page_size;
    a.max_tokens = mt > INT32_MAX ? INT32_MAX : int(mt);
  }
  a.max_pages = cache->max_pages_per_seq;
  a.num_pages = cache->num_pages;
  a.total_kv = total_kv;
  a.cap_rows = L.cap_rows;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.seq_lens = cache->seq_lens;
  a.block_table = cache->block_table;
  a.q_off = q_offsets;
  a.kv = cache->kv;
  a.scales = cache->scales;
  a.kv_dt = cache->dtype;
  a.q_nope = static_cast<const uint16_t*>(q_nope);
  a.q_pe = static_cast<const uint16_t*>(q_pe);
  a.w_uk = static_cast<const uint16_t*>(w_uk);
  a.w_uv = static_cast<const uint16_t*>(w_uv);
  a.scale_log2 = softmax_scale * kLog2e;
  char* ws = static_cast<char*>(workspace);
  a.cu = reinterpret_cast<int32_t*>(ws + L.cu);
  a.c_rows = reinterpret_cast<uint16_t*>(ws + L.rows);
  a.kv_up = reinterpret_cast<uint16_t*>(ws + L.kv);
  a.out = static_cast<uint16_t*>(o_heads);
  a.lse = lse;
  return launch_prefill(a, static_cast<hipStream_t>(stream)) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

}  // extern "C"
