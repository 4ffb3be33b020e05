// Kernel argument blocks and launchers shared by the C-ABI layer (api.hip) and
// the kernel translation units.
#pragma once

#include "partition.cuh"

namespace mla {

struct GenericDecodeArgs {
  const void* q_lat;
  const void* q_pe;
  mla_dtype_t q_dt;
  const void* kv;
  const float* scales;
  mla_dtype_t kv_dt;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int max_pages;
  int n_heads, d_rope, d_latent;
  float scale;
  PartParams pp;
  void* o_part;            // split partials, element type o_dt
  float* lse_part;
  int32_t* meta;
  void* o_lat;
  mla_dtype_t o_dt;
  float* lse;
};

struct V2DecodeArgs {
  const uint16_t* q_lat;   // [B, 128, 512] bf16
  const uint16_t* q_pe;    // [B, 128, 64] bf16
  const void* kv;          // [P, 64, 576] bf16 or fp8 E4M3 codes
  const float* scales;     // fp8: [P, 64, 5] fp32 group scales; else null
  mla_dtype_t kv_dt;
  const int32_t* block_table;
  const int32_t* seq_lens;
  int max_pages;
  int n_items;
  float scale_log2;        // softmax_scale * log2(e)
  PartParams pp;
  void* o_part;            // split partials, element type o_dt
  float* lse_part;
  int32_t* meta;
  void* o_lat;
  mla_dtype_t o_dt;
  float* lse;
};

struct MergeArgs {
  const int32_t* seq_lens;
  PartParams pp;
  int n_heads, d_latent;
  const void* o_part;      // split partials, element type o_dt
  const float* lse_part;
  const int32_t* meta;
  void* o_lat;
  mla_dtype_t o_dt;
  float* lse;
};

hipError_t launch_decode_generic(const GenericDecodeArgs& a, int n_items, hipStream_t st);
struct CacheStoreArgs {
  const void* rows;        // [B, d_c + d_rope]
  mla_dtype_t rows_dt;
  const int32_t* positions;
  float rope_base;
  void* kv;
  float* scales;
  mla_dtype_t kv_dt;
  const int32_t* block_table;
  int max_pages, page_size, num_pages;
  int d_latent, d_rope;
  int batch;
  int n_partials;          // > 1: rows holds that many fp32 k-slices of the projection
};

// out[s][b][n] = sum_{k in slice s} x[b][k] * W[n][k]; W = w0 rows [0, n0) over w1 rows [n0, N)
struct GemmArgs {
  const void* x;           // [batch, K]
  mla_dtype_t x_dt;
  const void* w0;          // [n0, K]
  const void* w1;          // [N - n0, K]
  mla_dtype_t w_dt;
  float* out;              // [slices, batch, N] fp32
  int batch, K, N, n0;
  int slices;              // set by gemm_ws_plan
  bool use_mfma;           // set by gemm_ws_plan
};

hipError_t launch_decode_v2(const V2DecodeArgs& a, hipStream_t st);
// 16 heads, d_c = 512, d_rope = 64, page 64, bf16 cache and queries (same arguments)
hipError_t launch_decode_lite(const V2DecodeArgs& a, hipStream_t st);
hipError_t launch_cache_store(const CacheStoreArgs& a, int batch, hipStream_t st);
struct QueryFinishArgs {
  const float* slices;     // [n_slices, batch, n_h * (d_h + d_rope)] fp32
  int n_slices, batch, n_heads, d_head, d_rope;
  const int32_t* positions;
  float rope_base;
  void* q_nope;            // [batch, n_h, d_h]
  void* q_pe;              // [batch, n_h, d_rope]
  mla_dtype_t out_dt;
};

constexpr int kGemmMaxSlices = 8;      // k slices of mla_cache_append's projection (its scratch holds 8)
constexpr int kQueryMaxSlices = 16;    // k slices of mla_query_prep's products
// k slices of the MFMA plan for an N x K bf16 product over `batch` rows (1 for every other plan)
int gemm_ws_slices(int N, int K, int batch, int max_slices);
void gemm_ws_plan(GemmArgs& a, int max_slices);   // chooses slices (<= max_slices) and the kernel
hipError_t launch_gemm_ws(const GemmArgs& a, hipStream_t st);
hipError_t launch_reduce_cast(const float* slices, int n_slices, int64_t count, void* out, mla_dtype_t out_dt,
                              hipStream_t st);
hipError_t launch_query_finish(const QueryFinishArgs& a, hipStream_t st);
hipError_t launch_merge(const MergeArgs& a, int batch, hipStream_t st);
// merge of split partials + W^UV projection (d_h 128, d_c 512, bf16)
hipError_t launch_merge_proj(const MergeArgs& a, const void* w_uv, void* o_heads, int batch, hipStream_t st);
hipError_t launch_expand(const int32_t* seq_lens, const int32_t* block_table, int batch, int q_len, int max_pages,
                         int32_t* lens_out, int32_t* bt_out, hipStream_t st);
hipError_t launch_absorb_generic(const void* q, mla_dtype_t q_dt, const void* w, mla_dtype_t w_dt, void* out,
                                 mla_dtype_t o_dt, int batch, int n_heads, int d_head, int d_latent, hipStream_t st);
hipError_t launch_outproj_generic(const void* o, mla_dtype_t o_dt, const void* w, mla_dtype_t w_dt, void* out,
                                  mla_dtype_t out_dt, int batch, int n_heads, int d_head, int d_latent,
                                  hipStream_t st);
hipError_t launch_absorb_v2(const void* q, const void* w, void* out, int batch, int n_heads, hipStream_t st);
hipError_t launch_outproj_v2(const void* o_lat, bool o_f32, const void* w, void* out, int batch, int n_heads,
                             hipStream_t st);

}  // namespace mla
