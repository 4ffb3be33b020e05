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

struct ProjectArgs {
  const void* h;           // [B, d_model]
  mla_dtype_t h_dt;
  const void* w_dkv;       // [d_c, d_model]
  const void* w_kr;        // [d_rope, d_model]
  mla_dtype_t w_dt;
  float* rows;             // [ksplit, B, d_c + d_rope]
  int batch, d_model, d_latent, d_rope;
  int ksplit;              // k slices (1: the generic kernel writes the rows directly)
};

hipError_t launch_decode_v2(const V2DecodeArgs& a, hipStream_t st);
hipError_t launch_cache_store(const CacheStoreArgs& a, int batch, hipStream_t st);
hipError_t launch_project(const ProjectArgs& a, hipStream_t st);
// k slices the projection of mla_cache_append uses for these operands
int project_ksplit(mla_dtype_t h_dt, mla_dtype_t w_dt, int width, int d_model);
hipError_t launch_merge(const MergeArgs& a, int batch, hipStream_t st);
hipError_t launch_absorb_generic(const void* q, mla_dtype_t q_dt, const void* w, mla_dtype_t w_dt, void* out,
                                 mla_dtype_t o_dt, int batch, int n_heads, int d_head, int d_latent, hipStream_t st);
hipError_t launch_outproj_generic(const void* o, mla_dtype_t o_dt, const void* w, mla_dtype_t w_dt, void* out,
                                  mla_dtype_t out_dt, int batch, int n_heads, int d_head, int d_latent,
                                  hipStream_t st);
hipError_t launch_absorb_v2(const void* q, const void* w, void* out, int batch, hipStream_t st);
hipError_t launch_outproj_v2(const void* o_lat, bool o_f32, const void* w, void* out, int batch, hipStream_t st);

}  // namespace mla
