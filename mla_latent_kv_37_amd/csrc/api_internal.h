// Host-side implementation pieces of the C ABI shared between api.hip and the
// no-allocation entry point (noalloc.hip).
#pragma once

#include "kernels.h"

namespace mla {

// mla_decode's checks and launch (dry = true: the checks only).  o_elem is the
// size of one partial element in the workspace layout: sizeof(float) for the
// public workspace, the output dtype's size where the library owns the memory.
mla_status_t decode_impl(const mla_dims_t* dims, int32_t batch, const void* q_lat, const void* q_pe,
                         mla_dtype_t q_dt, const mla_paged_cache_t* cache, float softmax_scale,
                         const mla_partition_t* part, void* workspace, size_t workspace_bytes, void* o_lat,
                         mla_dtype_t o_dt, float* lse, void* stream, bool dry, size_t o_elem, int bt_div);

// mla_merge_splits' checks and launch, with the same o_elem convention; q_len
// as for merge_out_proj_impl below.
mla_status_t merge_impl(const mla_dims_t* dims, int32_t batch, const int32_t* seq_lens, int32_t page_size,
                        int32_t max_pages_per_seq, const mla_partition_t* part, const void* workspace,
                        size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse, void* stream,
                        size_t o_elem, int q_len = 1);

// mla_merge_out_proj's checks and launch; q_len > 1: the virtual batch of a
// multi-token decode, lengths derived from seq_lens (PartParams::q_len).
mla_status_t merge_out_proj_impl(const mla_dims_t* dims, int32_t batch, const int32_t* seq_lens, int32_t page_size,
                                 int32_t max_pages_per_seq, const mla_partition_t* part, const void* workspace,
                                 size_t workspace_bytes, void* o_lat, mla_dtype_t o_dt, float* lse, const void* w_uv,
                                 mla_dtype_t w_dt, void* o_heads, mla_dtype_t out_dt, void* stream, int q_len);

// Workspace bytes of a partition with o_elem-byte partials.
mla_status_t decode_workspace_layout(const mla_dims_t* dims, int32_t batch, int32_t max_pages_per_seq,
                                     int32_t page_size, const mla_partition_t* part, size_t o_elem, size_t* bytes);

}  // namespace mla
