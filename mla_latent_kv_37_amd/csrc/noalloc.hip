// mla_decode_noalloc: mla_decode followed by mla_merge_splits, for callers that
// cannot allocate device memory.  The split partials (o_s, lse_s and the
// balanced partition's slot record) live in `scratch`, a file-scope device
// array of kNoallocScratchBytes that the library owns; every GPU the library
// runs on holds its own copy until the process ends.  Partials are packed at
// the output dtype's size (2 bytes per element for bf16 output), so 48 MiB
// holds 384 slots of 128 heads x 512 latent columns: one work item per compute
// unit on a 256-CU device plus 128 sequences.
//
// Host code never passes the array's name to a kernel (it is a host-side
// stand-in there): the device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and that address is what the
// kernels receive.
//
// Every call on one GPU shares that GPU's array: calls that overlap in time on
// one GPU (different streams, different host threads) race.  No part of the
// array must start at zero: the decode writes every partial and slot record
// that the merge reads.
#include <mutex>

#include "api_internal.h"

namespace mla {
namespace {

constexpr size_t kNoallocScratchBytes = size_t(48) << 20;
static_assert(kNoallocScratchBytes == MLA_NOALLOC_SCRATCH_BYTES, "mla.h states the scratch size");

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up once per device).
mla_status_t scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MLA_OK;
}

}  // namespace
}  // namespace mla

extern "C" mla_status_t mla_decode_noalloc(const mla_dims_t* dims, int32_t batch, const void* q_lat,
                                           const void* q_pe, mla_dtype_t q_dt, const mla_paged_cache_t* cache,
                                           float softmax_scale, const mla_partition_t* part, void* o_lat,
                                           mla_dtype_t o_dt, float* lse, void* stream) {
  using namespace mla;
  if (!cache) return MLA_ERR_INVALID_ARG;
  if (o_dt != MLA_F32 && o_dt != MLA_BF16) return o_dt == MLA_FP8_E4M3 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG;
  const size_t o_elem = o_dt == MLA_BF16 ? 2 : 4;
  size_t need = 0;
  if (mla_status_t s = decode_workspace_layout(dims, batch, cache->max_pages_per_seq, cache->page_size, part, o_elem,
                                               &need))
    return s;
  if (need > kNoallocScratchBytes) return MLA_ERR_WORKSPACE;   // the partition needs more than the array holds
  void* ws = nullptr;
  if (need > 0)
    if (mla_status_t s = scratch_ptr(&ws)) return s;
  // every argument is checked before anything is enqueued
  if (mla_status_t s = decode_impl(dims, batch, q_lat, q_pe, q_dt, cache, softmax_scale, part, ws, need, o_lat, o_dt,
                                   lse, stream, true, o_elem, 1))
    return s;
  if (mla_status_t s = decode_impl(dims, batch, q_lat, q_pe, q_dt, cache, softmax_scale, part, ws, need, o_lat, o_dt,
                                   lse, stream, false, o_elem, 1))
    return s;
  return merge_impl(dims, batch, cache->seq_lens, cache->page_size, cache->max_pages_per_seq, part, ws, need, o_lat,
                    o_dt, lse, stream, o_elem);
}
