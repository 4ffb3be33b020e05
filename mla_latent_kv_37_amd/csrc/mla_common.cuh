// Shared device/host helpers of libmla: element types, storage decoding and the
// partition of a batch's cache pages into work items.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla.h"

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
#define MLA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// scalar storage decode
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite or +-inf here).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// OCP E4M3FN code -> float, using gfx950's fp8 convert (OCP encoding on this target).
__device__ __forceinline__ float e4m3_to_f32(uint8_t c) {
  return __builtin_amdgcn_cvt_f32_fp8(uint32_t(c), 0);
}

template <mla_dtype_t DT> struct Elem;
template <> struct Elem<MLA_F32> {
  typedef float T;
  static __device__ __forceinline__ float load(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
};
template <> struct Elem<MLA_BF16> {
  typedef uint16_t T;
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  }
};
template <> struct Elem<MLA_FP8_E4M3> {
  typedef uint8_t T;
  static __device__ __forceinline__ float load(const void* p, int64_t i) {
    return e4m3_to_f32(static_cast<const uint8_t*>(p)[i]);
  }
};

__device__ __forceinline__ float load_any(const void* p, int64_t i, mla_dtype_t dt) {
  return dt == MLA_F32 ? Elem<MLA_F32>::load(p, i) : Elem<MLA_BF16>::load(p, i);
}
__device__ __forceinline__ void store_any(void* p, int64_t i, float v, mla_dtype_t dt) {
  if (dt == MLA_F32) static_cast<float*>(p)[i] = v;
  else static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
}

// ---------------------------------------------------------------------------
// partition of the batch into work items (see mla_partition_t in mla.h)
// ---------------------------------------------------------------------------
enum PartMode { PART_WHOLE = 0, PART_FIXED = 1, PART_BALANCED = 2 };

struct PartParams {
  int mode;
  int split_tokens;   // PART_FIXED
  int num_parts;      // PART_BALANCED (resolved, > 0)
  int fixed_slots;    // PART_FIXED: slots per sequence S
  int page_size;
  int batch;
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Read-only int32 metadata (block table, lengths) through the constant address
// space: scalar loads, counted by lgkmcnt, so waiting for them never waits for
// in-flight vector loads of cache tiles.
#define MLA_CONST __attribute__((address_space(4)))
__device__ __forceinline__ int load_const(const int32_t* p, int64_t i) {
  return ((const MLA_CONST int32_t*)(p))[i];
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt_hi[15:14]); fields not waited on are at their maximum.  Issued through
// the builtin so the compiler's own wait insertion knows what has completed.
constexpr int waitcnt_vm(int n) { return (n & 0xF) | (7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14); }
constexpr int waitcnt_lgkm(int n) { return 0xF | (7 << 4) | ((n & 0xF) << 8) | (3 << 14); }

// Workgroup barrier without the release/acquire fence that __syncthreads()
// implies (which waits for every outstanding vector memory operation).  The
// caller waits for what the other wavefronts must see (vmcnt for direct-to-LDS
// loads, lgkmcnt for LDS writes) before calling it.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// First page of part w when `pages` pages are divided into `parts` parts.
__host__ __device__ __forceinline__ int64_t part_start(int64_t w, int64_t pages, int64_t parts) {
  return (w * pages) / parts;
}

// The part holding global page p: the largest w with part_start(w) <= p.
__host__ __device__ __forceinline__ int part_of_page(int64_t p, int64_t pages, int64_t parts) {
  int64_t w = ((p + 1) * parts + pages - 1) / pages - 1;
  if (w < 0) w = 0;
  if (w > parts - 1) w = parts - 1;
  return int(w);
}

// One contiguous token range of one sequence, processed by one work item.
struct Segment {
  int b;
  int t0, t1;      // tokens [t0, t1)
  int slot;        // workspace slot for a partial result
  bool whole;      // covers the whole sequence: final output, no partial
};

}  // namespace mla
