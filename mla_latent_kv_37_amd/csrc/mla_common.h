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
  int max_tokens;     // max_pages_per_seq * page_size: longer lengths are read as this
  int q_len = 1;      // > 1: sequence i is new token i % q_len of seq_lens[i / q_len] (multi-token decode)
};

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// RoPE frequencies (mla_rope_t in mla.h): pair k of a d-wide RoPE slice turns
// at theta_k = base^(-2k/d) per position; with YaRN (scale s > 1) the pairs
// that turn fewer than alpha times over the original context are slowed by s,
// those turning more than beta times are kept, with a linear ramp in the
// number of turns between (the YaRN context extension the V2 explainer §3.1.3
// applies to the RoPE-carrying key).  fp64, as the angle that uses it.
struct RopeParams {
  float base;       // 0: no rotation
  float yarn_scale; // <= 1: plain RoPE
  float yarn_alpha, yarn_beta;
  float yarn_orig_ctx;
};
__device__ __forceinline__ double rope_theta(int k, int d, const RopeParams& r) {
  const double theta = pow(double(r.base), -2.0 * k / double(d));
  if (!(r.yarn_scale > 1.f)) return theta;
  const double turns = double(r.yarn_orig_ctx) * theta / (2.0 * 3.141592653589793);
  double g = (turns - double(r.yarn_alpha)) / (double(r.yarn_beta) - double(r.yarn_alpha));
  g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
  return (1.0 - g) * theta / double(r.yarn_scale) + g * theta;
}

// A sequence length as the kernels use it: clamped to [0, max_pages * page_size],
// so that no kernel reads past the sequence's block-table row whatever seq_lens
// holds (lengths outside that range are invalid input; mla_validate_cache_host
// reports them).
__host__ __device__ __forceinline__ int clamp_len(int T, const PartParams& pp) {
  return T < 0 ? 0 : (T > pp.max_tokens ? pp.max_tokens : T);
}

// Lengths of the sequences of a multi-token decode (q_len > 1): sequence i is
// new token t = i % q_len of cached sequence i / q_len, whose last q_len
// tokens are the new ones; token t sits at position T - q_len + t and attends
// to the T - q_len + t + 1 tokens up to it (none if that is not positive).
// seq_len_index gives the seq_lens entry to read, seq_len_of the length from
// that entry, clamped as clamp_len.  With q_len = 1 both are the identity.
__host__ __device__ __forceinline__ int seq_len_index(int i, const PartParams& pp) {
  return pp.q_len > 1 ? i / pp.q_len : i;
}
__host__ __device__ __forceinline__ int seq_len_of(int T, int i, const PartParams& pp) {
  if (pp.q_len > 1) T = T < 0 ? 0 : T - pp.q_len + i % pp.q_len + 1;
  return clamp_len(T, pp);
}

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

// One direct-to-LDS load: 64 lanes x 16 bytes from per-lane global addresses
// into 1 KB of LDS at `lds` (lane l's bytes at lds + 16 l).  Inline assembly,
// so the compiler does not track it: its completion is waited for with an
// explicit vmcnt before the barrier that publishes the data.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  const int m0 = uniform(int(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(m0), "v"(src)
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 15]
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
#define MLA_VM_CASE(i) case i: __builtin_amdgcn_s_waitcnt(waitcnt_vm(i)); break;
    MLA_VM_CASE(1) MLA_VM_CASE(2) MLA_VM_CASE(3) MLA_VM_CASE(4) MLA_VM_CASE(5) MLA_VM_CASE(6) MLA_VM_CASE(7)
    MLA_VM_CASE(8) MLA_VM_CASE(9) MLA_VM_CASE(10) MLA_VM_CASE(11) MLA_VM_CASE(12) MLA_VM_CASE(13) MLA_VM_CASE(14)
    MLA_VM_CASE(15)
#undef MLA_VM_CASE
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
  }
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Balanced partition cost stream.  The pages of the non-empty sequences, in
// sequence order, with kSegCost extra units after each one: sequence b's pages
// are units [u_b, u_b + n_b) and u_{b+1} = u_b + n_b + kSegCost.  The stream is
// C = P + kSegCost * (m - 1) units long (P pages, m non-empty sequences) and
// is cut into W equal (+-1 unit) parts.  The extra units stand for the fixed
// cost a work item pays for every further sequence it touches (that
// sequence's query loads and its output write), which per-phase timers put at
// about two pages of streaming for the 128-head kernel; without them the items
// holding two sequences finished last.  A single sequence is cut exactly as
// plain pages are.
constexpr int kSegCost = 2;

__host__ __device__ __forceinline__ int64_t cost_units(int64_t pages, int64_t nonempty) {
  return nonempty > 0 ? pages + int64_t(kSegCost) * (nonempty - 1) : 0;
}

// First unit of part w when `units` units are divided into `parts` parts.
__host__ __device__ __forceinline__ int64_t part_start(int64_t w, int64_t units, int64_t parts) {
  return (w * units) / parts;
}

// The part holding unit u: the largest w with part_start(w) <= u.
__host__ __device__ __forceinline__ int part_of_unit(int64_t u, int64_t units, int64_t parts) {
  int64_t w = ((u + 1) * parts + units - 1) / units - 1;
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
