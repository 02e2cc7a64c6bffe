// Shared device/host helpers of the tvp library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tvp.h"

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

#define TVP_CHECK_HIP(expr)                         \
  do {                                              \
    hipError_t e_ = (expr);                         \
    if (e_ != hipSuccess) return TVP_ERR_HIP;       \
  } while (0)

#define TVP_LAUNCH_CHECK()                          \
  do {                                              \
    if (hipGetLastError() != hipSuccess) return TVP_ERR_HIP; \
  } while (0)

namespace tvp {

constexpr int kTileN = 32;      // channels per packed tile
constexpr int kBlockK = 64;     // k per packed block
constexpr int kBlockBytes = 3072;  // 32 x 64 x 12 bits
constexpr int kBlockBytesHi8 = 2048;  // 32 x 64 x 8 bits: the 8-bit leading view of the records

// Bytes of one packed tile block in the tensor's format.
__host__ __device__ inline int block_bytes(int32_t format) { return format == TVP_FMT_HI8 ? kBlockBytesHi8 : kBlockBytes; }

// Record block (tile t, k-block j) of a packed weight, k-block-major.
__host__ __device__ inline int64_t rec_block(int64_t t, int64_t j, int64_t n_tiles) { return j * n_tiles + t; }

constexpr int kMaxReq = 64;      // requests per batched pass

// Per-request bookkeeping passed by value to the batched kernels.
struct ReqInfo {
  int32_t n_req;
  int32_t ctx_len[kMaxReq];
  int32_t node_ptr[kMaxReq + 1];
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// bf16 bits -> fp32 (exact)
__device__ inline float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN with the sign kept.
__device__ inline uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x0040u) & 0xFFFFu;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950.  Same result as f32_to_bf16 for every
// non-NaN input.
typedef __bf16 bf16x2_vec_t __attribute__((ext_vector_type(2)));
typedef float f32x2_vec_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_vec_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_vec_t));
}

// 16-byte streaming load (non-temporal hint: the weight stream is read once).
__device__ inline uint4 load_nt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Device-scope stores and loads (the agent-scope cache bits): a store is
// written through to the device's coherence point before it counts as
// complete, and a load is served from there, never from a stale line of this
// XCD's L2.  Data that one workgroup hands to another inside a launch
// travels this way, so the receiver may run on any XCD without a write-back
// or invalidate of a whole L2 (which a device-scope fence costs on this part).
__device__ inline void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival of one workgroup at a counter shared by `total` workgroups, after
// every thread's device-scope stores: each wavefront waits for its own
// stores to complete (s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their
// maxima), the workgroup meets at a barrier, and one thread increments the
// counter with a device-scope atomic.  Returns true (to every thread) in the
// workgroup that arrives last, which also puts the counter back to zero; by
// then every other workgroup's stores are complete, so its device-scope
// loads see them.  No workgroup waits for another.  `flag` is an LDS word.
__device__ inline bool arrive_last(uint32_t* counter, uint32_t total, int* flag) {
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == total - 1u;
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last ? 1 : 0;
  }
  __syncthreads();
  return *flag != 0;
}

// Order every LDS access of this wavefront issued before the call ahead of
// those issued after it, without waiting on outstanding global loads.
__device__ inline void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

}  // namespace tvp
