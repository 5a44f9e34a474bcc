#pragma once
// Device helpers for data that one workgroup writes and another reads within
// the same kernel (split-K partial tiles, attention partitions).  The XCDs'
// L2 caches are not coherent with each other, so such data is written and
// read with agent-scope relaxed atomics (sc1 accesses: coherent at device
// scope without writing back or invalidating the whole L2, which a
// device-scope fence would do once per workgroup), and a writer waits for its
// stores to complete (wait_vmcnt<0>) before it signals arrival with an
// agent-scope atomic on a counter.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef float pkv_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void st_agent(float* p, pkv_f32x4 v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  __hip_atomic_store(q, __builtin_bit_cast(uint64_t, float2{v[0], v[1]}), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, __builtin_bit_cast(uint64_t, float2{v[2], v[3]}), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ pkv_f32x4 ld_agent(const float* p) {
  uint64_t* q = const_cast<uint64_t*>(reinterpret_cast<const uint64_t*>(p));
  const float2 a = __builtin_bit_cast(float2, __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const float2 b = __builtin_bit_cast(float2, __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return pkv_f32x4{a.x, a.y, b.x, b.y};
}
__device__ __forceinline__ void st_agent2(float2* p, float2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_agent2(const float2* p) {
  return __builtin_bit_cast(float2, __hip_atomic_load(const_cast<uint64_t*>(reinterpret_cast<const uint64_t*>(p)),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// f16 activations shared between the phases of one persistent kernel (the
// same rules: written with agent-scope stores, read with agent-scope loads,
// so that no XCD serves a stale L2 copy of a vector another XCD rewrote).
typedef _Float16 pkv_h16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ pkv_h16x8 ld_agent_h8(const _Float16* p) {
  uint64_t* q = const_cast<uint64_t*>(reinterpret_cast<const uint64_t*>(p));
  const uint64_t a = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t b = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  typedef uint64_t u64x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(pkv_h16x8, u64x2{a, b});
}
__device__ __forceinline__ _Float16 ld_agent_h(const _Float16* p) {
  return __builtin_bit_cast(_Float16, __hip_atomic_load(const_cast<unsigned short*>(
                                                            reinterpret_cast<const unsigned short*>(p)),
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_agent_h(_Float16* p, _Float16 v) {
  __hip_atomic_store(reinterpret_cast<unsigned short*>(p), __builtin_bit_cast(unsigned short, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace pkv
