// rtq_mem.hpp -- memory-access helpers shared by the rotate-then-quantize
// kernels (gfx950): address-space pointer types, non-temporal streaming
// loads and stores, and wait-count helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace rtq {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

// Streaming global accesses.  Every input and output byte is touched exactly
// once, so loads and stores carry the non-temporal ("nt") cache policy: the
// stream does not displace other lines, and the outputs do not linger dirty
// in L2 / last-level cache for the next launch to write back.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kCachePolicyNT = 2;  // "nt" bit of a global_load_lds cache-policy operand

__device__ __forceinline__ void stream_store(uint4* p, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void stream_store(uint2* p, uint2 v) {
  const u32x2_t w = {v.x, v.y};
  __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void stream_store(uint32_t* p, uint32_t v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void stream_store(uint16_t* p, uint16_t v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}
__device__ __forceinline__ uint2 stream_load(const uint2* p) {
  const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(w.x, w.y);
}
__device__ __forceinline__ uint32_t stream_load(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint16_t stream_load(const uint16_t* p) { return __builtin_nontemporal_load(p); }

// A wave's LDS instructions execute in order, so exchanging data between the
// lanes of one wave through LDS that no other wave touches only needs the
// compiler kept from reordering the accesses.  (__syncthreads would also
// wait for every outstanding global store and load of the wave.)
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): this wave's LDS reads have returned.
__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// vmcnt(N) (gfx9 encoding: expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace rtq
