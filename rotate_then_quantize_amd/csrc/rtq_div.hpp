// rtq_div.hpp -- unsigned 32-bit division by a run-time invariant divisor with
// one multiply-high, used for the per-row seed rule
//   seed(r) = seed + ((r / rows_per_seed) % seed_period).
//
// Method: Granlund & Montgomery, "Division by Invariant Integers using
// Multiplication" (PLDI 1994), unsigned case: for 1 <= d < 2^32 let
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1, s1 = min(l, 1),
// s2 = max(l - 1, 0); then for every 0 <= n < 2^32
//   t = mulhi(m, n),  n / d = (t + ((n - t) >> s1)) >> s2.
// The host builds the constants once per call; the kernels apply them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtq {

struct Div32 {
  uint32_t m;
  uint32_t s1;
  uint32_t s2;
  uint32_t d;
};

inline Div32 make_div32(uint32_t d) {  // host only
  Div32 r;
  uint32_t l = 0;
  while (l < 32 && (1ull << l) < d) ++l;
  const unsigned __int128 two32 = (unsigned __int128)1 << 32;
  r.m = (uint32_t)((two32 * (((unsigned __int128)1 << l) - d)) / d + 1);
  r.s1 = l < 1 ? l : 1;
  r.s2 = l > 1 ? l - 1 : 0;
  r.d = d;
  return r;
}

__host__ __device__ inline uint32_t div32(uint32_t n, const Div32& v) {
  const uint32_t t = (uint32_t)(((uint64_t)v.m * n) >> 32);
  return (t + ((n - t) >> v.s1)) >> v.s2;
}

// Per-row sign-seed rule of one call.  rps == 0 means one seed for all rows;
// period == 0 means the block index is not wrapped.
struct SeedRule {
  uint64_t seed;
  uint32_t rps;
  uint32_t period;
  Div32 by_rps;
  Div32 by_period;
};

__host__ __device__ inline uint32_t seed_block(uint32_t row, const SeedRule& s) {
  return s.rps ? div32(row, s.by_rps) : 0u;
}

// Offset of a block's seed from the base seed: (block mod period), or block.
__host__ __device__ inline uint32_t seed_offset(uint32_t block, const SeedRule& s) {
  return s.period ? block - div32(block, s.by_period) * s.period : block;
}

__host__ __device__ inline uint64_t seed_of_block(uint32_t block, const SeedRule& s) {
  return s.seed + seed_offset(block, s);
}

// Sign words of the first seeds of a call, filled on the host and passed by
// value in the kernel arguments: entry j holds the D/64 words of seed
// (seed + j), word q bit e being the sign bit of element 64 q + e.  Seed
// offsets at or beyond `seeds` are evaluated on the device.
constexpr int kSignTableWords = 128;

struct SignTable {
  uint32_t seeds;
  uint32_t words_per_seed;
  uint64_t w[kSignTableWords];
};

}  // namespace rtq
