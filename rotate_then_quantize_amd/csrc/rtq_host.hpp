// rtq_host.hpp -- host-side helpers shared by the C ABI translation units:
// argument checks, the seed rule as the kernels apply it, and the launch.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "rtq.h"
#include "rtq_div.hpp"

namespace rtq {

// ---------------------------------------------------------------------------
// Host side: validation, launch configuration, dispatch.
// ---------------------------------------------------------------------------

using KernelFn = const void*;

// Rows per call: row indices are 32-bit on the device.
constexpr int64_t kMaxRows = 0xffffff00ll;

// One wave per tile.  The grid is derived from the row count alone (no
// occupancy query): the hardware dispatcher keeps every CU filled from a
// grid far larger than the machine.
inline rtq_status launch(KernelFn fn, int64_t tiles, void** kargs, hipStream_t stream) {
  if (tiles <= 0 || tiles > 0x7fffffff) return RTQ_ERR_INVALID_ARG;
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)tiles), dim3(64), kargs, 0, stream);
  return e == hipSuccess ? RTQ_OK : RTQ_ERR_HIP;
}

inline bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Supported (d, group): d in {64,128,256}; group in {32,64,128,256}, group <= d
// (group == d is one scale per vector, the per-token recipe).
inline rtq_status check_shape(int32_t d, int32_t g) {
  if (d != 64 && d != 128 && d != 256) return RTQ_ERR_UNSUPPORTED;
  if (g != 32 && g != 64 && g != 128 && g != 256) return RTQ_ERR_UNSUPPORTED;
  if (g > d) return RTQ_ERR_UNSUPPORTED;
  return RTQ_OK;
}

// The row seed rule as the kernels apply it: rows_per_seed >= n selects one
// seed for all rows, exactly as rows_per_seed == 0 does.
inline SeedRule make_seed_rule(uint64_t seed, int64_t rps, int32_t period, int64_t n) {
  SeedRule s;
  s.seed = seed;
  s.rps = (rps == 0 || rps >= n) ? 0u : (uint32_t)rps;
  s.period = (uint32_t)period;
  s.by_rps = make_div32(s.rps ? s.rps : 1u);
  s.by_period = make_div32(s.period ? s.period : 1u);
  return s;
}

// Sign words of the first seeds of a call for the kernels' sign table
// (defined with the int4 kernels in rtq.hip).
void fill_sign_table(SignTable& tb, const SeedRule& sr, int64_t n, int d);

// The one-lane-per-row int4 kernels with a per-channel lambda (d = 64 / 128),
// or null.  Their arguments: in, out0, out1, lambda, rows, SeedRule,
// SignTable.
KernelFn find_lane_lambda_kernel(bool fwd, int rot, int d, int g);

}  // namespace rtq
