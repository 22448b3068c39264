// rtq_lane.hpp -- device building blocks of the one-lane-per-vector kernels
// (d = 64 / 128): sign masks, direct-to-LDS tile loads, per-row quantize,
// scale row loads and stores.  Shared by rtq.hip, rtq_cache.hip and
// rtq_ext.hip.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "rtq_device.hpp"
#include "rtq_div.hpp"
#include "rtq_mem.hpp"

namespace rtq {

enum Rot : int { kSRFT = 0, kSRHT = 1 };

// ---------------------------------------------------------------------------
// Sign masks
// ---------------------------------------------------------------------------

// XOR mask of packed pair m (elements 2m, 2m+1) from a word of 64 sign bits
// (bit e = element e): bit 2m goes to bit 15 (low fp16), bit 2m+1 to bit 31.
__device__ __forceinline__ uint32_t pair_mask(uint64_t bits, int m) {
  const uint32_t v = (uint32_t)(bits >> (2 * m)) & 3u;
  return (v * 0x40008000u) & 0x80008000u;
}

// h ^ m for a wave-uniform mask m kept in an SGPR: one VALU instruction.
__device__ __forceinline__ uint32_t xor_uniform(uint32_t h, uint32_t m) {
  uint32_t r;
  asm("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(m), "v"(h));
  return r;
}

// Sign masks of one seed for the D/2 packed pairs of a row, wave-uniform:
// lane l evaluates the sign bits of elements l, l + 64, ... and a ballot
// gathers them into scalar registers.
template <int D>
struct UniformSigns {
  uint32_t m[D / 2];

  // Seed offset j (wave-uniform) of base seed s0: the sign words come from
  // the host-filled table when it holds j, otherwise from a ballot.
  __device__ __forceinline__ void setup(const SignTable& tb, uint32_t j, uint64_t s0, int lane) {
    if (j < tb.seeds) {
      sfor<D / 64>([&](auto Q) {
        constexpr int q = RTQ_CI(Q);
        const uint64_t bits = tb.w[j * (D / 64) + q];
        sfor<32>([&](auto M) { m[32 * q + RTQ_CI(M)] = pair_mask(bits, RTQ_CI(M)); });
      });
      return;
    }
    const uint64_t s = s0 + j;
    sfor<D / 64>([&](auto Q) {
      constexpr int q = RTQ_CI(Q);
      const uint64_t bits = __ballot(sign_bit(s, (uint32_t)(64 * q + lane)));
      sfor<32>([&](auto M) { m[32 * q + RTQ_CI(M)] = pair_mask(bits, RTQ_CI(M)); });
    });
  }

  __device__ __forceinline__ void apply(uint32_t (&h)[D / 2]) const {
    sfor<D / 2>([&](auto M) { h[RTQ_CI(M)] = xor_uniform(h[RTQ_CI(M)], m[RTQ_CI(M)]); });
  }
};

// Signs of a lane's own seed s, evaluated element by element; used only for
// the few tiles whose rows straddle a seed boundary.
template <int D>
__device__ __forceinline__ void apply_lane_signs(uint32_t (&h)[D / 2], uint64_t s) {
  sfor<D / 64>([&](auto Q) {
    uint64_t bits = 0;
#pragma unroll 1
    for (uint32_t e = 0; e < 64; ++e) bits |= (uint64_t)sign_bit(s, 64u * RTQ_CI(Q) + e) << e;
    sfor<32>([&](auto M) { h[32 * RTQ_CI(Q) + RTQ_CI(M)] ^= pair_mask(bits, RTQ_CI(M)); });
  });
}

// Seed of the row a lane owns in a tile (rows past the end reuse the last).
__device__ __forceinline__ uint64_t lane_seed(const SeedRule& sr, uint32_t row0, int rows, int lane) {
  return seed_of_block(seed_block(row0 + (uint32_t)(lane < rows ? lane : rows - 1), sr), sr);
}

// XOR masks flipping the fp16 sign bits of chunk k (elements 8k .. 8k+7) for
// seed offset j (wave-uniform) of base seed s0, from the host-filled table
// when it holds j (D = 256: four words per seed), otherwise evaluated here.
__device__ __forceinline__ uint4 chunk_masks(const SignTable& tb, uint32_t j, uint64_t s0, uint32_t k) {
  if (j < tb.seeds) {
    const uint64_t w0 = tb.w[4 * j], w1 = tb.w[4 * j + 1], w2 = tb.w[4 * j + 2], w3 = tb.w[4 * j + 3];
    const uint32_t q = k >> 3;
    const uint64_t w = q == 0 ? w0 : q == 1 ? w1 : q == 2 ? w2 : w3;
    const uint64_t byte = (w >> (8 * (k & 7))) & 0xffu;
    return make_uint4(pair_mask(byte, 0), pair_mask(byte, 1), pair_mask(byte, 2), pair_mask(byte, 3));
  }
  return chunk_sign_masks(s0 + j, k);
}

// ---------------------------------------------------------------------------
// d = 64 / 128: one lane per vector, 64 vectors per tile.
// ---------------------------------------------------------------------------

// Direct-to-LDS staging of one tile.  Load instruction j of lane i fills LDS
// slot 64j + i (hardware layout); slot s holds row r = s / CPR, chunk
// k = (s % CPR) ^ (r & 7).  The xor swizzle makes the owning lane's
// ds_read_b128 of its row conflict free while every row's chunks still come
// from one contiguous row in HBM.  A partial tile reloads its last row.
template <int CPR>
__device__ __forceinline__ void load_tile_to_lds(const uint4* __restrict__ xt, int rows, uint4* buf, int lane) {
  auto issue = [&](auto J, int rmax) {
    const int slot = RTQ_CI(J) * 64 + lane;
    const int r = slot / CPR;
    const int k = (slot % CPR) ^ (r & 7);
    const int rr = r < rmax ? r : rmax - 1;
    const uint32_t off = (uint32_t)(rr * CPR + k) * 16u;
    __builtin_amdgcn_global_load_lds((gbl_void_t*)((const char*)xt + off), (lds_void_t*)(buf + RTQ_CI(J) * 64), 16, 0,
                                     kCachePolicyNT);
  };
  if (rows == 64) {
    sfor<CPR>([&](auto J) { issue(J, 64); });
  } else {
    sfor<CPR>([&](auto J) { issue(J, rows); });
  }
}

template <int CPR>
__device__ __forceinline__ void read_own_row(const uint4* buf, int lane, uint32_t (&h)[CPR * 4]) {
  const int sw = lane & 7;
  sfor<CPR>([&](auto C) {
    const uint4 q = buf[lane * CPR + (RTQ_CI(C) ^ sw)];
    h[4 * RTQ_CI(C) + 0] = q.x;
    h[4 * RTQ_CI(C) + 1] = q.y;
    h[4 * RTQ_CI(C) + 2] = q.z;
    h[4 * RTQ_CI(C) + 3] = q.w;
  });
}

template <int D, int G, int ROT>
__device__ __forceinline__ void quantize_row(const uint32_t (&h)[D / 2], uint32_t (&cw)[D / 8],
                                             uint32_t (&sb)[D / G]) {
  float z[D];
  float zs;
  if constexpr (ROT == kSRFT) {
    srft_fwd_unscaled<D>(h, z);
    zs = SrftScale<D>::value;
  } else {
    fwht_from_f16<D>(h, z);
    zs = InvSqrt<D>::value;
  }
  quantize_pack<D, G>(z, zs, cw, sb);
}

// u = lambda (.) h (fp16 pairs times fp16 pairs, exact in fp32); lam holds d
// fp16 values, one per channel.
template <int D>
__device__ __forceinline__ void lambda_weight(const uint32_t (&h)[D / 2], const uint32_t* __restrict__ lam,
                                              float (&u)[D]) {
  sfor<D / 2>([&](auto K) {
    constexpr int k = RTQ_CI(K);
    const uint32_t l = lam[k];
    u[2 * k] = lo_f(h[k]) * lo_f(l);
    u[2 * k + 1] = hi_f(h[k]) * hi_f(l);
  });
}

// inv[c] = 1 / lambda_c for the D channels, lane c mod 64 computing channel
// c: one reciprocal per lane and 64 channels instead of one per value of
// every row (lambda is the same for all rows).  Visible to the whole wave
// after the caller's next LDS barrier.
template <int D>
__device__ __forceinline__ void lambda_reciprocals(const uint32_t* __restrict__ lam, float* inv, int lane) {
  sfor<D / 64>([&](auto I) {
    const int c = RTQ_CI(I) * 64 + lane;
    const uint32_t l = lam[c / 2];
    inv[c] = __builtin_amdgcn_rcpf((c & 1) ? hi_f(l) : lo_f(l));
  });
}

// u *= inv, channel by channel (inv from lambda_reciprocals, read as
// broadcasts).
template <int D>
__device__ __forceinline__ void lambda_unweight_lds(float (&u)[D], const float* inv) {
  sfor<D / 4>([&](auto K) {
    constexpr int k = RTQ_CI(K);
    const float4 r = *reinterpret_cast<const float4*>(inv + 4 * k);
    u[4 * k] *= r.x;
    u[4 * k + 1] *= r.y;
    u[4 * k + 2] *= r.z;
    u[4 * k + 3] *= r.w;
  });
}

// quantize_row of lambda (.) h: the transform then runs on fp32 input.
template <int D, int G, int ROT>
__device__ __forceinline__ void quantize_row_lambda(const uint32_t (&h)[D / 2], const uint32_t* __restrict__ lam,
                                                    uint32_t (&cw)[D / 8], uint32_t (&sb)[D / G]) {
  float u[D];
  lambda_weight<D>(h, lam, u);
  if constexpr (ROT == kSRFT) {
    float z[D];
    srft_fwd<D>(u, z);
    quantize_pack<D, G>(z, 1.0f, cw, sb);
  } else {
    fwht_f32<D>(u);
    quantize_pack<D, G>(u, InvSqrt<D>::value, cw, sb);
  }
}

// scales of one row, packed as written to memory (fp16 pairs, low half first)
template <int D, int G>
__device__ __forceinline__ void store_row_scales(uint8_t* __restrict__ st, uint32_t r, const uint32_t (&sb)[D / G]) {
  if constexpr (D / G == 1) {
    stream_store(reinterpret_cast<uint16_t*>(st) + r, (uint16_t)sb[0]);
  } else if constexpr (D / G == 2) {
    stream_store(reinterpret_cast<uint32_t*>(st) + r, sb[0] | (sb[1] << 16));
  } else {
    stream_store(reinterpret_cast<uint2*>(st) + r, make_uint2(sb[0] | (sb[1] << 16), sb[2] | (sb[3] << 16)));
  }
}

template <int D, int G>
__device__ __forceinline__ void load_row_scales(const uint8_t* __restrict__ st, uint32_t r, uint32_t (&sb)[D / G]) {
  if constexpr (D / G == 1) {
    sb[0] = stream_load(reinterpret_cast<const uint16_t*>(st) + r);
  } else if constexpr (D / G == 2) {
    const uint32_t w = stream_load(reinterpret_cast<const uint32_t*>(st) + r);
    sb[0] = w & 0xffffu;
    sb[1] = w >> 16;
  } else {
    const uint2 w = stream_load(reinterpret_cast<const uint2*>(st) + r);
    sb[0] = w.x & 0xffffu;
    sb[1] = w.x >> 16;
    sb[2] = w.y & 0xffffu;
    sb[3] = w.y >> 16;
  }
}

// Output transpose passes of the inverse: d = 128 in two passes of 32 rows.
template <int D> struct InvPhases { static constexpr int value = D == 128 ? 2 : 1; };

// Flip the sign bits of h by the lane's seed s: one ballot per 64 elements
// when every lane of the wave has the same seed, element by element otherwise.
template <int D>
__device__ __forceinline__ void flip_signs(uint32_t (&h)[D / 2], uint64_t s, int lane) {
  const uint64_t s0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(s >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)s);
  if (__all(s == s0)) {
    sfor<D / 64>([&](auto Q) {
      constexpr int q = RTQ_CI(Q);
      const uint64_t bits = __ballot(sign_bit(s0, (uint32_t)(64 * q + lane)));
      sfor<32>([&](auto M) { h[32 * q + RTQ_CI(M)] ^= pair_mask(bits, RTQ_CI(M)); });
    });
  } else {
    apply_lane_signs<D>(h, s);
  }
}

}  // namespace rtq
