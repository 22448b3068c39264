// rtq.hip -- fused rotate-then-quantize int4 kernels for MI355X (gfx950) and
// the C ABI declared in include/rtq.h.
//
// The method ("Quantization Speed Is Often a Kernel Problem", sections
// "First, the 17%" and "Fusing four steps into two kernels is not enough"):
// each K/V vector is multiplied by a fixed +-1 pattern and rotated (SRFT = real
// FFT, SRHT = Hadamard control), quantized to int4 with one absmax fp16 scale
// per group; the inverse dequantizes, rotates back and flips the signs.  One
// launch does the forward step for all rows, one launch the inverse.
//
// Mapping to CDNA4:
//   * A wave (64 lanes, one wave per workgroup) owns a tile of rows.  d = 64
//     and d = 128 vectors live in the registers of one lane (64 rows per
//     tile); d = 256 vectors span two lanes, lane v (even samples for SRFT,
//     first half for SRHT) and lane v+32 (32 rows per tile).
//   * Rows are read and written with fully coalesced 16-byte accesses and
//     transposed to / from the owning lane through a padded, wave-private LDS
//     tile (no barriers between waves).  The +-1 signs are applied on the
//     16-byte chunks during that transposition: a lane always handles the
//     same chunk position, so its XOR masks are computed once per seed.
//   * The transforms, the absmax reduction, rounding, clamping and nibble
//     packing are straight-line register code (rtq_device.hpp); there is no
//     dense contraction and no MFMA.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "rtq.h"
#include "rtq_device.hpp"

namespace rtq {

enum Rot : int { kSRFT = 0, kSRHT = 1 };

__device__ __forceinline__ void lds_sync() { __syncthreads(); }  // one-wave workgroup

// Cached XOR masks of this lane's chunk position for the seed of the current
// tile, recomputed only when the seed changes.
struct SignCache {
  uint64_t seed;
  uint4 m;
  bool valid;
};

// Prepare the cache for a tile [row0, row0 + rows); returns whether every row
// of the tile uses the same seed.
__device__ __forceinline__ bool tile_signs(SignCache& sc, uint64_t seed, int64_t row0, int rows, int64_t rps,
                                           int32_t period, uint32_t kpos) {
  const bool uniform = (rps == 0) || (row0 / rps == (row0 + rows - 1) / rps);
  if (uniform) {
    const uint64_t s = row_seed(seed, row0, rps, period);
    if (!sc.valid || sc.seed != s) {
      sc.m = chunk_sign_masks(s, kpos);
      sc.seed = s;
      sc.valid = true;
    }
  }
  return uniform;
}

// ---------------------------------------------------------------------------
// d = 64 / 128: one lane per vector, 64 vectors per tile.
// ---------------------------------------------------------------------------

template <int D, int G, int ROT>
__global__ __launch_bounds__(64) void fwd_lane_kernel(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, int64_t n, uint64_t seed,
                                                      int64_t rps, int32_t period) {
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int LROW = CPR + 1;  // padded LDS row (uint4), keeps ds_read_b128 conflict free
  __shared__ uint4 lds[64 * LROW];
  const int lane = threadIdx.x;
  const uint32_t kpos = lane % CPR;
  const int64_t tiles = (n + 63) / 64;
  SignCache sc;
  sc.valid = false;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t row0 = t * 64;
    const int rows = (int)(n - row0 < 64 ? n - row0 : 64);
    const bool uniform = tile_signs(sc, seed, row0, rows, rps, period, kpos);
    // coalesced load of the tile, sign flip, transpose into LDS
    if (uniform) {
      uint4 v[CPR];
      sfor<CPR>([&](auto J) {
        const int rl = (RTQ_CI(J) * 64 + lane) / CPR;
        v[RTQ_CI(J)] = rl < rows ? x[(row0 + rl) * CPR + kpos] : make_uint4(0, 0, 0, 0);
      });
      sfor<CPR>([&](auto J) {
        const int rl = (RTQ_CI(J) * 64 + lane) / CPR;
        lds[rl * LROW + kpos] = xor4(v[RTQ_CI(J)], sc.m);
      });
    } else {  // the tile crosses a seed boundary: signs per row
#pragma unroll 1
      for (int j = 0; j < CPR; ++j) {
        const int rl = (j * 64 + lane) / CPR;
        const uint4 q = rl < rows ? x[(row0 + rl) * CPR + kpos] : make_uint4(0, 0, 0, 0);
        lds[rl * LROW + kpos] = xor4(q, chunk_sign_masks(row_seed(seed, row0 + rl, rps, period), kpos));
      }
    }
    lds_sync();
    uint32_t h[D / 2];
    sfor<CPR>([&](auto C) {
      const uint4 q = lds[lane * LROW + RTQ_CI(C)];
      h[4 * RTQ_CI(C) + 0] = q.x;
      h[4 * RTQ_CI(C) + 1] = q.y;
      h[4 * RTQ_CI(C) + 2] = q.z;
      h[4 * RTQ_CI(C) + 3] = q.w;
    });
    lds_sync();
    float z[D];
    float zs;
    if constexpr (ROT == kSRFT) {
      srft_fwd<D>(h, z);
      zs = 1.0f;
    } else {
      fwht_from_f16<D>(h, z);
      zs = (float)(1.0 / csqrt((double)D));
    }
    uint32_t cw[D / 8], sb[D / G];
    quantize_pack<D, G>(z, zs, cw, sb);
    if (lane < rows) {
      const int64_t row = row0 + lane;
      sfor<D / 32>([&](auto C) {
        codes[row * (D / 32) + RTQ_CI(C)] =
            make_uint4(cw[4 * RTQ_CI(C)], cw[4 * RTQ_CI(C) + 1], cw[4 * RTQ_CI(C) + 2], cw[4 * RTQ_CI(C) + 3]);
      });
      if constexpr (D / G == 1) {
        reinterpret_cast<uint16_t*>(scales)[row] = (uint16_t)sb[0];
      } else if constexpr (D / G == 2) {
        reinterpret_cast<uint32_t*>(scales)[row] = sb[0] | (sb[1] << 16);
      } else {
        reinterpret_cast<uint2*>(scales)[row] = make_uint2(sb[0] | (sb[1] << 16), sb[2] | (sb[3] << 16));
      }
    }
  }
}

template <int D, int G, int ROT>
__global__ __launch_bounds__(64) void inv_lane_kernel(const uint4* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, uint4* __restrict__ y,
                                                      int64_t n, uint64_t seed, int64_t rps, int32_t period) {
  constexpr int CPR = D / 8;
  constexpr int LROW = CPR + 1;
  __shared__ uint4 lds[64 * LROW];
  const int lane = threadIdx.x;
  const uint32_t kpos = lane % CPR;
  const int64_t tiles = (n + 63) / 64;
  SignCache sc;
  sc.valid = false;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t row0 = t * 64;
    const int rows = (int)(n - row0 < 64 ? n - row0 : 64);
    const bool uniform = tile_signs(sc, seed, row0, rows, rps, period, kpos);
    uint32_t cw[D / 8], sb[D / G];
    {
      const int64_t row = row0 + (lane < rows ? lane : 0);
      sfor<D / 32>([&](auto C) {
        const uint4 q = codes[row * (D / 32) + RTQ_CI(C)];
        cw[4 * RTQ_CI(C) + 0] = q.x;
        cw[4 * RTQ_CI(C) + 1] = q.y;
        cw[4 * RTQ_CI(C) + 2] = q.z;
        cw[4 * RTQ_CI(C) + 3] = q.w;
      });
      if constexpr (D / G == 1) {
        sb[0] = reinterpret_cast<const uint16_t*>(scales)[row];
      } else if constexpr (D / G == 2) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(scales)[row];
        sb[0] = w & 0xffffu;
        sb[1] = w >> 16;
      } else {
        const uint2 w = reinterpret_cast<const uint2*>(scales)[row];
        sb[0] = w.x & 0xffffu;
        sb[1] = w.x >> 16;
        sb[2] = w.y & 0xffffu;
        sb[3] = w.y >> 16;
      }
    }
    float z[D], u[D];
    if constexpr (ROT == kSRFT) {
      dequant_unpack<D, G>(cw, sb, 1.0f, z);
      srft_inv<D, One>(z, u);
    } else {
      dequant_unpack<D, G>(cw, sb, (float)(1.0 / csqrt((double)D)), u);
      fwht_f32<D>(u);
    }
    // fp16 row into LDS, then coalesced sign flip and store
    sfor<CPR>([&](auto C) {
      constexpr int c = RTQ_CI(C);
      lds[lane * LROW + c] = make_uint4(pack_f16x2(u[8 * c + 0], u[8 * c + 1]), pack_f16x2(u[8 * c + 2], u[8 * c + 3]),
                                        pack_f16x2(u[8 * c + 4], u[8 * c + 5]), pack_f16x2(u[8 * c + 6], u[8 * c + 7]));
    });
    lds_sync();
    if (uniform) {
      sfor<CPR>([&](auto J) {
        const int rl = (RTQ_CI(J) * 64 + lane) / CPR;
        if (rl < rows) y[(row0 + rl) * CPR + kpos] = xor4(lds[rl * LROW + kpos], sc.m);
      });
    } else {
#pragma unroll 1
      for (int j = 0; j < CPR; ++j) {
        const int rl = (j * 64 + lane) / CPR;
        if (rl < rows)
          y[(row0 + rl) * CPR + kpos] =
              xor4(lds[rl * LROW + kpos], chunk_sign_masks(row_seed(seed, row0 + rl, rps, period), kpos));
      }
    }
    lds_sync();
  }
}

// ---------------------------------------------------------------------------
// d = 256: two lanes per vector (lane v and lane v + 32), 32 vectors per tile.
//   SRFT: lane p holds the samples u_{2m+p} (m = 0..127), computes their real
//     DFT of length 128 (E for p = 0, O for p = 1), both lanes exchange E and O
//     (ds_bpermute), and combine X_a = E_a + w^a O_a (lane 0, bins 0..64) and
//     X_{128-a} = conj(E_a - w^a O_a) (lane 1, bins 64..128).  Lane 1 keeps its
//     coordinates mirrored (local index 127 - i) with Re/Im swapped, which
//     makes its register layout identical to lane 0's; the mirror is undone
//     on the packed codes and scales.
//   SRHT: lane p holds the contiguous half p; H_256 = H_2 (x) H_128, so each
//     lane applies H_128 and the halves combine as F0 + F1 / F0 - F1.
// ---------------------------------------------------------------------------

struct Srft256Sub {  // scales of the length-128 sub-DFT bins: X-scaled for d = 256
  static constexpr double s0 = 1.0 / 16.0;
  static constexpr double sm = 0.08838834764831844055010554526311;  // sqrt(2/256)
  static constexpr double si = 0.08838834764831844055010554526311;
};

template <int G, int ROT>
__global__ __launch_bounds__(64) void fwd_pair_kernel(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, int64_t n, uint64_t seed,
                                                      int64_t rps, int32_t period) {
  constexpr int D = 256, CPR = 32, LROW = CPR + 1;
  __shared__ uint4 lds[32 * LROW];
  const int lane = threadIdx.x;
  const int p = lane >> 5, v = lane & 31;
  const uint32_t kpos = lane & 31;
  const float sigma = p ? -1.0f : 1.0f;
  const int64_t tiles = (n + 31) / 32;
  SignCache sc;
  sc.valid = false;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t row0 = t * 32;
    const int rows = (int)(n - row0 < 32 ? n - row0 : 32);
    const bool uniform = tile_signs(sc, seed, row0, rows, rps, period, kpos);
    auto put = [&](int rl, uint4 q) {
      if constexpr (ROT == kSRFT) {
        // de-interleave: evens to the first half of the LDS row, odds to the second
        uint2* row = reinterpret_cast<uint2*>(&lds[rl * LROW]);
        row[kpos] = make_uint2(__builtin_amdgcn_perm(q.y, q.x, 0x05040100u), __builtin_amdgcn_perm(q.w, q.z, 0x05040100u));
        row[32 + kpos] = make_uint2(__builtin_amdgcn_perm(q.y, q.x, 0x07060302u), __builtin_amdgcn_perm(q.w, q.z, 0x07060302u));
      } else {
        lds[rl * LROW + kpos] = q;
      }
    };
    if (uniform) {
      uint4 in[16];
      sfor<16>([&](auto J) {
        const int rl = 2 * RTQ_CI(J) + p;
        in[RTQ_CI(J)] = rl < rows ? x[(row0 + rl) * CPR + kpos] : make_uint4(0, 0, 0, 0);
      });
      sfor<16>([&](auto J) { put(2 * RTQ_CI(J) + p, xor4(in[RTQ_CI(J)], sc.m)); });
    } else {
#pragma unroll 1
      for (int j = 0; j < 16; ++j) {
        const int rl = 2 * j + p;
        const uint4 q = rl < rows ? x[(row0 + rl) * CPR + kpos] : make_uint4(0, 0, 0, 0);
        put(rl, xor4(q, chunk_sign_masks(row_seed(seed, row0 + rl, rps, period), kpos)));
      }
    }
    lds_sync();
    uint32_t h[64];
    sfor<16>([&](auto C) {
      const uint4 q = lds[v * LROW + 16 * p + RTQ_CI(C)];
      h[4 * RTQ_CI(C) + 0] = q.x;
      h[4 * RTQ_CI(C) + 1] = q.y;
      h[4 * RTQ_CI(C) + 2] = q.z;
      h[4 * RTQ_CI(C) + 3] = q.w;
    });
    lds_sync();
    float L[128];
    float zs;
    if constexpr (ROT == kSRFT) {
      float fr[65], fi[65];
      rfft_bins<128, Srft256Sub>(h, fr, fi);
      const int src_e = v, src_o = v + 32;
      // slot 0: E_0 + sigma * O_0 (real)
      {
        const float e0 = __shfl(fr[0], src_e), o0 = __shfl(fr[0], src_o);
        L[0] = __builtin_fmaf(sigma, o0, e0);
      }
      sfor<63>([&](auto A) {
        constexpr int a = RTQ_CI(A) + 1;
        const float er = __shfl(fr[a], src_e), ei = __shfl(fi[a], src_e);
        const float orr = __shfl(fr[a], src_o), oi = __shfl(fi[a], src_o);
        constexpr float c = (float)cos2pi(a, 256), s = (float)sin2pi(a, 256);  // w^a = c - i s
        const float tr = __builtin_fmaf(c, orr, s * oi);
        const float ti = __builtin_fmaf(c, oi, -s * orr);
        const float rr = __builtin_fmaf(sigma, tr, er);
        const float ri = __builtin_fmaf(sigma, ei, ti);
        L[2 * a - 1] = p ? ri : rr;
        L[2 * a] = p ? rr : ri;
      });
      {  // slot 64: X_64 = E_64 - i O_64; lane 0 keeps Re, lane 1 keeps Im
        const float e64 = __shfl(fr[64], src_e), o64 = __shfl(fr[64], src_o);
        L[127] = p ? -o64 : e64;
      }
      zs = 1.0f;
    } else {
      float f[128];
      fwht_from_f16<128>(h, f);
      sfor<128>([&](auto K) {
        const float r = __shfl_xor(f[RTQ_CI(K)], 32);
        L[RTQ_CI(K)] = __builtin_fmaf(sigma, f[RTQ_CI(K)], r);
      });
      zs = 1.0f / 16.0f;
    }
    uint32_t cw[16], sb[128 / G];
    quantize_pack<128, G>(L, zs, cw, sb);
    if constexpr (ROT == kSRFT) {
      // lane 1: codes and scales are in mirrored order -> reverse them
      uint32_t rev[16];
      sfor<16>([&](auto W) { rev[RTQ_CI(W)] = nibble_reverse(cw[15 - RTQ_CI(W)]); });
      sfor<16>([&](auto W) { cw[RTQ_CI(W)] = p ? rev[RTQ_CI(W)] : cw[RTQ_CI(W)]; });
      uint32_t sr[128 / G];
      sfor<128 / G>([&](auto W) { sr[RTQ_CI(W)] = sb[128 / G - 1 - RTQ_CI(W)]; });
      sfor<128 / G>([&](auto W) { sb[RTQ_CI(W)] = p ? sr[RTQ_CI(W)] : sb[RTQ_CI(W)]; });
    }
    if (v < rows) {
      const int64_t row = row0 + v;
      sfor<4>([&](auto C) {
        codes[row * 8 + 4 * p + RTQ_CI(C)] =
            make_uint4(cw[4 * RTQ_CI(C)], cw[4 * RTQ_CI(C) + 1], cw[4 * RTQ_CI(C) + 2], cw[4 * RTQ_CI(C) + 3]);
      });
      // this lane's half of the row's scales: 128/G values
      if constexpr (128 / G == 1) {
        reinterpret_cast<uint16_t*>(scales)[row * 2 + p] = (uint16_t)sb[0];
      } else if constexpr (128 / G == 2) {
        reinterpret_cast<uint32_t*>(scales)[row * 2 + p] = sb[0] | (sb[1] << 16);
      } else {
        reinterpret_cast<uint2*>(scales)[row * 2 + p] = make_uint2(sb[0] | (sb[1] << 16), sb[2] | (sb[3] << 16));
      }
    }
  }
}

template <int G, int ROT>
__global__ __launch_bounds__(64) void inv_pair_kernel(const uint4* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, uint4* __restrict__ y,
                                                      int64_t n, uint64_t seed, int64_t rps, int32_t period) {
  constexpr int CPR = 32, LROW = CPR + 1;
  __shared__ uint4 lds[32 * LROW];
  const int lane = threadIdx.x;
  const int p = lane >> 5, v = lane & 31;
  const uint32_t kpos = lane & 31;
  const float sigma = p ? -1.0f : 1.0f;
  const int64_t tiles = (n + 31) / 32;
  SignCache sc;
  sc.valid = false;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t row0 = t * 32;
    const int rows = (int)(n - row0 < 32 ? n - row0 : 32);
    const bool uniform = tile_signs(sc, seed, row0, rows, rps, period, kpos);
    uint32_t cw[16], sb[128 / G];
    {
      const int64_t row = row0 + (v < rows ? v : 0);
      sfor<4>([&](auto C) {
        const uint4 q = codes[row * 8 + 4 * p + RTQ_CI(C)];
        cw[4 * RTQ_CI(C) + 0] = q.x;
        cw[4 * RTQ_CI(C) + 1] = q.y;
        cw[4 * RTQ_CI(C) + 2] = q.z;
        cw[4 * RTQ_CI(C) + 3] = q.w;
      });
      if constexpr (128 / G == 1) {
        sb[0] = reinterpret_cast<const uint16_t*>(scales)[row * 2 + p];
      } else if constexpr (128 / G == 2) {
        const uint32_t w = reinterpret_cast<const uint32_t*>(scales)[row * 2 + p];
        sb[0] = w & 0xffffu;
        sb[1] = w >> 16;
      } else {
        const uint2 w = reinterpret_cast<const uint2*>(scales)[row * 2 + p];
        sb[0] = w.x & 0xffffu;
        sb[1] = w.x >> 16;
        sb[2] = w.y & 0xffffu;
        sb[3] = w.y >> 16;
      }
    }
    float u[128];
    if constexpr (ROT == kSRFT) {
      // lane 1 holds its half in mirrored order: undo on the packed form
      uint32_t rev[16];
      sfor<16>([&](auto W) { rev[RTQ_CI(W)] = nibble_reverse(cw[15 - RTQ_CI(W)]); });
      sfor<16>([&](auto W) { cw[RTQ_CI(W)] = p ? rev[RTQ_CI(W)] : cw[RTQ_CI(W)]; });
      uint32_t sr[128 / G];
      sfor<128 / G>([&](auto W) { sr[RTQ_CI(W)] = sb[128 / G - 1 - RTQ_CI(W)]; });
      sfor<128 / G>([&](auto W) { sb[RTQ_CI(W)] = p ? sr[RTQ_CI(W)] : sb[RTQ_CI(W)]; });
      float L[128];
      dequant_unpack<128, G>(cw, sb, 1.0f, L);
      // P = lane v's slots (X_a), Q = lane v+32's slots (X_{128-a}, Re/Im swapped)
      const int src0 = v, src1 = v + 32;
      float yv[128];
      {
        const float p0 = __shfl(L[0], src0), q0 = __shfl(L[0], src1);
        yv[0] = 0.5f * __builtin_fmaf(sigma, q0, p0);
      }
      sfor<63>([&](auto A) {
        constexpr int a = RTQ_CI(A) + 1;
        const float pr = __shfl(L[2 * a - 1], src0), pi = __shfl(L[2 * a], src0);
        const float qr = __shfl(L[2 * a], src1), qi = __shfl(L[2 * a - 1], src1);
        const float fr = 0.5f * __builtin_fmaf(sigma, qr, pr);  // E (lane 0) or t (lane 1)
        const float fi = 0.5f * __builtin_fmaf(-sigma, qi, pi);
        // lane 1: O_a = w^-a t_a with w^-a = c + i s; lane 0 multiplies by 1
        constexpr float c = (float)cos2pi(a, 256), s = (float)sin2pi(a, 256);
        const float cc = p ? c : 1.0f, ss = p ? s : 0.0f;
        yv[2 * a - 1] = __builtin_fmaf(cc, fr, -ss * fi);
        yv[2 * a] = __builtin_fmaf(cc, fi, ss * fr);
      });
      {
        const float p64 = __shfl(L[127], src0), q64 = __shfl(L[127], src1);
        constexpr float r2 = 0.70710678118654752440f;
        yv[127] = (p ? -q64 : p64) * r2;
      }
      srft_inv<128, Sqrt2>(yv, u);
    } else {
      float f[128];
      dequant_unpack<128, G>(cw, sb, 1.0f / 16.0f, f);
      fwht_f32<128>(f);
      sfor<128>([&](auto K) {
        const float r = __shfl_xor(f[RTQ_CI(K)], 32);
        u[RTQ_CI(K)] = __builtin_fmaf(sigma, f[RTQ_CI(K)], r);
      });
    }
    // fp16 samples into LDS (SRFT: lane p's samples are u_{2m+p}; they go to
    // the p-th half of the row and are re-interleaved on the way out)
    sfor<16>([&](auto C) {
      constexpr int c = RTQ_CI(C);
      lds[v * LROW + 16 * p + c] = make_uint4(pack_f16x2(u[8 * c + 0], u[8 * c + 1]), pack_f16x2(u[8 * c + 2], u[8 * c + 3]),
                                              pack_f16x2(u[8 * c + 4], u[8 * c + 5]), pack_f16x2(u[8 * c + 6], u[8 * c + 7]));
    });
    lds_sync();
    auto get = [&](int rl) -> uint4 {
      if constexpr (ROT == kSRFT) {
        const uint2* row = reinterpret_cast<const uint2*>(&lds[rl * LROW]);
        const uint2 e = row[kpos], o = row[32 + kpos];
        return make_uint4(__builtin_amdgcn_perm(o.x, e.x, 0x05040100u), __builtin_amdgcn_perm(o.x, e.x, 0x07060302u),
                          __builtin_amdgcn_perm(o.y, e.y, 0x05040100u), __builtin_amdgcn_perm(o.y, e.y, 0x07060302u));
      } else {
        return lds[rl * LROW + kpos];
      }
    };
    if (uniform) {
      sfor<16>([&](auto J) {
        const int rl = 2 * RTQ_CI(J) + p;
        if (rl < rows) y[(row0 + rl) * CPR + kpos] = xor4(get(rl), sc.m);
      });
    } else {
#pragma unroll 1
      for (int j = 0; j < 16; ++j) {
        const int rl = 2 * j + p;
        if (rl < rows)
          y[(row0 + rl) * CPR + kpos] = xor4(get(rl), chunk_sign_masks(row_seed(seed, row0 + rl, rps, period), kpos));
      }
    }
    lds_sync();
  }
}

// ---------------------------------------------------------------------------
// Host side: validation, launch configuration, dispatch.
// ---------------------------------------------------------------------------

struct Args {
  const void* in0;
  const void* in1;  // scales for the inverse, unused for the forward
  void* out0;
  void* out1;       // scales for the forward, unused for the inverse
  int64_t n;
  uint64_t seed;
  int64_t rps;
  int32_t period;
  hipStream_t stream;
};

using KernelFn = const void*;

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> g(mu);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = cus;
  }
  return cache[dev];
}

// Resident waves per CU for a kernel: occupancy query, cached per (kernel, device).
int blocks_per_cu(KernelFn fn) {
  static std::mutex mu;
  struct Entry { KernelFn fn; int dev; int blocks; };
  static Entry cache[256];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < used; ++i)
      if (cache[i].fn == fn && cache[i].dev == dev) return cache[i].blocks;
  }
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, 64, 0) != hipSuccess || blocks <= 0) blocks = 4;
  std::lock_guard<std::mutex> g(mu);
  if (used < 256) cache[used++] = Entry{fn, dev, blocks};
  return blocks;
}

rtq_status launch(KernelFn fn, int64_t tiles, void** kargs, hipStream_t stream) {
  const int cus = device_cu_count();
  if (cus <= 0) return RTQ_ERR_HIP;
  const int64_t resident = (int64_t)cus * blocks_per_cu(fn);
  const int64_t grid = tiles < resident ? tiles : resident;
  const hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(64), kargs, 0, stream);
  return e == hipSuccess ? RTQ_OK : RTQ_ERR_HIP;
}

template <int D, int G, int ROT>
KernelFn pick_fwd() {
  if constexpr (D == 256) return reinterpret_cast<KernelFn>(&fwd_pair_kernel<G, ROT>);
  else return reinterpret_cast<KernelFn>(&fwd_lane_kernel<D, G, ROT>);
}
template <int D, int G, int ROT>
KernelFn pick_inv() {
  if constexpr (D == 256) return reinterpret_cast<KernelFn>(&inv_pair_kernel<G, ROT>);
  else return reinterpret_cast<KernelFn>(&inv_lane_kernel<D, G, ROT>);
}

template <int ROT>
KernelFn find_kernel(bool fwd, int d, int g) {
#define RTQ_CASE(DD, GG) \
  if (d == DD && g == GG) return fwd ? pick_fwd<DD, GG, ROT>() : pick_inv<DD, GG, ROT>();
  RTQ_CASE(64, 32) RTQ_CASE(64, 64)
  RTQ_CASE(128, 32) RTQ_CASE(128, 64) RTQ_CASE(128, 128)
  RTQ_CASE(256, 32) RTQ_CASE(256, 64) RTQ_CASE(256, 128)
#undef RTQ_CASE
  return nullptr;
}

bool ranges_overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Supported (d, group): d in {64,128,256}; group in {32,64,128,256}, group <= d.
// (d = 256, group = 256) is a per-token scale over two lanes and is not built.
rtq_status check_shape(int32_t d, int32_t g) {
  if (d != 64 && d != 128 && d != 256) return RTQ_ERR_UNSUPPORTED;
  if (g != 32 && g != 64 && g != 128 && g != 256) return RTQ_ERR_UNSUPPORTED;
  if (g > d) return RTQ_ERR_UNSUPPORTED;
  if (d == 256 && g == 256) return RTQ_ERR_UNSUPPORTED;
  return RTQ_OK;
}

rtq_status run(bool fwd, int rot, const void* in0, const void* in1, void* out0, void* out1, int64_t n, int32_t d,
               int32_t g, uint64_t seed, int64_t rps, int32_t period, hipStream_t stream) {
  if (n < 0 || rps < 0 || period < 0) return RTQ_ERR_INVALID_ARG;
  const rtq_status shape = check_shape(d, g);
  if (shape != RTQ_OK) return shape;
  if (n == 0) return RTQ_OK;
  if (n > (INT64_MAX / 4) / d) return RTQ_ERR_INVALID_ARG;
  const int64_t fp16_bytes = n * 2 * d, code_bytes = n * (d / 2), scale_bytes = n * 2 * (d / g);
  if (fwd) {
    // in0 = x, out0 = codes, out1 = scales
    if (!in0 || !out0 || !out1) return RTQ_ERR_INVALID_ARG;
    if (!aligned16(in0) || !aligned16(out0) || !aligned16(out1)) return RTQ_ERR_INVALID_ARG;
    if (ranges_overlap(in0, fp16_bytes, out0, code_bytes) || ranges_overlap(in0, fp16_bytes, out1, scale_bytes) ||
        ranges_overlap(out0, code_bytes, out1, scale_bytes))
      return RTQ_ERR_INVALID_ARG;
  } else {
    // in0 = codes, in1 = scales, out0 = y
    if (!in0 || !in1 || !out0) return RTQ_ERR_INVALID_ARG;
    if (!aligned16(in0) || !aligned16(in1) || !aligned16(out0)) return RTQ_ERR_INVALID_ARG;
    if (ranges_overlap(out0, fp16_bytes, in0, code_bytes) || ranges_overlap(out0, fp16_bytes, in1, scale_bytes))
      return RTQ_ERR_INVALID_ARG;
  }
  const KernelFn fn = rot == kSRFT ? find_kernel<kSRFT>(fwd, d, g) : find_kernel<kSRHT>(fwd, d, g);
  if (!fn) return RTQ_ERR_UNSUPPORTED;
  const int vpt = d == 256 ? 32 : 64;
  const int64_t tiles = (n + vpt - 1) / vpt;
  if (fwd) {
    const void* x = in0;
    void* codes = out0;
    void* scales = out1;
    void* kargs[] = {&x, &codes, &scales, &n, &seed, &rps, &period};
    return launch(fn, tiles, kargs, stream);
  }
  const void* codes = in0;
  const void* scales = in1;
  void* y = out0;
  void* kargs[] = {&codes, &scales, &y, &n, &seed, &rps, &period};
  return launch(fn, tiles, kargs, stream);
}

}  // namespace rtq

#define RTQ_API extern "C" __attribute__((visibility("default")))

RTQ_API rtq_status srft_quant_fwd(const void* x_f16, void* codes_u8, void* scales_f16, int64_t n, int32_t d,
                                  int32_t group, uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                  hipStream_t stream) {
  return rtq::run(true, rtq::kSRFT, x_f16, nullptr, codes_u8, scales_f16, n, d, group, seed, rows_per_seed,
                  seed_period, stream);
}

RTQ_API rtq_status srft_dequant_inv(const void* codes_u8, const void* scales_f16, void* y_f16, int64_t n, int32_t d,
                                    int32_t group, uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                    hipStream_t stream) {
  return rtq::run(false, rtq::kSRFT, codes_u8, scales_f16, y_f16, nullptr, n, d, group, seed, rows_per_seed,
                  seed_period, stream);
}

RTQ_API rtq_status srht_quant_fwd(const void* x_f16, void* codes_u8, void* scales_f16, int64_t n, int32_t d,
                                  int32_t group, uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                  hipStream_t stream) {
  return rtq::run(true, rtq::kSRHT, x_f16, nullptr, codes_u8, scales_f16, n, d, group, seed, rows_per_seed,
                  seed_period, stream);
}

RTQ_API rtq_status srht_dequant_inv(const void* codes_u8, const void* scales_f16, void* y_f16, int64_t n, int32_t d,
                                    int32_t group, uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                    hipStream_t stream) {
  return rtq::run(false, rtq::kSRHT, codes_u8, scales_f16, y_f16, nullptr, n, d, group, seed, rows_per_seed,
                  seed_period, stream);
}

RTQ_API const char* rtq_status_string(rtq_status status) {
  switch (status) {
    case RTQ_OK: return "RTQ_OK: success";
    case RTQ_ERR_INVALID_ARG:
      return "RTQ_ERR_INVALID_ARG: null or misaligned pointer, negative size, or overlapping buffers";
    case RTQ_ERR_UNSUPPORTED: return "RTQ_ERR_UNSUPPORTED: (d, group) is not supported";
    case RTQ_ERR_HIP: return "RTQ_ERR_HIP: the HIP runtime reported an error";
  }
  return "rtq: unknown status";
}
