// rtq_pair.hpp -- d = 256 tiles of the fused rotate-then-quantize kernels
// (MI355X, gfx950): two lanes per vector (lane v and lane v + 32), 32
// vectors per tile.  The tiles are written once and used by the plain
// entry points (rows of a contiguous [n, 256] tensor) and by the cache-layout
// entry points (rows placed by strides), through a row policy:
//
//   struct Rows {
//     uint32_t row0;  // first row of the tile in the input numbering
//     int rows;       // rows in the tile (1 .. 32)
//     bool uniform;   // every row of the tile has the same sign seed
//     static constexpr bool kStreamStores;  // non-temporal scale / output stores (streaming tiles)
//     uint4 uniform_masks(uint32_t k) const;      // sign masks of chunk k, the tile's seed
//     uint4 row_masks(int rl, uint32_t k) const;  // sign masks of chunk k, row rl's seed
//     size_t cache_row(int rl) const;             // codes / scales row of tile row rl
//     uint4* y_chunk(uint4* y, int rl, uint32_t k) const;  // 16-byte chunk k of row rl of y
//   };
//
//   SRFT: lane p holds the samples u_{2m+p} (m = 0..127), computes their real
//     DFT of length 128 (E for p = 0, O for p = 1), both lanes exchange E and O
//     (ds_bpermute), and combine X_a = E_a + w^a O_a (lane 0, bins 0..64) and
//     X_{128-a} = conj(E_a - w^a O_a) (lane 1, bins 64..128).  Lane 1 keeps its
//     coordinates mirrored (local index 127 - i) with Re/Im swapped, which
//     makes its register layout identical to lane 0's; the mirror is undone
//     on the packed codes and scales.
//   SRHT: lane p holds the contiguous half p; H_256 = H_2 (x) H_128, so each
//     lane applies H_128 and the halves combine as F0 + F1 / F0 - F1.
//
// Method: "Quantization Speed Is Often a Kernel Problem", "First, the 17%"
// and "Fusing four steps into two kernels is not enough" (rotate + quantize
// in one kernel, dequantize + inverse-rotate in the other).
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "rtq_device.hpp"
#include "rtq_div.hpp"
#include "rtq_lane.hpp"
#include "rtq_mem.hpp"

namespace rtq {

// The unnormalized real-DFT bins (scale 1 on every bin), for rfft_bins.
struct UnitBins {
  static constexpr double s0 = 1.0, sm = 1.0, si = 1.0;
};

// u = lambda (.) (the lane's 128 samples), exact in fp32.  SRFT: lane p holds
// the samples 2m + p, h[k] = (sample 4k + p, sample 4k + 2 + p), whose
// weights are half p of lambda words 2k and 2k + 1.  SRHT: lane p holds
// samples 128 p + m, h[k] = (128 p + 2k, 128 p + 2k + 1) = lambda word 64 p + k.
template <int ROT>
__device__ __forceinline__ void lambda_half(const uint32_t (&h)[64], const uint32_t* __restrict__ lam, int p,
                                            float (&u)[128]) {
  if constexpr (ROT == kSRFT) {
    const uint32_t sh = 16u * (uint32_t)p;
    sfor<64>([&](auto K) {
      constexpr int k = RTQ_CI(K);
      u[2 * k] = lo_f(h[k]) * lo_f(lam[2 * k] >> sh);
      u[2 * k + 1] = hi_f(h[k]) * lo_f(lam[2 * k + 1] >> sh);
    });
  } else {
    const uint32_t* lp = lam + 64 * p;
    sfor<64>([&](auto K) {
      constexpr int k = RTQ_CI(K);
      const uint32_t l = lp[k];
      u[2 * k] = lo_f(h[k]) * lo_f(l);
      u[2 * k + 1] = hi_f(h[k]) * hi_f(l);
    });
  }
}

// 1/lambda of the 128 samples each half of the pair holds, as inv[p * 132 + m]
// for half p and its sample m (SRFT: channel 2m + p, SRHT: 128p + m); rows
// are padded to 132 floats so that the two halves read different banks.
// One reciprocal per lane and 64 channels per tile, instead of one per value
// (lambda is the same for every row).
template <int ROT>
__device__ __forceinline__ void pair_lambda_reciprocals(const uint32_t* __restrict__ lam, float* inv, int lane) {
  sfor<4>([&](auto I) {
    const int idx = RTQ_CI(I) * 64 + lane, p = idx >> 7, m = idx & 127;
    const int ch = ROT == kSRFT ? 2 * m + p : 128 * p + m;
    const uint32_t l = lam[ch >> 1];
    inv[p * 132 + m] = __builtin_amdgcn_rcpf((ch & 1) ? hi_f(l) : lo_f(l));
  });
}
constexpr int kPairLambdaFloats = 2 * 132;

// u /= lambda for the lane's 128 output samples (u[m] is sample m of half p),
// from the reciprocal table, read as broadcasts.
__device__ __forceinline__ void unweight_half(float (&u)[128], const float* inv, int p) {
  const float* r = inv + p * 132;
  sfor<32>([&](auto J) {
    constexpr int j = RTQ_CI(J);
    const float4 q = *reinterpret_cast<const float4*>(r + 4 * j);
    u[4 * j] *= q.x;
    u[4 * j + 1] *= q.y;
    u[4 * j + 2] *= q.z;
    u[4 * j + 3] *= q.w;
  });
}

// Non-temporal store for streaming tiles, ordinary (L2-merged) store for rows
// scattered by a cache layout.
template <bool NT, class T>
__device__ __forceinline__ void put_store(T* p, T v) {
  if constexpr (NT) stream_store(p, v);
  else *p = v;
}

// Forward tile: rows R.row0 .. R.row0 + R.rows - 1 of x (contiguous, 32
// 16-byte chunks per row) into the codes / scales rows R.cache_row(.), with
// B-bit codes (one little-endian bit stream per row, 32 B bytes) and an
// optional per-channel lambda.  lds holds 32 x 33 uint4.
template <int G, int ROT, class Rows, int B = 4>
__device__ __forceinline__ void fwd_pair_tile(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                              uint8_t* __restrict__ scales, const Rows& R, uint4* lds, int lane,
                                              const uint32_t* __restrict__ lam = nullptr) {
  constexpr int D = 256, CPR = 32, LROW = CPR + 1;
  const int p = lane >> 5, v = lane & 31;
  const uint32_t kpos = lane & 31;
  const float sigma = p ? -1.0f : 1.0f;
  {
    const uint32_t row0 = R.row0;
    const int rows = R.rows;
    const bool uniform = R.uniform;
    uint4 cm = make_uint4(0, 0, 0, 0);
    if (uniform) cm = R.uniform_masks(kpos);
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
      const uint4* xt = x + (size_t)row0 * CPR;
      uint4 in[16];
      sfor<16>([&](auto J) {
        const int rl = 2 * RTQ_CI(J) + p;
        in[RTQ_CI(J)] = rl < rows ? stream_load(xt + ((uint32_t)(rl * CPR) + kpos)) : make_uint4(0, 0, 0, 0);
      });
      sfor<16>([&](auto J) { put(2 * RTQ_CI(J) + p, xor4(in[RTQ_CI(J)], cm)); });
    } else {
#pragma unroll 1
      for (int j = 0; j < 16; ++j) {
        const int rl = 2 * j + p;
        const uint4 q = rl < rows ? stream_load(x + ((size_t)(row0 + rl) * CPR + kpos)) : make_uint4(0, 0, 0, 0);
        put(rl, xor4(q, R.row_masks(rl, kpos)));
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
    wait_lds_reads();
    lds_sync();
    float L[128];
    float zs;
    constexpr int CWW = 4 * B;  // code words of the lane's half row
    uint32_t cw[CWW], sb[128 / G];
    if constexpr (ROT == kSRFT) {
      float fr[65], fi[65];  // unnormalized; sqrt(2/256) is applied by the quantizer
      if (lam != nullptr) {
        float uw[128];
        lambda_half<kSRFT>(h, lam, p, uw);
        rfft_bins<128, UnitBins>(uw, fr, fi);
      } else {
        rdft<128, 1, 0, 64>(h, fr, fi);
      }
      // Partner exchange by ds_bpermute.  Every 4 bins the next addresses are
      // tied to the last result, so each group of shuffles issues only once
      // the previous group has been consumed; this keeps the exchange from
      // holding all 260 shuffled values at once (register pressure).
      int addr_e = v * 4, addr_o = (v + 32) * 4;
      auto shf = [](float x, int addr) { return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(x))); };
      // slot 0: E_0 + sigma * O_0 (real)
      auto bin0 = [&]() {
        const float e0 = shf(fr[0], addr_e), o0 = shf(fr[0], addr_o);
        constexpr float r2 = 0.70710678118654752440f;  // real end bins: 1/16 = sqrt(2/256) / sqrt(2)
        L[0] = __builtin_fmaf(sigma, o0, e0) * r2;
      };
      // bin a = 1 .. 63: slots 2a - 1 and 2a
      auto bin = [&](auto A) {
        constexpr int a = RTQ_CI(A);
        const float er = shf(fr[a], addr_e), ei = shf(fi[a], addr_e);
        const float orr = shf(fr[a], addr_o), oi = shf(fi[a], addr_o);
        constexpr float c = (float)cos2pi(a, 256), s = (float)sin2pi(a, 256);  // w^a = c - i s
        const float tr = __builtin_fmaf(c, orr, s * oi);
        const float ti = __builtin_fmaf(c, oi, -s * orr);
        const float rr = __builtin_fmaf(sigma, tr, er);
        const float ri = __builtin_fmaf(sigma, ei, ti);
        L[2 * a - 1] = p ? ri : rr;
        L[2 * a] = p ? rr : ri;
        if constexpr (a % 4 == 0) asm volatile("" : "+v"(addr_e), "+v"(addr_o) : "v"(L[2 * a]));
      };
      // slot 127: X_64 = E_64 - i O_64; lane 0 keeps Re, lane 1 keeps Im
      auto bin64 = [&]() {
        const float e64 = shf(fr[64], addr_e), o64 = shf(fr[64], addr_o);
        L[127] = p ? -o64 : e64;
      };
      // later shuffles wait for w
      auto after = [&](uint32_t w) { asm volatile("" : "+v"(addr_e), "+v"(addr_o) : "v"(w)); };
      zs = SrftScale<256>::value;
      if constexpr (B == 4) {
        // Quantize each group as soon as the bins that fill it are exchanged:
        // the finished coordinates of at most one group are then live, not
        // all 128 (they had been spilled at three waves per SIMD).  Group gi
        // holds slots gi*G .. gi*G+G-1; bin a fills slots 2a-1 and 2a.
        sfor<128 / G>([&](auto GI) {
          constexpr int gi = RTQ_CI(GI), lo = gi * G, hi = lo + G - 1;
          constexpr int a0 = lo / 2 + 1, a1 = (hi + 1) / 2 < 63 ? (hi + 1) / 2 : 63;
          if constexpr (gi == 0) bin0();
          sfor<a1 - a0 + 1>([&](auto K) { bin(ic<a0 + RTQ_CI(K)>{}); });
          if constexpr (hi == 127) bin64();
          quantize_pack_group<gi, 128, G>(L, zs, cw, sb);
          // the next group's shuffles wait for this group's codes (else the
          // compiler sinks every group's quantization below all shuffles)
          if constexpr (hi < 127) after(cw[(lo + G) / 8 - 1]);
        });
      } else {
        bin0();
        sfor<63>([&](auto A) { bin(ic<RTQ_CI(A) + 1>{}); });
        bin64();
      }
    } else {
      float f[128];
      if (lam != nullptr) {
        lambda_half<kSRHT>(h, lam, p, f);
        fwht_f32<128>(f);
      } else {
        fwht_from_f16<128>(h, f);
      }
      zs = 1.0f / 16.0f;
      auto combine = [&](auto K) {
        const float r = __shfl_xor(f[RTQ_CI(K)], 32);
        L[RTQ_CI(K)] = __builtin_fmaf(sigma, f[RTQ_CI(K)], r);
      };
      // a shuffle of x waits for w
      auto after = [](float& x, uint32_t w) { asm volatile("" : "+v"(x) : "v"(w)); };
      if constexpr (B == 4) {
        // group by group, as for the SRFT: quantize each group once its
        // values are combined; the next group's shuffles wait for its codes
        sfor<128 / G>([&](auto GI) {
          constexpr int gi = RTQ_CI(GI), lo = gi * G;
          sfor<G>([&](auto K) { combine(ic<lo + RTQ_CI(K)>{}); });
          quantize_pack_group<gi, 128, G>(L, zs, cw, sb);
          if constexpr (lo + G < 128) after(f[lo + G], cw[(lo + G) / 8 - 1]);
        });
      } else {
        sfor<128>([&](auto K) { combine(K); });
      }
    }
    if constexpr (B != 4) {
      // SRFT lane 1 holds its half mirrored: put it in natural order first
      // (a b-bit stream has no cheap field reversal), then quantize
      if constexpr (ROT == kSRFT) {
        float Ln[128];
        sfor<128>([&](auto I) { Ln[RTQ_CI(I)] = p ? L[127 - RTQ_CI(I)] : L[RTQ_CI(I)]; });
        quantize_pack_bits<128, G, B>(Ln, zs, cw, sb);
      } else {
        quantize_pack_bits<128, G, B>(L, zs, cw, sb);
      }
    } else if constexpr (ROT == kSRFT) {
      // (quantized above) lane 1: codes and scales are in mirrored order -> reverse them
      uint32_t rev[16];
      sfor<16>([&](auto W) { rev[RTQ_CI(W)] = nibble_reverse(cw[15 - RTQ_CI(W)]); });
      sfor<16>([&](auto W) { cw[RTQ_CI(W)] = p ? rev[RTQ_CI(W)] : cw[RTQ_CI(W)]; });
      uint32_t sr[128 / G];
      sfor<128 / G>([&](auto W) { sr[RTQ_CI(W)] = sb[128 / G - 1 - RTQ_CI(W)]; });
      sfor<128 / G>([&](auto W) { sb[RTQ_CI(W)] = p ? sr[RTQ_CI(W)] : sb[RTQ_CI(W)]; });
    }  // SRHT, 4 bits: quantized above
    if (v < rows) {
      const size_t row = R.cache_row(v);
      constexpr bool nt = Rows::kStreamStores;
      // Each lane writes its half row in 16-byte pieces, so one store
      // instruction leaves one or two pieces in each 128-byte line: ordinary
      // stores let L2 merge them into full lines.  (With the non-temporal
      // hint 8-bit codes ran 2.2x slower, and int4 codes 1-2% slower.)
      sfor<B>([&](auto C) {
        put_store<false>(codes + (row * (2 * B) + B * p + RTQ_CI(C)),
                     make_uint4(cw[4 * RTQ_CI(C)], cw[4 * RTQ_CI(C) + 1], cw[4 * RTQ_CI(C) + 2], cw[4 * RTQ_CI(C) + 3]));
      });
      // this lane's half of the row's scales: 128/G values
      if constexpr (128 / G == 1) {
        put_store<nt>(reinterpret_cast<uint16_t*>(scales) + (row * 2 + p), (uint16_t)sb[0]);
      } else if constexpr (128 / G == 2) {
        put_store<nt>(reinterpret_cast<uint32_t*>(scales) + (row * 2 + p), sb[0] | (sb[1] << 16));
      } else {
        put_store<nt>(reinterpret_cast<uint2*>(scales) + (row * 2 + p), make_uint2(sb[0] | (sb[1] << 16), sb[2] | (sb[3] << 16)));
      }
    }
  }
}

// Inverse tile: the codes / scales rows R.cache_row(.) into the rows of y
// that R.y_chunk addresses, for B-bit codes and an optional lambda.  lds
// holds 32 x 17 uint4.
template <int G, int ROT, class Rows, int B = 4>
__device__ __forceinline__ void inv_pair_tile(const uint4* __restrict__ codes, const uint8_t* __restrict__ scales,
                                              uint4* __restrict__ y, const Rows& R, uint4* lds, int lane,
                                              const uint32_t* __restrict__ lam = nullptr, float* inv_lam = nullptr) {
  constexpr int CPR = 32;
  if (lam != nullptr) pair_lambda_reciprocals<ROT>(lam, inv_lam, lane);  // read after a barrier below
  const int p = lane >> 5, v = lane & 31;
  const uint32_t kpos = lane & 31;
  const float sigma = p ? -1.0f : 1.0f;
  {
    const int rows = R.rows;
    const bool uniform = R.uniform;
    uint32_t cw[4 * B], sb[128 / G];
    {
      const size_t row = R.cache_row(v < rows ? v : 0);
      sfor<B>([&](auto C) {
        const uint4 q = stream_load(codes + (row * (2 * B) + B * p + RTQ_CI(C)));
        cw[4 * RTQ_CI(C) + 0] = q.x;
        cw[4 * RTQ_CI(C) + 1] = q.y;
        cw[4 * RTQ_CI(C) + 2] = q.z;
        cw[4 * RTQ_CI(C) + 3] = q.w;
      });
      if constexpr (128 / G == 1) {
        sb[0] = stream_load(reinterpret_cast<const uint16_t*>(scales) + (row * 2 + p));
      } else if constexpr (128 / G == 2) {
        const uint32_t w = stream_load(reinterpret_cast<const uint32_t*>(scales) + (row * 2 + p));
        sb[0] = w & 0xffffu;
        sb[1] = w >> 16;
      } else {
        const uint2 w = stream_load(reinterpret_cast<const uint2*>(scales) + (row * 2 + p));
        sb[0] = w.x & 0xffffu;
        sb[1] = w.x >> 16;
        sb[2] = w.y & 0xffffu;
        sb[3] = w.y >> 16;
      }
    }
    float u[128];
    if constexpr (ROT == kSRFT) {
      // lane 1 keeps its half in mirrored order (the halving of E and t is
      // folded into the dequantization)
      float L[128];
      if constexpr (B == 4) {  // undo the mirror on the packed form
        uint32_t rev[16];
        sfor<16>([&](auto W) { rev[RTQ_CI(W)] = nibble_reverse(cw[15 - RTQ_CI(W)]); });
        sfor<16>([&](auto W) { cw[RTQ_CI(W)] = p ? rev[RTQ_CI(W)] : cw[RTQ_CI(W)]; });
        uint32_t sr[128 / G];
        sfor<128 / G>([&](auto W) { sr[RTQ_CI(W)] = sb[128 / G - 1 - RTQ_CI(W)]; });
        sfor<128 / G>([&](auto W) { sb[RTQ_CI(W)] = p ? sr[RTQ_CI(W)] : sb[RTQ_CI(W)]; });
        dequant_unpack<128, G>(cw, sb, 0.5f, L);
      } else {  // dequantize in natural order, then mirror the values
        float Ln[128];
        dequant_unpack_bits<128, G, B>(cw, sb, 0.5f, Ln);
        sfor<128>([&](auto I) { L[RTQ_CI(I)] = p ? Ln[127 - RTQ_CI(I)] : Ln[RTQ_CI(I)]; });
      }
      // P = lane v's slots (X_a), Q = lane v+32's slots (X_{128-a}, Re/Im swapped)
      const int src0 = v, src1 = v + 32;
      float yv[128];
      {
        const float p0 = __shfl(L[0], src0), q0 = __shfl(L[0], src1);
        yv[0] = __builtin_fmaf(sigma, q0, p0);
      }
      sfor<63>([&](auto A) {
        constexpr int a = RTQ_CI(A) + 1;
        const float pr = __shfl(L[2 * a - 1], src0), pi = __shfl(L[2 * a], src0);
        const float qr = __shfl(L[2 * a], src1), qi = __shfl(L[2 * a - 1], src1);
        const float fr = __builtin_fmaf(sigma, qr, pr);  // E (lane 0) or t (lane 1)
        const float fi = __builtin_fmaf(-sigma, qi, pi);
        // lane 1: O_a = w^-a t_a with w^-a = c + i s; lane 0 multiplies by 1
        constexpr float c = (float)cos2pi(a, 256), s = (float)sin2pi(a, 256);
        const float cc = p ? c : 1.0f, ss = p ? s : 0.0f;
        yv[2 * a - 1] = __builtin_fmaf(cc, fr, -ss * fi);
        yv[2 * a] = __builtin_fmaf(cc, fi, ss * fr);
      });
      {
        const float p64 = __shfl(L[127], src0), q64 = __shfl(L[127], src1);
        constexpr float sq2 = 1.41421356237309504880f;  // 2 / sqrt(2): L is halved
        yv[127] = (p ? -q64 : p64) * sq2;
      }
      srft_inv<128, Sqrt2>(yv, u);
    } else {
      float f[128];
      if constexpr (B == 4) dequant_unpack<128, G>(cw, sb, 1.0f / 16.0f, f);
      else dequant_unpack_bits<128, G, B>(cw, sb, 1.0f / 16.0f, f);
      fwht_f32<128>(f);
      sfor<128>([&](auto K) {
        const float r = __shfl_xor(f[RTQ_CI(K)], 32);
        u[RTQ_CI(K)] = __builtin_fmaf(sigma, f[RTQ_CI(K)], r);
      });
    }
    if (lam != nullptr) {
      lds_sync();
      unweight_half(u, inv_lam, p);
    }
    // fp16 samples out through LDS in two passes of 16 output chunks per row
    // (a 9 KB tile).  SRFT: lane p's samples are u_{2m+p}; pass ph takes its
    // 64 samples 64 ph .. 64 ph + 63 into the p-th half of the LDS row and
    // re-interleaves them on the way out.  SRHT: lane p holds output chunks
    // 16 p .. 16 p + 15, written in pass p.
    constexpr int LR2 = 17;
    const int kk = lane & 15, rsub = lane >> 4;
    sfor<2>([&](auto PH) {
      constexpr int ph = RTQ_CI(PH);
      if constexpr (ph > 0) {
        wait_lds_reads();
        lds_sync();
      }
      if constexpr (ROT == kSRFT) {
        sfor<8>([&](auto C) {
          constexpr int c = 8 * ph + RTQ_CI(C);
          lds[v * LR2 + 8 * p + RTQ_CI(C)] =
              make_uint4(pack_f16x2(u[8 * c + 0], u[8 * c + 1]), pack_f16x2(u[8 * c + 2], u[8 * c + 3]),
                         pack_f16x2(u[8 * c + 4], u[8 * c + 5]), pack_f16x2(u[8 * c + 6], u[8 * c + 7]));
        });
      } else {
        if (p == ph) {
          sfor<16>([&](auto C) {
            constexpr int c = RTQ_CI(C);
            lds[v * LR2 + c] =
                make_uint4(pack_f16x2(u[8 * c + 0], u[8 * c + 1]), pack_f16x2(u[8 * c + 2], u[8 * c + 3]),
                           pack_f16x2(u[8 * c + 4], u[8 * c + 5]), pack_f16x2(u[8 * c + 6], u[8 * c + 7]));
          });
        }
      }
      lds_sync();
      const uint32_t k = 16u * ph + (uint32_t)kk;  // output chunk this lane stores
      auto get = [&](int rl) -> uint4 {
        if constexpr (ROT == kSRFT) {
          const uint2* row = reinterpret_cast<const uint2*>(&lds[rl * LR2]);
          const uint2 e = row[kk], o = row[16 + kk];
          return make_uint4(__builtin_amdgcn_perm(o.x, e.x, 0x05040100u), __builtin_amdgcn_perm(o.x, e.x, 0x07060302u),
                            __builtin_amdgcn_perm(o.y, e.y, 0x05040100u), __builtin_amdgcn_perm(o.y, e.y, 0x07060302u));
        } else {
          return lds[rl * LR2 + kk];
        }
      };
      if (uniform) {
        const uint4 m = R.uniform_masks(k);
        sfor<8>([&](auto J) {
          const int rl = rsub + 4 * RTQ_CI(J);
          if (rl < rows) put_store<Rows::kStreamStores>(R.y_chunk(y, rl, k), xor4(get(rl), m));
        });
      } else {
#pragma unroll 1
        for (int j = 0; j < 8; ++j) {
          const int rl = rsub + 4 * j;
          if (rl < rows)
            put_store<Rows::kStreamStores>(R.y_chunk(y, rl, k), xor4(get(rl), R.row_masks(rl, k)));
        }
      }
    });
    wait_lds_reads();
    lds_sync();
  }
}

// Row policy of the plain entry points: tile rows row0 .. row0 + rows - 1 of
// a contiguous [n, 256] tensor, under the call's seed rule.
struct TileRows {
  uint32_t row0;
  int rows;
  bool uniform;
  uint32_t b0;  // seed block of row0
  const SeedRule& sr;
  const SignTable& tb;
  static constexpr bool kStreamStores = true;
  __device__ uint4 uniform_masks(uint32_t k) const { return chunk_masks(tb, seed_offset(b0, sr), sr.seed, k); }
  __device__ uint4 row_masks(int rl, uint32_t k) const {
    return chunk_sign_masks(seed_of_block(seed_block(row0 + (uint32_t)rl, sr), sr), k);
  }
  __device__ size_t cache_row(int rl) const { return (size_t)row0 + (uint32_t)rl; }
  __device__ uint4* y_chunk(uint4* y, int rl, uint32_t k) const {
    return y + (size_t)row0 * 32 + ((uint32_t)(rl * 32) + k);
  }
};

__device__ __forceinline__ TileRows tile_rows(uint32_t n, const SeedRule& sr, const SignTable& tb) {
  const uint32_t row0 = blockIdx.x * 32u;
  const int rows = (int)(n - row0 < 32u ? n - row0 : 32u);
  const uint32_t b0 = seed_block(row0, sr), b1 = seed_block(row0 + (uint32_t)(rows - 1), sr);
  return TileRows{row0, rows, b0 == b1, b0, sr, tb};
}

}  // namespace rtq
