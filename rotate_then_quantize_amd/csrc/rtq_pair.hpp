// rtq_pair.hpp -- d = 256 tiles of the fused rotate-then-quantize kernels
// (MI355X, gfx950): two lanes per vector (lane v and lane v + 32, "half 0"
// and "half 1" of the pair), 32 vectors per tile.  The tiles are written once
// and used by the plain entry points (rows of a contiguous [n, 256] tensor)
// and by the cache-layout entry points (rows placed by strides), through a
// row policy:
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
// Coordinates of the packed rotated vector each half holds, as two segments
// of 64 (its registers L[0..63] and L[64..127], in order):
//   SRFT: half 0 coordinates [0, 64) and [192, 256), half 1 [64, 128) and [128, 192);
//   SRHT: half 0 coordinates [0, 64) and [128, 192), half 1 [64, 128) and [192, 256).
// A group of 32 or 64 coordinates lies in one lane, and a lane's codes and
// scales are whole runs of the row's bytes; a group of 128 or 256 spans the
// pair and its absmax is reduced across it.  Both halves run the same
// instructions on their own data.
//
// The halves exchange values with v_permlane32_swap (one VALU instruction per
// register pair, no LDS).  Swapping registers A and B leaves lane v with
// (A of lane v, A of lane v + 32) and lane v + 32 with (B of lane v, B of
// lane v + 32) in (A, B).
//
//   SRFT forward: half p holds the samples u_{2m+p} (m = 0..127) and computes
//     the unnormalized real DFT of its 128 samples, E (p = 0) or O (p = 1),
//     bins 0..64.  With w = exp(-2 pi i / 256), X_b = E_b + w^b O_b and
//     X_{128-b} = conj(E_b - w^b O_b).  For a = 1..31, half 0 forms bins a and
//     128 - a, half 1 bins a + 32 and 96 - a: one swap of bin registers a and
//     a + 32 gives half 0 (E_a, O_a) and half 1 (E_{a+32}, O_{a+32}), and each
//     half reads its own twiddle w^b from an LDS table.  Bins 0, 32 and 64 are
//     formed in both halves and each keeps the coordinates it owns.
//   SRFT inverse: the same exchange backwards: each half forms E and O of its
//     bins from X_b and X_{128-b}, one swap gives half 0 every E_b and half 1
//     every O_b, and each half runs the inverse real DFT of 128 points.
//   SRHT: H_256 = H_2 (x) H_128.  Forward: half p holds the contiguous half p
//     of the samples and applies H_128 (F_p); one swap of registers k and
//     k + 64 gives half 0 (F_0[k], F_1[k]) and half 1 (F_0[k+64], F_1[k+64]),
//     whose sum and difference are the coordinates each owns.  Inverse: each
//     half forms z_i + z_{128+i} and z_i - z_{128+i} of its coordinates, one
//     swap gives half 0 every sum and half 1 every difference, and each
//     applies H_128.
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

// ---------------------------------------------------------------------------
// Lane-pair exchange
// ---------------------------------------------------------------------------

// (a, b) <- v_permlane32_swap(a, b): lane v ends with (a of lane v, a of lane
// v + 32), lane v + 32 with (b of lane v, b of lane v + 32).
__device__ __forceinline__ void pair_swap(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// x of lane v (lo) and of lane v + 32 (hi), in both lanes of the pair.
__device__ __forceinline__ void pair_both(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// Block of 64 packed coordinates that segment s (0 or 1) of half p holds.
template <int ROT>
__device__ __forceinline__ uint32_t seg_block(int p, int s) {
  if constexpr (ROT == kSRFT) return p ? 1u + (uint32_t)s : 3u * (uint32_t)s;  // half 0: 0, 3; half 1: 1, 2
  else return (uint32_t)p + 2u * (uint32_t)s;                                   // half 0: 0, 2; half 1: 1, 3
}

// cos and sin of 2 pi b / 256 for b = 0 .. 63 (the twiddles w^b = c - i s of
// the pair exchange), and c - s, c + s (the inverse exchange with the
// Hartley step folded in), from the same compile-time evaluation as the
// transforms' constants.  Copied into LDS once per tile; half p reads entry
// a + 32 p.
struct PairTwiddles {
  float cs[128];
  float hd[128];
};
consteval PairTwiddles make_pair_twiddles() {
  PairTwiddles t{};
  for (int b = 0; b < 64; ++b) {
    const double c = cos2pi(b, 256), sn = sin2pi(b, 256);
    t.cs[2 * b] = (float)c;
    t.cs[2 * b + 1] = (float)sn;
    t.hd[2 * b] = (float)(c - sn);
    t.hd[2 * b + 1] = (float)(c + sn);
  }
  return t;
}
static __constant__ PairTwiddles kPairTwiddles = make_pair_twiddles();

// The forward's table, (c, s) per entry.
__device__ __forceinline__ void load_pair_twiddles(float* tw, int lane) {
  reinterpret_cast<float2*>(tw)[lane] = reinterpret_cast<const float2*>(kPairTwiddles.cs)[lane];
}

// The inverse's table, (c, s, c - s, c + s) per entry.
__device__ __forceinline__ void load_pair_twiddles_inv(float* tw, int lane) {
  const float2 a = reinterpret_cast<const float2*>(kPairTwiddles.cs)[lane];
  const float2 b = reinterpret_cast<const float2*>(kPairTwiddles.hd)[lane];
  reinterpret_cast<float4*>(tw)[lane] = make_float4(a.x, a.y, b.x, b.y);
}

// The twiddle tables' LDS copies (one object per kernel).
__device__ __forceinline__ float* pair_twiddle_lds() {
  __shared__ float tw[128];
  return tw;
}
__device__ __forceinline__ float* pair_twiddle_lds_inv() {
  __shared__ float tw[256];
  return tw;
}

// ---------------------------------------------------------------------------
// Groups of a lane's 128 coordinates
// ---------------------------------------------------------------------------

// Local groups: LG coordinates each (G for groups of 32 and 64; 64 for the
// groups of 128 and 256 that span the pair).
template <int G> struct PairGroups {
  static constexpr int LG = G <= 64 ? G : 64;
  static constexpr int NLG = 128 / LG;
};

// max |L[i]| over local group GI.
template <int GI, int LG>
__device__ __forceinline__ float local_absmax(const float (&L)[128]) {
  float a = 0.0f;
  sfor<LG>([&](auto I) { a = fmaxf(a, fabsf(L[GI * LG + RTQ_CI(I)])); });
  return a;
}

// Quantize local group GI of (zs * L) with the group's absmax a_raw (of the
// unscaled values, over the whole group wherever it lies): s = fp16_rne(
// zs * a_raw / 2^(B-1)) saturated at 65504, q = clamp(rne(zs * L / s),
// -2^(B-1), 2^(B-1) - 1), q = 0 when s == 0.  Codes form the lane's bit
// stream (code j at bits [j B, (j + 1) B) of cw; for B = 4 the nibble
// layout, two codes per byte, even code low).  B = 4 rounds and packs with
// pack8_int4; other widths round with fma(L, 1/s',
// 1.5 * 2^23), whose fp32 result lies in [2^23, 2^24) where the spacing is 1,
// so the fma's single rounding is round-half-even of L / s' and the low bits
// are q in two's complement, and the caller zeroes cw first.
template <int GI, int LG, int B>
__device__ __forceinline__ void quantize_local_group(const float (&L)[128], float zs, float a_raw,
                                                     uint32_t (&cw)[4 * B], uint32_t (&sb)[128 / LG]) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  constexpr float kLo = -(float)(1 << (B - 1)), kHi = (float)((1 << (B - 1)) - 1);
  constexpr float kInvRange = 1.0f / (float)(1 << (B - 1));
  constexpr int g0 = GI * LG;
  const float a = a_raw * zs;
  uint32_t bits = __half_as_ushort(__float2half_rn(a * kInvRange));
  bits = bits < 0x7bffu ? bits : 0x7bffu;  // saturate (inf -> 65504)
  sb[GI] = bits;
  const float s = __half2float(__ushort_as_half((unsigned short)bits));
  const float inv = bits == 0u ? 0.0f : __builtin_amdgcn_rcpf(s) * zs;
  if constexpr (B == 4) {
    sfor<LG / 8>([&](auto W) {
      constexpr int base = g0 + RTQ_CI(W) * 8;
      cw[base / 8] = pack8_int4(&L[base], inv);
    });
  } else {
    constexpr uint32_t kMask = (1u << B) - 1u;
    sfor<LG>([&](auto I) {
      constexpr int i = g0 + RTQ_CI(I);
      constexpr int pos = i * B, w = pos / 32, sh = pos % 32;
      const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(L[i], inv, kMagic), kMagic + kLo, kMagic + kHi);
      const uint32_t f = __float_as_uint(t) & kMask;
      cw[w] |= f << sh;
      if constexpr (sh + B > 32) cw[w + 1] |= f >> (32 - sh);
    });
  }
}

// Quantize every local group of a lane (groups of G, B-bit codes), with the
// absmax of groups that span the pair (G = 128, 256) reduced across it.
template <int G, int B>
__device__ __forceinline__ void quantize_pair_groups(const float (&L)[128], float zs, uint32_t (&cw)[4 * B],
                                                     uint32_t (&sb)[PairGroups<G>::NLG]) {
  constexpr int LG = PairGroups<G>::LG;
  if constexpr (G <= 64) {
    sfor<128 / LG>([&](auto GI) {
      constexpr int gi = RTQ_CI(GI);
      quantize_local_group<gi, LG, B>(L, zs, local_absmax<gi, LG>(L), cw, sb);
    });
  } else {
    // local group k lies in global group k (G = 128) or 0 (G = 256) in both halves
    float a0 = local_absmax<0, 64>(L), a1 = local_absmax<1, 64>(L);
    float m0, m1;
    if constexpr (G == 128) {
      pair_swap(a0, a1);                  // lane v: (a0, a0 of v + 32); lane v + 32: (a1 of v, a1)
      pair_both(fmaxf(a0, a1), m0, m1);   // group 0's absmax from lane v, group 1's from lane v + 32
    } else {
      float lo, hi;
      pair_both(fmaxf(a0, a1), lo, hi);
      m0 = m1 = fmaxf(lo, hi);
    }
    quantize_local_group<0, 64, B>(L, zs, m0, cw, sb);
    quantize_local_group<1, 64, B>(L, zs, m1, cw, sb);
  }
}

// A lane's codes (two segments of 64 B-bit codes, 8 B bytes each) to or from
// its row of 32 B bytes: segment s goes to bytes 8 B seg_block(p, s).  Even
// B moves 16-byte pieces, B = 3 8-byte pieces.
template <int ROT, int B, bool NT>
__device__ __forceinline__ void store_pair_codes(uint4* codes, size_t row, int p, const uint32_t (&cw)[4 * B]) {
  if constexpr (B % 2 == 0) {
    constexpr int PS = B / 2;  // 16-byte pieces per segment
    sfor<2>([&](auto S) {
      uint4* dst = codes + row * (2 * B) + seg_block<ROT>(p, RTQ_CI(S)) * PS;
      sfor<PS>([&](auto C) {
        constexpr int w = (RTQ_CI(S) * PS + RTQ_CI(C)) * 4;
        put_store<NT>(dst + RTQ_CI(C), make_uint4(cw[w], cw[w + 1], cw[w + 2], cw[w + 3]));
      });
    });
  } else {
    uint2* base = reinterpret_cast<uint2*>(codes);
    sfor<2>([&](auto S) {
      uint2* dst = base + row * (4 * B) + seg_block<ROT>(p, RTQ_CI(S)) * B;
      sfor<B>([&](auto C) {
        constexpr int w = (RTQ_CI(S) * B + RTQ_CI(C)) * 2;
        put_store<NT>(dst + RTQ_CI(C), make_uint2(cw[w], cw[w + 1]));
      });
    });
  }
}

// A lane's codes and (load_pair_scales) scales, by ordinary loads.  Each
// load instruction takes one or two 16-byte pieces of every 128-byte line it
// touches, and the pair's other pieces come with the next instructions:
// with the non-temporal hint the L2 let many lines go in between and the
// d = 256 inverse fetched 10.7% more than its codes and scales (7% slower).
template <int ROT, int B>
__device__ __forceinline__ void load_pair_codes(const uint4* codes, size_t row, int p, uint32_t (&cw)[4 * B]) {
  if constexpr (B % 2 == 0) {
    constexpr int PS = B / 2;
    sfor<2>([&](auto S) {
      const uint4* src = codes + row * (2 * B) + seg_block<ROT>(p, RTQ_CI(S)) * PS;
      sfor<PS>([&](auto C) {
        constexpr int w = (RTQ_CI(S) * PS + RTQ_CI(C)) * 4;
        const uint4 q = src[RTQ_CI(C)];
        cw[w] = q.x;
        cw[w + 1] = q.y;
        cw[w + 2] = q.z;
        cw[w + 3] = q.w;
      });
    });
  } else {
    const uint2* base = reinterpret_cast<const uint2*>(codes);
    sfor<2>([&](auto S) {
      const uint2* src = base + row * (4 * B) + seg_block<ROT>(p, RTQ_CI(S)) * B;
      sfor<B>([&](auto C) {
        constexpr int w = (RTQ_CI(S) * B + RTQ_CI(C)) * 2;
        const uint2 q = src[RTQ_CI(C)];
        cw[w] = q.x;
        cw[w + 1] = q.y;
      });
    });
  }
}

// A lane's scales to or from its row of 512 / G bytes.  G = 32: local groups
// 2s, 2s + 1 are global groups 2 b, 2 b + 1 of block b = seg_block(p, s) (a
// 4-byte word each); G = 64: local group s is global group b (2 bytes each);
// G = 128 and 256: the row's scales, identical in both halves, written by
// half 0.
template <int ROT, int G, bool NT>
__device__ __forceinline__ void store_pair_scales(uint8_t* scales, size_t row, int p,
                                                  const uint32_t (&sb)[PairGroups<G>::NLG]) {
  if constexpr (G == 32) {
    uint32_t* r = reinterpret_cast<uint32_t*>(scales) + row * 4;
    put_store<NT>(r + seg_block<ROT>(p, 0), sb[0] | (sb[1] << 16));
    put_store<NT>(r + seg_block<ROT>(p, 1), sb[2] | (sb[3] << 16));
  } else if constexpr (G == 64) {
    uint16_t* r = reinterpret_cast<uint16_t*>(scales) + row * 4;
    put_store<NT>(r + seg_block<ROT>(p, 0), (uint16_t)sb[0]);
    put_store<NT>(r + seg_block<ROT>(p, 1), (uint16_t)sb[1]);
  } else if constexpr (G == 128) {
    if (p == 0) put_store<NT>(reinterpret_cast<uint32_t*>(scales) + row, sb[0] | (sb[1] << 16));
  } else {
    if (p == 0) put_store<NT>(reinterpret_cast<uint16_t*>(scales) + row, (uint16_t)sb[0]);
  }
}

template <int ROT, int G>
__device__ __forceinline__ void load_pair_scales(const uint8_t* scales, size_t row, int p,
                                                 uint32_t (&sb)[PairGroups<G>::NLG]) {
  if constexpr (G == 32) {
    const uint32_t* r = reinterpret_cast<const uint32_t*>(scales) + row * 4;
    const uint32_t w0 = r[seg_block<ROT>(p, 0)], w1 = r[seg_block<ROT>(p, 1)];
    sb[0] = w0 & 0xffffu;
    sb[1] = w0 >> 16;
    sb[2] = w1 & 0xffffu;
    sb[3] = w1 >> 16;
  } else if constexpr (G == 64) {
    const uint16_t* r = reinterpret_cast<const uint16_t*>(scales) + row * 4;
    sb[0] = r[seg_block<ROT>(p, 0)];
    sb[1] = r[seg_block<ROT>(p, 1)];
  } else if constexpr (G == 128) {
    const uint32_t w = reinterpret_cast<const uint32_t*>(scales)[row];
    sb[0] = w & 0xffffu;
    sb[1] = w >> 16;
  } else {
    sb[0] = sb[1] = reinterpret_cast<const uint16_t*>(scales)[row];
  }
}

// ---------------------------------------------------------------------------
// SRFT exchange of the pair
// ---------------------------------------------------------------------------

// One bin of the forward exchange (a = 1..31): bins a and a + 32 of E and O
// (fr, fi: the lane's own real DFT) become coordinates 2b-1, 2b (X_b) and
// 255-2b, 256-2b (X_{128-b}) of the lane's bin b = a + 32 p, as local
// registers L[2a-1], L[2a], L[127-2a], L[128-2a].
template <int A>
__device__ __forceinline__ void srft_fwd_bin(float (&fr)[65], float (&fi)[65], const float2* twl, float (&L)[128]) {
  constexpr int a = A;
  pair_swap(fr[a], fr[a + 32]);  // (E_b, O_b) re in both halves
  pair_swap(fi[a], fi[a + 32]);
  const float2 t = twl[a];       // w^b = t.x - i t.y
  const float er = fr[a], ei = fi[a], orr = fr[a + 32], oi = fi[a + 32];
  const float xr = __builtin_fmaf(t.x, orr, __builtin_fmaf(t.y, oi, er));   // X_b = E + w^b O
  const float xi = __builtin_fmaf(t.x, oi, __builtin_fmaf(-t.y, orr, ei));
  L[2 * a - 1] = xr;
  L[2 * a] = xi;
  L[127 - 2 * a] = __builtin_fmaf(2.0f, er, -xr);  // Re X_{128-b} = 2 Re E - Re X_b
  L[128 - 2 * a] = __builtin_fmaf(-2.0f, ei, xi);  // Im X_{128-b} = Im X_b - 2 Im E
}

// Bins 0, 32 and 64 of the forward exchange.  Half 0 owns X_0 (L[0]), X_128
// (L[127]), Re X_32 (L[63]) and Im X_96 (L[64]); half 1 owns Im X_32 (L[0]),
// Re X_96 (L[127]) and X_64 = E_64 - i O_64 (L[63], L[64]).  The real end
// bins carry 1/sqrt2 (their orthonormal scale is 1/16, the others'
// sqrt(2/256), which the quantizer applies).
__device__ __forceinline__ void srft_fwd_edges(float (&fr)[65], float (&fi)[65], int p, float (&L)[128]) {
  pair_swap(fr[0], fr[64]);  // half 0: (E_0, O_0), half 1: (E_64, O_64)
  float e32r, o32r, e32i, o32i;
  pair_both(fr[32], e32r, o32r);
  pair_both(fi[32], e32i, o32i);
  constexpr float h = 0.70710678118654752440f;  // w^32 = h - i h
  const float xr = __builtin_fmaf(h, o32r, __builtin_fmaf(h, o32i, e32r));
  const float xi = __builtin_fmaf(h, o32i, __builtin_fmaf(-h, o32r, e32i));
  const float yr = __builtin_fmaf(2.0f, e32r, -xr), yi = __builtin_fmaf(-2.0f, e32i, xi);  // X_96
  const float P = fr[0], Q = fr[64];
  constexpr float r2 = 0.70710678118654752440f;
  L[0] = p ? xi : (P + Q) * r2;
  L[127] = p ? yr : (P - Q) * r2;
  L[63] = p ? P : xr;
  L[64] = p ? -Q : yi;
}

// The inverse exchange takes the lane's coordinates L (z / 2, times any
// common factor) to the packed 128-point spectrum Y of the lane's own samples
// (E for half 0, O for half 1) in the convention of srft_inv<128, Sqrt2>,
// times the same factor.  This gives its entries 0, 63, 64 and 127 (bins 0,
// 32, 64 and 96).
__device__ __forceinline__ void srft_inv_edges(const float (&L)[128], int p, float& y0, float& y63, float& y64,
                                               float& y127) {
  const float sigma = p ? -1.0f : 1.0f;
  float x0, imx32, x128, rex96, rex32, rex64, imx96, imx64;
  pair_both(L[0], x0, imx32);
  pair_both(L[127], x128, rex96);
  pair_both(L[63], rex32, rex64);
  pair_both(L[64], imx96, imx64);
  y0 = __builtin_fmaf(sigma, x128, x0);  // E_0 or O_0
  const float er = rex32 + rex96, ei = imx32 - imx96, dr = rex32 - rex96, di = imx32 + imx96;
  constexpr float h = 0.70710678118654752440f;  // w^-32 = h + i h
  y63 = p ? h * (dr - di) : er;
  y64 = p ? h * (di + dr) : ei;
  constexpr float sq2 = 1.41421356237309504880f;  // E_64 = Re X_64, O_64 = -Im X_64
  y127 = (p ? -imx64 : rex64) * sq2;
}

// The inverse exchange followed by srft_inv_hartley's first step, folded
// together: g_m = Re Y_m - Im Y_m and g_{128-m} = Re Y_m + Im Y_m of the
// lane's spectrum Y (m = 1 .. 63), g_0 = sqrt2 Y_0, g_64 = sqrt2 Y_64.  For
// the O half, Re - Im and Re + Im of w^-b (dr + i di) come straight from
// c - s and c + s: (c - s) dr - (c + s) di and (c + s) dr + (c - s) di.
__device__ __forceinline__ void srft_inv_exchange_hartley(const float (&L)[128], const float4* twl, int p,
                                                          float (&g)[128]) {
  constexpr float sq2 = 1.41421356237309504880f;
  {
    float y0, y63, y64, y127;
    srft_inv_edges(L, p, y0, y63, y64, y127);
    g[0] = sq2 * y0;
    g[64] = sq2 * y127;
    g[32] = y63 - y64;
    g[96] = y63 + y64;
  }
  sfor<31>([&](auto A) {
    constexpr int a = RTQ_CI(A) + 1;
    const float ar = L[2 * a - 1], ai = L[2 * a], br = L[127 - 2 * a], bi = L[128 - 2 * a];
    const float er = ar + br, ei = ai - bi;  // E_b = (X_b + conj X_{128-b}) / 2
    const float dr = ar - br, di = ai + bi;  // w^b O_b
    const float4 t = twl[a];                 // (c, s, c - s, c + s) of w^-b = c + i s
    float em = er - ei, ep = er + ei;
    float om = __builtin_fmaf(t.z, dr, -t.w * di), op = __builtin_fmaf(t.w, dr, t.z * di);
    pair_swap(em, om);  // half 0: bins a and a + 32 of E; half 1: of O
    pair_swap(ep, op);
    g[a] = em;
    g[128 - a] = ep;
    g[a + 32] = om;
    g[96 - a] = op;
  });
}

// ---------------------------------------------------------------------------
// Forward tile
// ---------------------------------------------------------------------------

// Forward tile: rows R.row0 .. R.row0 + R.rows - 1 of x (contiguous, 32
// 16-byte chunks per row) into the codes / scales rows R.cache_row(.), with
// B-bit codes (one little-endian bit stream per row, 32 B bytes) and an
// optional per-channel lambda.  lds holds 16 x 33 uint4.
template <int G, int ROT, class Rows, int B = 4>
__device__ __forceinline__ void fwd_pair_tile(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                              uint8_t* __restrict__ scales, const Rows& R, uint4* lds, int lane,
                                              const uint32_t* __restrict__ lam = nullptr) {
  constexpr int CPR = 32, LROW = CPR + 1;
  constexpr int NLG = PairGroups<G>::NLG;
  const int p = lane >> 5, v = lane & 31;
  const uint32_t kpos = lane & 31;
  float* tw = pair_twiddle_lds();
  if constexpr (ROT == kSRFT) load_pair_twiddles(tw, lane);  // read after the barrier below
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
    // The tile reaches LDS in two passes of 16 rows (rows 0..15, then 16..31),
    // each read back by the lanes of its rows: a 16-row buffer leaves room
    // for three waves per SIMD.
    uint32_t h[64];
    auto fetch = [&]() {
      const int lr = v & 15;
      sfor<16>([&](auto C) {
        const uint4 q = lds[lr * LROW + 16 * p + RTQ_CI(C)];
        h[4 * RTQ_CI(C) + 0] = q.x;
        h[4 * RTQ_CI(C) + 1] = q.y;
        h[4 * RTQ_CI(C) + 2] = q.z;
        h[4 * RTQ_CI(C) + 3] = q.w;
      });
    };
    if (uniform) {
      const uint4* xt = x + (size_t)row0 * CPR;
      uint4 in[16];
      if (rows == 32) {  // a full tile loads without per-row guards (about 100 instructions less)
        sfor<16>([&](auto J) { in[RTQ_CI(J)] = stream_load(xt + ((uint32_t)((2 * RTQ_CI(J) + p) * CPR) + kpos)); });
      } else {
        sfor<16>([&](auto J) {
          const int rl = 2 * RTQ_CI(J) + p;
          in[RTQ_CI(J)] = rl < rows ? stream_load(xt + ((uint32_t)(rl * CPR) + kpos)) : make_uint4(0, 0, 0, 0);
        });
      }
      sfor<2>([&](auto P) {
        constexpr int ps = RTQ_CI(P);
        if constexpr (ps > 0) {
          wait_lds_reads();
          lds_sync();
        }
        sfor<8>([&](auto J) { put(2 * RTQ_CI(J) + p, xor4(in[8 * ps + RTQ_CI(J)], cm)); });
        lds_sync();
        if ((v >> 4) == ps) fetch();
      });
    } else {
      sfor<2>([&](auto P) {
        constexpr int ps = RTQ_CI(P);
        if constexpr (ps > 0) {
          wait_lds_reads();
          lds_sync();
        }
#pragma unroll 1
        for (int j = 0; j < 8; ++j) {
          const int rl = 16 * ps + 2 * j + p;
          const uint4 q = rl < rows ? stream_load(x + ((size_t)(row0 + rl) * CPR + kpos)) : make_uint4(0, 0, 0, 0);
          put(2 * j + p, xor4(q, R.row_masks(rl, kpos)));
        }
        lds_sync();
        if ((v >> 4) == ps) fetch();
      });
    }
    wait_lds_reads();
    lds_sync();
    float L[128];
    float zs;
    uint32_t cw[4 * B], sb[NLG];
    if constexpr (B != 4) sfor<4 * B>([&](auto K) { cw[RTQ_CI(K)] = 0u; });
    if constexpr (ROT == kSRFT) {
      float fr[65], fi[65];  // unnormalized; sqrt(2/256) is applied by the quantizer
      if (lam != nullptr) {
        float uw[128];
        lambda_half<kSRFT>(h, lam, p, uw);
        rfft_bins<128, UnitBins>(uw, fr, fi);
      } else {
        rdft<128, 1, 0, 64>(h, fr, fi);
      }
      zs = SrftScale<256>::value;
      const float2* twl = reinterpret_cast<const float2*>(tw) + 32 * p;
      srft_fwd_edges(fr, fi, p, L);
      if constexpr (G == 32) {
        // bins 1..16 complete local groups 0 and 3, bins 17..31 groups 1 and 2:
        // quantize each pair of groups as soon as it is complete
        sfor<16>([&](auto A) { srft_fwd_bin<RTQ_CI(A) + 1>(fr, fi, twl, L); });
        quantize_local_group<0, 32, B>(L, zs, local_absmax<0, 32>(L), cw, sb);
        quantize_local_group<3, 32, B>(L, zs, local_absmax<3, 32>(L), cw, sb);
        sfor<15>([&](auto A) { srft_fwd_bin<RTQ_CI(A) + 17>(fr, fi, twl, L); });
        quantize_local_group<1, 32, B>(L, zs, local_absmax<1, 32>(L), cw, sb);
        quantize_local_group<2, 32, B>(L, zs, local_absmax<2, 32>(L), cw, sb);
      } else {
        sfor<31>([&](auto A) { srft_fwd_bin<RTQ_CI(A) + 1>(fr, fi, twl, L); });
        quantize_pair_groups<G, B>(L, zs, cw, sb);
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
      // coordinates k (half 0) or 64 + k (half 1), and 128 + k or 192 + k
      auto combine = [&](auto K) {
        constexpr int k = RTQ_CI(K);
        pair_swap(f[k], f[k + 64]);
        L[k] = f[k] + f[k + 64];
        L[k + 64] = f[k] - f[k + 64];
      };
      if constexpr (G == 32) {
        sfor<32>([&](auto K) { combine(K); });
        quantize_local_group<0, 32, B>(L, zs, local_absmax<0, 32>(L), cw, sb);
        quantize_local_group<2, 32, B>(L, zs, local_absmax<2, 32>(L), cw, sb);
        sfor<32>([&](auto K) { combine(ic<RTQ_CI(K) + 32>{}); });
        quantize_local_group<1, 32, B>(L, zs, local_absmax<1, 32>(L), cw, sb);
        quantize_local_group<3, 32, B>(L, zs, local_absmax<3, 32>(L), cw, sb);
      } else {
        sfor<64>([&](auto K) { combine(K); });
        quantize_pair_groups<G, B>(L, zs, cw, sb);
      }
    }
    if (v < rows) {
      const size_t row = R.cache_row(v);
      // Each lane writes two runs of its row in 16- or 8-byte pieces, so one
      // store instruction leaves one or two pieces in each 128-byte line:
      // ordinary stores let L2 merge them into full lines.
      store_pair_codes<ROT, B, false>(codes, row, p, cw);
      store_pair_scales<ROT, G, Rows::kStreamStores>(scales, row, p, sb);
    }
  }
}

// ---------------------------------------------------------------------------
// Inverse tile
// ---------------------------------------------------------------------------

// Inverse tile: the codes / scales rows R.cache_row(.) into the rows of y
// that R.y_chunk addresses, for B-bit codes, divided by lambda when LAM.
// lds holds 544 uint4 (16 x 33 used for SRFT, 32 x 17 for SRHT).  The lambda
// case is a template parameter: with both transform paths behind a run-time
// branch the compiler merges their common steps and spills about 130
// registers.
template <int G, int ROT, class Rows, int B = 4, bool LAM = false>
__device__ __forceinline__ void inv_pair_tile(const uint4* __restrict__ codes, const uint8_t* __restrict__ scales,
                                              uint4* __restrict__ y, const Rows& R, uint4* lds, int lane,
                                              const uint32_t* __restrict__ lam = nullptr, float* inv_lam = nullptr) {
  constexpr int NLG = PairGroups<G>::NLG, LG = PairGroups<G>::LG;
  if constexpr (LAM) pair_lambda_reciprocals<ROT>(lam, inv_lam, lane);  // read after a barrier below
  float* tw = pair_twiddle_lds_inv();
  if constexpr (ROT == kSRFT) load_pair_twiddles_inv(tw, lane);  // read after the first barrier below
  const int p = lane >> 5, v = lane & 31;
  {
    const int rows = R.rows;
    const bool uniform = R.uniform;
    uint32_t cw[4 * B], sb[NLG];
    {
      const size_t row = R.cache_row(v < rows ? v : 0);
      load_pair_codes<ROT, B>(codes, row, p, cw);
      load_pair_scales<ROT, G>(scales, row, p, sb);
    }
    // Every sample is rounded to fp16 pairs before the output passes begin,
    // so that no transform value stays live across them (the compiler would
    // otherwise finish the last butterflies lazily inside the second pass and
    // spill around the first).
    uint32_t hw[64];
    auto pack_all = [&](const float (&u)[128]) {
      sfor<64>([&](auto M) { hw[RTQ_CI(M)] = pack_f16x2(u[2 * RTQ_CI(M)], u[2 * RTQ_CI(M) + 1]); });
    };
    if constexpr (ROT == kSRFT) {
      // L = z / 2 (the halving of E and O) times 1/sqrt(128), the factor
      // srft_inv_hartley expects on its input
      constexpr float kDeq = (float)(0.5 / csqrt(128.0));
      float L[128], yv[128];
      if constexpr (B == 4) dequant_unpack<128, LG>(cw, sb, kDeq, L);
      else dequant_unpack_bits<128, LG, B>(cw, sb, kDeq, L);
      lds_sync();  // the twiddle and reciprocal tables are written
      const float4* twl = reinterpret_cast<const float4*>(tw) + 32 * p;
      srft_inv_exchange_hartley(L, twl, p, yv);
      hartley_f32_packed<128, LAM>(yv, hw, LAM ? inv_lam + p * 132 : nullptr);  // u / lambda when LAM
    } else {
      float L[128], u[128];
      if constexpr (B == 4) dequant_unpack<128, LG>(cw, sb, 1.0f / 16.0f, L);
      else dequant_unpack_bits<128, LG, B>(cw, sb, 1.0f / 16.0f, L);
      // half 0: z_k + z_{128+k}, half 1: z_k - z_{128+k}, k = 0 .. 127
      sfor<64>([&](auto K) {
        constexpr int k = RTQ_CI(K);
        float s = L[k] + L[k + 64], d = L[k] - L[k + 64];
        pair_swap(s, d);
        u[k] = s;
        u[k + 64] = d;
      });
      fwht_f32<128>(u);
      if constexpr (LAM) {
        lds_sync();
        unweight_half(u, inv_lam, p);
      }
      pack_all(u);
    }
    sfor<16>([&](auto Q) { pin_words<4 * RTQ_CI(Q)>(hw); });
    // fp16 samples out through LDS in two passes (a 9 KB tile).
    //   SRFT: lane p holds the samples u_{2m+p}.  Pass ph takes whole rows
    //   16 ph .. 16 ph + 15: their lanes write their samples of parity p to
    //   part p of the LDS row, and the wave re-interleaves the even and odd
    //   samples and stores two whole rows (1 KB of contiguous output) per
    //   instruction.
    //   SRHT: lane p holds output chunks 16 p .. 16 p + 15, written in pass p
    //   for every row (whole-row passes measured slower here).
    if constexpr (ROT == kSRFT) {
      // uint4 per LDS row: 16 of evens, a pad, 16 of odds.  An odd row stride
      // puts the 16 rows one access writes in 16 different groups of 4 banks.
      constexpr int LR3 = 33;
      const uint32_t k = (uint32_t)(lane & 31);  // output chunk this lane stores
      const int rh = lane >> 5;
      auto get = [&](int r) -> uint4 {  // chunk k of local row r
        const uint2* row = reinterpret_cast<const uint2*>(&lds[r * LR3]);
        const uint2 e = row[k], o = row[34 + k];
        return make_uint4(__builtin_amdgcn_perm(o.x, e.x, 0x05040100u), __builtin_amdgcn_perm(o.x, e.x, 0x07060302u),
                          __builtin_amdgcn_perm(o.y, e.y, 0x05040100u), __builtin_amdgcn_perm(o.y, e.y, 0x07060302u));
      };
      sfor<2>([&](auto PH) {
        constexpr int ph = RTQ_CI(PH);
        if constexpr (ph > 0) {
          wait_lds_reads();
          lds_sync();
        }
        if ((v >> 4) == ph) {
          sfor<16>([&](auto C) {
            constexpr int c = RTQ_CI(C);
            lds[(v & 15) * LR3 + 17 * p + c] = make_uint4(hw[4 * c], hw[4 * c + 1], hw[4 * c + 2], hw[4 * c + 3]);
          });
        }
        lds_sync();
        if (uniform && rows == 32) {  // a full tile stores without per-row guards
          const uint4 m = R.uniform_masks(k);
          sfor<8>([&](auto J) {
            const int r = 2 * RTQ_CI(J) + rh;
            put_store<Rows::kStreamStores>(R.y_chunk(y, 16 * ph + r, k), xor4(get(r), m));
          });
        } else if (uniform) {
          const uint4 m = R.uniform_masks(k);
          sfor<8>([&](auto J) {
            const int r = 2 * RTQ_CI(J) + rh;
            if (16 * ph + r < rows) put_store<Rows::kStreamStores>(R.y_chunk(y, 16 * ph + r, k), xor4(get(r), m));
          });
        } else {
#pragma unroll 1
          for (int j = 0; j < 8; ++j) {
            const int r = 2 * j + rh, rl = 16 * ph + r;
            if (rl < rows) put_store<Rows::kStreamStores>(R.y_chunk(y, rl, k), xor4(get(r), R.row_masks(rl, k)));
          }
        }
      });
    } else {
      constexpr int LR2 = 17;
      const int kk = lane & 15, rsub = lane >> 4;
      sfor<2>([&](auto PH) {
        constexpr int ph = RTQ_CI(PH);
        if constexpr (ph > 0) {
          wait_lds_reads();
          lds_sync();
        }
        if (p == ph) {
          sfor<16>([&](auto C) {
            constexpr int c = RTQ_CI(C);
            lds[v * LR2 + c] = make_uint4(hw[4 * c], hw[4 * c + 1], hw[4 * c + 2], hw[4 * c + 3]);
          });
        }
        lds_sync();
        const uint32_t k = 16u * ph + (uint32_t)kk;  // output chunk this lane stores
        auto get = [&](int rl) -> uint4 { return lds[rl * LR2 + kk]; };
        if (uniform && rows == 32) {  // a full tile stores without per-row guards
          const uint4 m = R.uniform_masks(k);
          sfor<8>([&](auto J) {
            const int rl = rsub + 4 * RTQ_CI(J);
            put_store<Rows::kStreamStores>(R.y_chunk(y, rl, k), xor4(get(rl), m));
          });
        } else if (uniform) {
          const uint4 m = R.uniform_masks(k);
          sfor<8>([&](auto J) {
            const int rl = rsub + 4 * RTQ_CI(J);
            if (rl < rows) put_store<Rows::kStreamStores>(R.y_chunk(y, rl, k), xor4(get(rl), m));
          });
        } else {
#pragma unroll 1
          for (int j = 0; j < 8; ++j) {
            const int rl = rsub + 4 * j;
            if (rl < rows) put_store<Rows::kStreamStores>(R.y_chunk(y, rl, k), xor4(get(rl), R.row_masks(rl, k)));
          }
        }
      });
    }
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
