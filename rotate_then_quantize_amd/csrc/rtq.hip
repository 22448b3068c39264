// rtq.hip -- fused rotate-then-quantize int4 kernels for MI355X (gfx950) and
// the C ABI declared in include/rtq.h.
//
// The method ("Quantization Speed Is Often a Kernel Problem", sections
// "First, the 17%" and "Fusing four steps into two kernels is not enough"):
// each K/V vector gets its signs flipped by a seeded +-1 vector and is rotated
// (SRFT = real FFT, SRHT = Hadamard control), then quantized to int4 with one
// absmax fp16 scale per group; the inverse dequantizes, rotates back and flips the signs.  One
// launch does the forward step for all rows, one launch the inverse.
//
// Mapping to CDNA4:
//   * A wave (64 lanes, one wave per workgroup) owns a tile of rows.  d = 64
//     and d = 128 vectors live in the registers of one lane (64 rows per
//     tile); d = 256 vectors span two lanes, lane v (even samples for SRFT,
//     first half for SRHT) and lane v+32 (32 rows per tile).
//   * Rows are read and written with fully coalesced 16-byte accesses and
//     transposed to / from the owning lane through a wave-private LDS tile:
//     forward tiles arrive by direct-to-LDS loads (global_load_lds_dwordx4)
//     with an xor swizzle that keeps the per-row LDS reads conflict free, and
//     the packed codes leave through LDS as full 1 KB stores.  All global
//     accesses are non-temporal: each byte is used once.
//   * The +-1 signs of a tile come from one SplitMix64 evaluation per lane, a
//     ballot, and scalar bit extraction, then one v_xor per packed pair.
//   * The transforms, the absmax reduction, rounding, clamping and nibble
//     packing are straight-line register code (rtq_device.hpp); there is no
//     dense contraction and no MFMA.
//   * Row indices are 32-bit (any tensor that fits in HBM has fewer than 2^32
//     rows); addresses are a wave-uniform 64-bit tile base plus 32-bit lane
//     offsets; the seed rule divides with precomputed multipliers
//     (rtq_div.hpp).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "rtq.h"
#include "rtq_device.hpp"
#include "rtq_div.hpp"
#include "rtq_host.hpp"
#include "rtq_lane.hpp"
#include "rtq_mem.hpp"

namespace rtq {

// ---------------------------------------------------------------------------
// d = 64 / 128: one lane per vector, 64 vectors per tile.
// ---------------------------------------------------------------------------

// One forward tile: rows row0 .. row0 + rows - 1, lane l owning row row0 + l.
// kUniform: every row has seed s (masks are scalar); otherwise s is the
// lane's own seed.
template <int D, int G, int ROT, bool kUniform>
__device__ __forceinline__ void fwd_lane_tile(const uint4* __restrict__ xt, uint4* __restrict__ ct,
                                              uint8_t* __restrict__ st, int rows, const SignTable& tb,
                                              uint32_t j, uint64_t s, uint4* buf, int lane) {
  constexpr int CPR = D / 8;  // 16-byte chunks per input row
  constexpr int CW = D / 32;  // 16-byte chunks per code row
  load_tile_to_lds<CPR>(xt, rows, buf, lane);
  UniformSigns<D> sg;
  if constexpr (kUniform) sg.setup(tb, j, s, lane);  // overlaps the loads
  wait_vmcnt<0>();
  lds_sync();
  uint32_t h[D / 2];
  read_own_row<CPR>(buf, lane, h);
  if constexpr (kUniform) sg.apply(h);
  else apply_lane_signs<D>(h, s);
  uint32_t cw[D / 8], sb[D / G];
  quantize_row<D, G, ROT>(h, cw, sb);
  // codes leave through LDS (the input tile is no longer needed)
  lds_sync();
  sfor<CW>([&](auto C) {
    buf[lane * CW + RTQ_CI(C)] =
        make_uint4(cw[4 * RTQ_CI(C)], cw[4 * RTQ_CI(C) + 1], cw[4 * RTQ_CI(C) + 2], cw[4 * RTQ_CI(C) + 3]);
  });
  lds_sync();
  sfor<CW>([&](auto J) {
    const int c = RTQ_CI(J) * 64 + lane;  // chunk of the tile's code block (row c / CW)
    if (c / CW < rows) stream_store(ct + (uint32_t)c, buf[c]);
  });
  if (lane < rows) store_row_scales<D, G>(st, (uint32_t)lane, sb);
}

// Forward step, one 64-row tile per wave.
template <int D, int G, int ROT>
__global__ __launch_bounds__(64) void fwd_lane_kernel(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, uint32_t n, SeedRule sr, SignTable tb) {
  constexpr int CPR = D / 8;
  constexpr int CW = D / 32;
  __shared__ uint4 buf[64 * CPR];
  const int lane = threadIdx.x;
  const uint32_t row0 = blockIdx.x * 64u;
  const int rows = (int)(n - row0 < 64u ? n - row0 : 64u);
  const uint4* xt = x + (size_t)row0 * CPR;
  uint4* ct = codes + (size_t)row0 * CW;
  uint8_t* st = scales + (size_t)row0 * (2 * D / G);
  const uint32_t b0 = seed_block(row0, sr), b1 = seed_block(row0 + (uint32_t)(rows - 1), sr);
  if (b0 == b1) fwd_lane_tile<D, G, ROT, true>(xt, ct, st, rows, tb, seed_offset(b0, sr), sr.seed, buf, lane);
  else fwd_lane_tile<D, G, ROT, false>(xt, ct, st, rows, tb, 0, lane_seed(sr, row0, rows, lane), buf, lane);
}

// Direct-to-LDS staging of a tile's code block (CW 16-byte chunks per row, in
// row order): load instruction j of lane i fills slot 64j + i with chunk
// 64j + i, a partial tile repeating its last row.
template <int CW>
__device__ __forceinline__ void load_codes_to_lds(const uint4* __restrict__ ct, int rows, uint4* buf, int lane) {
  sfor<CW>([&](auto J) {
    const int c = RTQ_CI(J) * 64 + lane;
    const int r = c / CW;
    const int rr = r < rows ? r : rows - 1;
    const uint32_t off = (uint32_t)(rr * CW + c % CW) * 16u;
    __builtin_amdgcn_global_load_lds((gbl_void_t*)((const char*)ct + off), (lds_void_t*)(buf + RTQ_CI(J) * 64), 16,
                                     0, kCachePolicyNT);
  });
}

// One inverse tile: rows row0 .. row0 + rows - 1, lane l owning row row0 + l.
// The code block arrives coalesced in LDS, each lane reads its own row, and
// the fp16 output leaves through the same LDS buffer (padded rows) as
// coalesced 16-byte stores.
template <int D, int G, int ROT, bool kUniform>
__device__ __forceinline__ void inv_lane_tile(const uint4* __restrict__ ct, const uint8_t* __restrict__ st,
                                              uint4* __restrict__ yt, int rows, const SignTable& tb, uint32_t j,
                                              uint64_t s, uint4* lds, int lane) {
  constexpr int CPR = D / 8;
  constexpr int CW = D / 32;
  const uint32_t r = (uint32_t)(lane < rows ? lane : rows - 1);
  load_codes_to_lds<CW>(ct, rows, lds, lane);
  uint32_t sb[D / G];
  load_row_scales<D, G>(st, r, sb);
  UniformSigns<D> sg;
  if constexpr (kUniform) sg.setup(tb, j, s, lane);  // overlaps the loads
  wait_vmcnt<0>();
  lds_sync();
  uint32_t cw[D / 8];
  sfor<CW>([&](auto C) {
    const uint4 q = lds[r * CW + RTQ_CI(C)];
    cw[4 * RTQ_CI(C) + 0] = q.x;
    cw[4 * RTQ_CI(C) + 1] = q.y;
    cw[4 * RTQ_CI(C) + 2] = q.z;
    cw[4 * RTQ_CI(C) + 3] = q.w;
  });
  float z[D], u[D];
  if constexpr (ROT == kSRFT) {
    dequant_unpack<D, G>(cw, sb, 1.0f, z);
    srft_inv<D, One>(z, u);
  } else {
    dequant_unpack<D, G>(cw, sb, InvSqrt<D>::value, u);
    fwht_f32<D>(u);
  }
  uint32_t h[D / 2];
  sfor<D / 2>([&](auto M) { h[RTQ_CI(M)] = pack_f16x2(u[2 * RTQ_CI(M)], u[2 * RTQ_CI(M) + 1]); });
  if constexpr (kUniform) sg.apply(h);
  else apply_lane_signs<D>(h, s);
  // Own row into LDS (the code block has been read), then coalesced chunks
  // out.  d = 128 goes in two halves of 8 chunks per row, which halves the
  // LDS tile (9 KB) so that LDS does not cap the resident waves.
  wait_lds_reads();
  lds_sync();
  constexpr int PH = InvPhases<D>::value;
  constexpr int PC = CPR / PH, LR = PC + 1;
  sfor<PH>([&](auto P) {
    constexpr int ph = RTQ_CI(P);
    if constexpr (ph > 0) {
      wait_lds_reads();
      lds_sync();
    }
    sfor<PC>([&](auto C) {
      constexpr int c = ph * PC + RTQ_CI(C);
      lds[lane * LR + RTQ_CI(C)] = make_uint4(h[4 * c], h[4 * c + 1], h[4 * c + 2], h[4 * c + 3]);
    });
    lds_sync();
    sfor<PC>([&](auto J) {
      const int idx = RTQ_CI(J) * 64 + lane;
      const int rl = idx / PC, kk = idx % PC;
      if (rl < rows) stream_store(yt + (uint32_t)(rl * CPR + ph * PC + kk), lds[rl * LR + kk]);
    });
  });
}

// Inverse step, one 64-row tile per wave.  At most 168 VGPRs (3 waves per
// SIMD): d = 128 then spills a little, and still runs 5% faster than at 2.
template <int D, int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void inv_lane_kernel(
    const uint4* __restrict__ codes, const uint8_t* __restrict__ scales, uint4* __restrict__ y, uint32_t n,
    SeedRule sr, SignTable tb) {
  constexpr int CPR = D / 8;
  constexpr int CW = D / 32;
  constexpr int LT = 64 * (CPR / InvPhases<D>::value + 1);  // output tile (uint4)
  __shared__ uint4 lds[LT > 64 * CW ? LT : 64 * CW];
  const int lane = threadIdx.x;
  const uint32_t row0 = blockIdx.x * 64u;
  const int rows = (int)(n - row0 < 64u ? n - row0 : 64u);
  const uint4* ct = codes + (size_t)row0 * CW;
  const uint8_t* st = scales + (size_t)row0 * (2 * D / G);
  uint4* yt = y + (size_t)row0 * CPR;
  const uint32_t b0 = seed_block(row0, sr), b1 = seed_block(row0 + (uint32_t)(rows - 1), sr);
  if (b0 == b1) inv_lane_tile<D, G, ROT, true>(ct, st, yt, rows, tb, seed_offset(b0, sr), sr.seed, lds, lane);
  else inv_lane_tile<D, G, ROT, false>(ct, st, yt, rows, tb, 0, lane_seed(sr, row0, rows, lane), lds, lane);
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


template <int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void fwd_pair_kernel(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                                      uint8_t* __restrict__ scales, uint32_t n, SeedRule sr, SignTable tb) {
  constexpr int D = 256, CPR = 32, LROW = CPR + 1;
  __shared__ uint4 lds[32 * LROW];
  const int lane = threadIdx.x;
  const int p = lane >> 5, v = lane & 31;
  const uint32_t kpos = lane & 31;
  const float sigma = p ? -1.0f : 1.0f;
  {
    const uint32_t row0 = blockIdx.x * 32u;
    const int rows = (int)(n - row0 < 32u ? n - row0 : 32u);
    const uint32_t b0 = seed_block(row0, sr), b1 = seed_block(row0 + (uint32_t)(rows - 1), sr);
    const bool uniform = b0 == b1;
    uint4 cm = make_uint4(0, 0, 0, 0);
    if (uniform) cm = chunk_masks(tb, seed_offset(b0, sr), sr.seed, kpos);
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
        put(rl, xor4(q, chunk_sign_masks(seed_of_block(seed_block(row0 + rl, sr), sr), kpos)));
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
    if constexpr (ROT == kSRFT) {
      float fr[65], fi[65];
      rdft<128, 1, 0, 64>(h, fr, fi);  // unnormalized; sqrt(2/256) is applied by the quantizer
      // Partner exchange by ds_bpermute.  Every 4 bins the next addresses are
      // tied to the last result, so each group of shuffles issues only once
      // the previous group has been consumed; this keeps the exchange from
      // holding all 260 shuffled values at once (register pressure).
      int addr_e = v * 4, addr_o = (v + 32) * 4;
      auto shf = [](float x, int addr) { return __int_as_float(__builtin_amdgcn_ds_bpermute(addr, __float_as_int(x))); };
      // slot 0: E_0 + sigma * O_0 (real)
      {
        const float e0 = shf(fr[0], addr_e), o0 = shf(fr[0], addr_o);
        constexpr float r2 = 0.70710678118654752440f;  // real end bins: 1/16 = sqrt(2/256) / sqrt(2)
        L[0] = __builtin_fmaf(sigma, o0, e0) * r2;
      }
      sfor<63>([&](auto A) {
        constexpr int a = RTQ_CI(A) + 1;
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
      });
      {  // slot 64: X_64 = E_64 - i O_64; lane 0 keeps Re, lane 1 keeps Im
        const float e64 = shf(fr[64], addr_e), o64 = shf(fr[64], addr_o);
        L[127] = p ? -o64 : e64;
      }
      zs = SrftScale<256>::value;
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
      const size_t row = (size_t)row0 + v;
      sfor<4>([&](auto C) {
        stream_store(codes + (row * 8 + 4 * p + RTQ_CI(C)),
                     make_uint4(cw[4 * RTQ_CI(C)], cw[4 * RTQ_CI(C) + 1], cw[4 * RTQ_CI(C) + 2], cw[4 * RTQ_CI(C) + 3]));
      });
      // this lane's half of the row's scales: 128/G values
      if constexpr (128 / G == 1) {
        stream_store(reinterpret_cast<uint16_t*>(scales) + (row * 2 + p), (uint16_t)sb[0]);
      } else if constexpr (128 / G == 2) {
        stream_store(reinterpret_cast<uint32_t*>(scales) + (row * 2 + p), sb[0] | (sb[1] << 16));
      } else {
        stream_store(reinterpret_cast<uint2*>(scales) + (row * 2 + p), make_uint2(sb[0] | (sb[1] << 16), sb[2] | (sb[3] << 16)));
      }
    }
  }
}

template <int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void inv_pair_kernel(const uint4* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, uint4* __restrict__ y,
                                                      uint32_t n, SeedRule sr, SignTable tb) {
  constexpr int CPR = 32;
  __shared__ uint4 lds[32 * 17];
  const int lane = threadIdx.x;
  const int p = lane >> 5, v = lane & 31;
  const uint32_t kpos = lane & 31;
  const float sigma = p ? -1.0f : 1.0f;
  {
    const uint32_t row0 = blockIdx.x * 32u;
    const int rows = (int)(n - row0 < 32u ? n - row0 : 32u);
    const uint32_t b0 = seed_block(row0, sr), b1 = seed_block(row0 + (uint32_t)(rows - 1), sr);
    const bool uniform = b0 == b1;
    uint32_t cw[16], sb[128 / G];
    {
      const size_t row = (size_t)row0 + (v < rows ? v : 0);
      sfor<4>([&](auto C) {
        const uint4 q = stream_load(codes + (row * 8 + 4 * p + RTQ_CI(C)));
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
      // lane 1 holds its half in mirrored order: undo on the packed form
      uint32_t rev[16];
      sfor<16>([&](auto W) { rev[RTQ_CI(W)] = nibble_reverse(cw[15 - RTQ_CI(W)]); });
      sfor<16>([&](auto W) { cw[RTQ_CI(W)] = p ? rev[RTQ_CI(W)] : cw[RTQ_CI(W)]; });
      uint32_t sr[128 / G];
      sfor<128 / G>([&](auto W) { sr[RTQ_CI(W)] = sb[128 / G - 1 - RTQ_CI(W)]; });
      sfor<128 / G>([&](auto W) { sb[RTQ_CI(W)] = p ? sr[RTQ_CI(W)] : sb[RTQ_CI(W)]; });
      float L[128];
      dequant_unpack<128, G>(cw, sb, 0.5f, L);  // the halving of E and t folded in
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
      dequant_unpack<128, G>(cw, sb, 1.0f / 16.0f, f);
      fwht_f32<128>(f);
      sfor<128>([&](auto K) {
        const float r = __shfl_xor(f[RTQ_CI(K)], 32);
        u[RTQ_CI(K)] = __builtin_fmaf(sigma, f[RTQ_CI(K)], r);
      });
    }
    // fp16 samples out through LDS in two passes of 16 output chunks per row
    // (a 9 KB tile).  SRFT: lane p's samples are u_{2m+p}; pass ph takes its
    // 64 samples 64 ph .. 64 ph + 63 into the p-th half of the LDS row and
    // re-interleaves them on the way out.  SRHT: lane p holds output chunks
    // 16 p .. 16 p + 15, written in pass p.
    constexpr int LR2 = 17;
    const int kk = lane & 15, rsub = lane >> 4;
    uint4* yt = y + (size_t)row0 * CPR;
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
        const uint4 m = chunk_masks(tb, seed_offset(b0, sr), sr.seed, k);
        sfor<8>([&](auto J) {
          const int rl = rsub + 4 * RTQ_CI(J);
          if (rl < rows) stream_store(yt + ((uint32_t)(rl * CPR) + k), xor4(get(rl), m));
        });
      } else {
#pragma unroll 1
        for (int j = 0; j < 8; ++j) {
          const int rl = rsub + 4 * j;
          if (rl < rows)
            stream_store(yt + ((uint32_t)(rl * CPR) + k),
                         xor4(get(rl), chunk_sign_masks(seed_of_block(seed_block(row0 + rl, sr), sr), k)));
        }
      }
    });
    wait_lds_reads();
    lds_sync();
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Sign words of the seeds a call uses (as many as the table holds).  The
// table is a pure function of (seed, d, number of seeds); the last one built
// on each host thread is kept to skip recomputing it for repeated calls.
void fill_sign_table(SignTable& tb, const SeedRule& sr, int64_t n, int d) {
  const uint32_t wps = (uint32_t)d / 64u;
  uint64_t distinct = 1;
  if (sr.rps) {
    const uint64_t blocks = ((uint64_t)n + sr.rps - 1) / sr.rps;
    distinct = sr.period && sr.period < blocks ? sr.period : blocks;
  }
  const uint32_t seeds = (uint32_t)(distinct < kSignTableWords / wps ? distinct : kSignTableWords / wps);
  thread_local SignTable memo;
  thread_local uint64_t memo_seed = 0;
  thread_local bool memo_valid = false;
  if (memo_valid && memo_seed == sr.seed && memo.words_per_seed == wps && memo.seeds >= seeds) {
    tb = memo;
    tb.seeds = seeds;
    return;
  }
  tb.seeds = seeds;
  tb.words_per_seed = wps;
  for (uint32_t j = 0; j < kSignTableWords; ++j) tb.w[j] = 0;
  for (uint32_t j = 0; j < seeds; ++j)
    for (uint32_t q = 0; q < wps; ++q) {
      uint64_t w = 0;
      for (uint32_t e = 0; e < 64; ++e) w |= (uint64_t)sign_bit(sr.seed + j, 64u * q + e) << e;
      tb.w[j * wps + q] = w;
    }
  memo = tb;
  memo_seed = sr.seed;
  memo_valid = true;
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

rtq_status run(bool fwd, int rot, const void* in0, const void* in1, void* out0, void* out1, int64_t n, int32_t d,
               int32_t g, uint64_t seed, int64_t rps, int32_t period, hipStream_t stream) {
  if (n < 0 || rps < 0 || period < 0) return RTQ_ERR_INVALID_ARG;
  const rtq_status shape = check_shape(d, g);
  if (shape != RTQ_OK) return shape;
  if (n == 0) return RTQ_OK;
  if (n > kMaxRows) return RTQ_ERR_INVALID_ARG;
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
  uint32_t n32 = (uint32_t)n;
  SeedRule sr = make_seed_rule(seed, rps, period, n);
  SignTable tb;
  fill_sign_table(tb, sr, n, d);
  if (fwd) {
    const void* x = in0;
    void* codes = out0;
    void* scales = out1;
    void* kargs[] = {&x, &codes, &scales, &n32, &sr, &tb};
    return launch(fn, tiles, kargs, stream);
  }
  const void* codes = in0;
  const void* scales = in1;
  void* y = out0;
  void* kargs[] = {&codes, &scales, &y, &n32, &sr, &tb};
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

