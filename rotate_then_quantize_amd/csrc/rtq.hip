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
#include "rtq_pair.hpp"

namespace rtq {

// ---------------------------------------------------------------------------
// d = 64 / 128: one lane per vector, 64 vectors per tile.
// ---------------------------------------------------------------------------

// One forward tile: rows row0 .. row0 + rows - 1, lane l owning row row0 + l.
// kUniform: every row has seed s (masks are scalar); otherwise s is the
// lane's own seed.  LAM: each channel i is first multiplied by lam_i (d fp16
// values, a per-channel scale), as in the width-and-lambda entry points.
template <int D, int G, int ROT, bool kUniform, bool LAM = false>
__device__ __forceinline__ void fwd_lane_tile(const uint4* __restrict__ xt, uint4* __restrict__ ct,
                                              uint8_t* __restrict__ st, int rows, const SignTable& tb,
                                              uint32_t j, uint64_t s, uint4* buf, int lane,
                                              const uint32_t* __restrict__ lam = nullptr) {
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
  if constexpr (LAM) quantize_row_lambda<D, G, ROT>(h, lam, cw, sb);
  else quantize_row<D, G, ROT>(h, cw, sb);
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

// The forward step with a per-channel lambda (the plain kernel below writes
// the same steps out without it).
template <int D, int G, int ROT, bool LAM>
__device__ __forceinline__ void fwd_lane_body(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                              uint8_t* __restrict__ scales, const uint32_t* __restrict__ lam,
                                              uint32_t n, const SeedRule& sr, const SignTable& tb) {
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
  if (b0 == b1)
    fwd_lane_tile<D, G, ROT, true, LAM>(xt, ct, st, rows, tb, seed_offset(b0, sr), sr.seed, buf, lane, lam);
  else
    fwd_lane_tile<D, G, ROT, false, LAM>(xt, ct, st, rows, tb, 0, lane_seed(sr, row0, rows, lane), buf, lane, lam);
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

// The same with a per-channel lambda (4-bit codes of the width-and-lambda
// entry points).  Two waves per SIMD, the most a 16 KB tile leaves room for
// at d = 128, and a register budget (256) that keeps them.
template <int D, int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void fwd_lane_lambda_kernel(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                                             uint8_t* __restrict__ scales,
                                                             const uint32_t* __restrict__ lam, uint32_t n, SeedRule sr,
                                                             SignTable tb) {
  fwd_lane_body<D, G, ROT, true>(x, codes, scales, lam, n, sr, tb);
}

// Chunk k of code row r sits at slot r * CW + (k ^ code_swizzle<CW>(r)) of
// the staged code block: the 16 lanes of one LDS access, reading chunk k of
// rows r .. r + 15, then hit 16 different groups of 4 banks (without the xor
// the rows 16 / CW apart share a group).
template <int CW>
__device__ __forceinline__ int code_swizzle(int r) {
  static_assert(CW == 2 || CW == 4, "code chunks per row");
  return (r >> (CW == 4 ? 2 : 3)) & (CW - 1);
}

// Direct-to-LDS staging of a tile's code block (CW 16-byte chunks per row, in
// row order, swizzled as above): load instruction j of lane i fills slot
// 64j + i, a partial tile repeating its last row.
template <int CW>
__device__ __forceinline__ void load_codes_to_lds(const uint4* __restrict__ ct, int rows, uint4* buf, int lane) {
  sfor<CW>([&](auto J) {
    const int c = RTQ_CI(J) * 64 + lane;
    const int r = c / CW;
    const int rr = r < rows ? r : rows - 1;
    const uint32_t off = (uint32_t)(rr * CW + ((c % CW) ^ code_swizzle<CW>(r))) * 16u;
    __builtin_amdgcn_global_load_lds((gbl_void_t*)((const char*)ct + off), (lds_void_t*)(buf + RTQ_CI(J) * 64), 16,
                                     0, kCachePolicyNT);
  });
}

// One inverse tile: rows row0 .. row0 + rows - 1, lane l owning row row0 + l.
// The code block arrives coalesced in LDS, each lane reads its own row, and
// the fp16 output leaves through the same LDS buffer (padded rows) as
// coalesced 16-byte stores.
template <int D, int G, int ROT, bool kUniform, bool LAM = false>
__device__ __forceinline__ void inv_lane_tile(const uint4* __restrict__ ct, const uint8_t* __restrict__ st,
                                              uint4* __restrict__ yt, int rows, const SignTable& tb, uint32_t j,
                                              uint64_t s, uint4* lds, int lane,
                                              const uint32_t* __restrict__ lam = nullptr, float* inv_lam = nullptr) {
  constexpr int CPR = D / 8;
  constexpr int CW = D / 32;
  const uint32_t r = (uint32_t)(lane < rows ? lane : rows - 1);
  load_codes_to_lds<CW>(ct, rows, lds, lane);
  if constexpr (LAM) lambda_reciprocals<D>(lam, inv_lam, lane);  // read after the barrier below
  uint32_t sb[D / G];
  load_row_scales<D, G>(st, r, sb);
  UniformSigns<D> sg;
  if constexpr (kUniform) sg.setup(tb, j, s, lane);  // overlaps the loads
  wait_vmcnt<0>();
  lds_sync();
  uint32_t cw[D / 8];
  sfor<CW>([&](auto C) {
    const uint4 q = lds[r * CW + (RTQ_CI(C) ^ code_swizzle<CW>((int)r))];
    cw[4 * RTQ_CI(C) + 0] = q.x;
    cw[4 * RTQ_CI(C) + 1] = q.y;
    cw[4 * RTQ_CI(C) + 2] = q.z;
    cw[4 * RTQ_CI(C) + 3] = q.w;
  });
  uint32_t h[D / 2];
  if constexpr (ROT == kSRFT && !LAM) {
    float z[D];
    dequant_unpack<D, G>(cw, sb, HartleyIn<D>::value, z);
    srft_inv_hartley_packed<D>(z, h);
  } else {
    float z[D], u[D];
    if constexpr (ROT == kSRFT) {
      dequant_unpack<D, G>(cw, sb, HartleyIn<D>::value, z);
      srft_inv_hartley<D>(z, u);
    } else {
      dequant_unpack<D, G>(cw, sb, InvSqrt<D>::value, u);
      fwht_f32<D>(u);
    }
    if constexpr (LAM) lambda_unweight_lds<D>(u, inv_lam);  // the per-channel lambda divided out
    sfor<D / 2>([&](auto M) { h[RTQ_CI(M)] = pack_f16x2(u[2 * RTQ_CI(M)], u[2 * RTQ_CI(M) + 1]); });
  }
  if constexpr (kUniform) sg.apply(h);
  else apply_lane_signs<D>(h, s);
  // Own row into LDS (the code block has been read), then coalesced chunks
  // out.  d = 128 goes in two passes of 32 whole rows (a 9 KB LDS tile, so
  // that LDS does not cap the resident waves): in pass ph the lanes of rows
  // 32 ph .. 32 ph + 31 write their rows, and each store instruction then
  // writes four whole rows (1 KB of contiguous output).
  wait_lds_reads();
  lds_sync();
  constexpr int PH = InvPhases<D>::value;
  constexpr int RP = 64 / PH, LR = CPR + 1;  // rows per pass, LDS row stride (uint4)
  sfor<PH>([&](auto P) {
    constexpr int ph = RTQ_CI(P);
    if constexpr (ph > 0) {
      wait_lds_reads();
      lds_sync();
    }
    if (PH == 1 || lane / RP == ph) {
      sfor<CPR>([&](auto C) {
        constexpr int c = RTQ_CI(C);
        lds[(lane % RP) * LR + c] = make_uint4(h[4 * c], h[4 * c + 1], h[4 * c + 2], h[4 * c + 3]);
      });
    }
    lds_sync();
    auto out = [&](auto J) {
      const int idx = RTQ_CI(J) * 64 + lane;
      const int rl = idx / CPR, kk = idx % CPR;  // row of this pass, chunk
      return stream_store(yt + (uint32_t)((RP * ph + rl) * CPR + kk), lds[rl * LR + kk]);
    };
    constexpr int NJ = RP * CPR / 64;  // store instructions per pass
    if (rows == 64) {  // a full tile stores without per-row guards
      sfor<NJ>([&](auto J) { out(J); });
    } else {
      sfor<NJ>([&](auto J) {
        if (RP * ph + (RTQ_CI(J) * 64 + lane) / CPR < rows) out(J);
      });
    }
  });
}

// The inverse step with a per-channel lambda (the plain kernel below writes
// the same steps out without it).
template <int D, int G, int ROT, bool LAM>
__device__ __forceinline__ void inv_lane_body(const uint4* __restrict__ codes, const uint8_t* __restrict__ scales,
                                              uint4* __restrict__ y, const uint32_t* __restrict__ lam, uint32_t n,
                                              const SeedRule& sr, const SignTable& tb) {
  constexpr int CPR = D / 8;
  constexpr int CW = D / 32;
  constexpr int LT = 64 / InvPhases<D>::value * (CPR + 1);  // output tile (uint4)
  __shared__ uint4 lds[LT > 64 * CW ? LT : 64 * CW];
  __shared__ __attribute__((aligned(16))) float inv_lam[D];  // 1 / lambda per channel
  const int lane = threadIdx.x;
  const uint32_t row0 = blockIdx.x * 64u;
  const int rows = (int)(n - row0 < 64u ? n - row0 : 64u);
  const uint4* ct = codes + (size_t)row0 * CW;
  const uint8_t* st = scales + (size_t)row0 * (2 * D / G);
  uint4* yt = y + (size_t)row0 * CPR;
  const uint32_t b0 = seed_block(row0, sr), b1 = seed_block(row0 + (uint32_t)(rows - 1), sr);
  if (b0 == b1)
    inv_lane_tile<D, G, ROT, true, LAM>(ct, st, yt, rows, tb, seed_offset(b0, sr), sr.seed, lds, lane, lam, inv_lam);
  else
    inv_lane_tile<D, G, ROT, false, LAM>(ct, st, yt, rows, tb, 0, lane_seed(sr, row0, rows, lane), lds, lane, lam,
                                         inv_lam);
}

// Inverse step, one 64-row tile per wave.  At most 168 VGPRs (3 waves per
// SIMD): d = 128 then spills a little, and still runs 5% faster than at 2.
template <int D, int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void inv_lane_kernel(
    const uint4* __restrict__ codes, const uint8_t* __restrict__ scales, uint4* __restrict__ y, uint32_t n,
    SeedRule sr, SignTable tb) {
  constexpr int CPR = D / 8;
  constexpr int CW = D / 32;
  constexpr int LT = 64 / InvPhases<D>::value * (CPR + 1);  // output tile (uint4)
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

// The same with a per-channel lambda (4-bit codes of the width-and-lambda
// entry points).
template <int D, int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void inv_lane_lambda_kernel(
    const uint4* __restrict__ codes, const uint8_t* __restrict__ scales, uint4* __restrict__ y,
    const uint32_t* __restrict__ lam, uint32_t n, SeedRule sr, SignTable tb) {
  inv_lane_body<D, G, ROT, true>(codes, scales, y, lam, n, sr, tb);
}

// ---------------------------------------------------------------------------
// d = 256: two lanes per vector, 32 vectors per tile (rtq_pair.hpp), over the
// rows of a contiguous [n, 256] tensor.
// ---------------------------------------------------------------------------

// Three waves per SIMD (at most 168 VGPRs): every group size fits without
// spills.
template <int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void fwd_pair_kernel(
    const uint4* __restrict__ x, uint4* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t n, SeedRule sr,
    SignTable tb) {
  __shared__ uint4 lds[16 * 33];
  fwd_pair_tile<G, ROT>(x, codes, scales, tile_rows(n, sr, tb), lds, threadIdx.x);
}

// Three waves per SIMD (at most 168 VGPRs): both rotations fit without
// spills.
template <int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void inv_pair_kernel(
    const uint4* __restrict__ codes, const uint8_t* __restrict__ scales, uint4* __restrict__ y, uint32_t n,
    SeedRule sr, SignTable tb) {
  __shared__ uint4 lds[32 * 17];
  inv_pair_tile<G, ROT>(codes, scales, y, tile_rows(n, sr, tb), lds, threadIdx.x);
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
  RTQ_CASE(256, 32) RTQ_CASE(256, 64) RTQ_CASE(256, 128) RTQ_CASE(256, 256)
#undef RTQ_CASE
  return nullptr;
}

// The 4-bit lambda kernels (one lane per row), for the width-and-lambda
// entry points: null for d = 256 or an unsupported group, and for the d = 128
// inverse, which spills about 1 KB per lane at three waves per SIMD (the
// general kernel fits two waves without spills).
KernelFn find_lane_lambda_kernel(bool fwd, int rot, int d, int g) {
#define RTQ_LAM(KERNEL, DD, GG)                                                      \
  if (d == DD && g == GG)                                                            \
    return rot == kSRFT ? reinterpret_cast<KernelFn>(&KERNEL<DD, GG, kSRFT>)         \
                        : reinterpret_cast<KernelFn>(&KERNEL<DD, GG, kSRHT>);
  if (fwd) {
    RTQ_LAM(fwd_lane_lambda_kernel, 64, 32) RTQ_LAM(fwd_lane_lambda_kernel, 64, 64)
    RTQ_LAM(fwd_lane_lambda_kernel, 128, 32) RTQ_LAM(fwd_lane_lambda_kernel, 128, 64)
    RTQ_LAM(fwd_lane_lambda_kernel, 128, 128)
  } else {
    RTQ_LAM(inv_lane_lambda_kernel, 64, 32) RTQ_LAM(inv_lane_lambda_kernel, 64, 64)
  }
#undef RTQ_LAM
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

