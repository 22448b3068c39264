// rtq_ext.hip -- forward and inverse with 3-, 4-, 6- or 8-bit codes and an
// optional per-channel lambda (d = 64 / 128 / 256), and their C ABI entry
// points (include/rtq.h).
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
// Other code widths (3, 4, 6, 8 bits) and a per-channel lambda (d = 64 / 128)
// ("Quantization Speed Is Often a Kernel Problem", "First, the 17%": the
// fused recipe adds one scale per channel to the per-group absmax, and the
// quality study runs 3- to 8-bit codes).  lambda multiplies each channel
// before the sign flip and is divided out after the inverse rotation; B-bit
// codes fill one little-endian bit stream per row.  One lane per row, 64 rows
// per wave; tiles move through LDS as in the int4 kernels.
// ---------------------------------------------------------------------------

template <int D, int G, int ROT, int B>
__global__ __launch_bounds__(64) void fwd_ext_kernel(const uint4* __restrict__ x, uint32_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, const uint32_t* __restrict__ lam,
                                                     uint32_t n, SeedRule sr) {
  constexpr int CPR = D / 8;
  constexpr int CWW = D * B / 32;  // code words per row
  static_assert(CWW <= 4 * CPR, "the code tile fits the input tile");
  __shared__ uint4 buf[64 * CPR];
  const int lane = threadIdx.x;
  const uint32_t row0 = blockIdx.x * 64u;
  const int rows = (int)(n - row0 < 64u ? n - row0 : 64u);
  load_tile_to_lds<CPR>(x + (size_t)row0 * CPR, rows, buf, lane);
  const uint64_t s = lane_seed(sr, row0, rows, lane);
  wait_vmcnt<0>();
  lds_sync();
  uint32_t h[D / 2];
  read_own_row<CPR>(buf, lane, h);
  flip_signs<D>(h, s, lane);
  float z[D];
  float zs;
  if (lam != nullptr) {
    float u[D];
    lambda_weight<D>(h, lam, u);
    if constexpr (ROT == kSRFT) {
      srft_fwd<D>(u, z);
      zs = 1.0f;
    } else {
      fwht_f32<D>(u);
      sfor<D>([&](auto I) { z[RTQ_CI(I)] = u[RTQ_CI(I)]; });
      zs = InvSqrt<D>::value;
    }
  } else if constexpr (ROT == kSRFT) {
    srft_fwd_unscaled<D>(h, z);
    zs = SrftScale<D>::value;
  } else {
    fwht_from_f16<D>(h, z);
    zs = InvSqrt<D>::value;
  }
  uint32_t cw[CWW], sb[D / G];
  quantize_pack_bits<D, G, B>(z, zs, cw, sb);
  // code words out through LDS (the input tile is no longer needed), as
  // coalesced 4-byte stores of the tile's contiguous code block
  uint32_t* lw = reinterpret_cast<uint32_t*>(buf);
  lds_sync();
  sfor<CWW>([&](auto K) { lw[lane * CWW + RTQ_CI(K)] = cw[RTQ_CI(K)]; });
  lds_sync();
  const int total = rows * CWW;
  uint32_t* ct = codes + (size_t)row0 * CWW;
  sfor<CWW>([&](auto J) {
    const int idx = RTQ_CI(J) * 64 + lane;
    if (idx < total) stream_store(ct + idx, lw[idx]);
  });
  if (lane < rows) store_row_scales<D, G>(scales + (size_t)row0 * (2 * D / G), (uint32_t)lane, sb);
}

template <int D, int G, int ROT, int B>
__global__ __launch_bounds__(64) void inv_ext_kernel(const uint32_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, uint4* __restrict__ y,
                                                     const uint32_t* __restrict__ lam, uint32_t n, SeedRule sr) {
  constexpr int CPR = D / 8;
  constexpr int CWW = D * B / 32;
  constexpr int PH = InvPhases<D>::value;
  constexpr int PC = CPR / PH, LR = PC + 1;
  constexpr int LT = 64 * LR;  // output staging (uint4)
  __shared__ uint4 lds[LT > 16 * CWW ? LT : 16 * CWW];
  __shared__ __attribute__((aligned(16))) float inv_lam[D];  // 1 / lambda per channel
  uint32_t* lw = reinterpret_cast<uint32_t*>(lds);
  const int lane = threadIdx.x;
  const uint32_t row0 = blockIdx.x * 64u;
  const int rows = (int)(n - row0 < 64u ? n - row0 : 64u);
  const uint32_t r = (uint32_t)(lane < rows ? lane : rows - 1);
  // the tile's code block, coalesced 4-byte loads into LDS
  const int total = rows * CWW;
  const uint32_t* ct = codes + (size_t)row0 * CWW;
  sfor<CWW>([&](auto J) {
    const int idx = RTQ_CI(J) * 64 + lane;
    lw[idx] = stream_load(ct + (idx < total ? idx : total - 1));
  });
  uint32_t sb[D / G];
  load_row_scales<D, G>(scales + (size_t)row0 * (2 * D / G), r, sb);
  const uint64_t s = lane_seed(sr, row0, rows, lane);
  if (lam != nullptr) lambda_reciprocals<D>(lam, inv_lam, lane);  // read after the barrier below
  wait_lds_reads();
  lds_sync();
  uint32_t cw[CWW];
  sfor<CWW>([&](auto K) { cw[RTQ_CI(K)] = lw[r * CWW + RTQ_CI(K)]; });
  float z[D], u[D];
  if constexpr (ROT == kSRFT) {
    dequant_unpack_bits<D, G, B>(cw, sb, HartleyIn<D>::value, z);
    srft_inv_hartley<D>(z, u);
  } else {
    dequant_unpack_bits<D, G, B>(cw, sb, InvSqrt<D>::value, u);
    fwht_f32<D>(u);
  }
  if (lam != nullptr) lambda_unweight_lds<D>(u, inv_lam);
  uint32_t h[D / 2];
  sfor<D / 2>([&](auto M) { h[RTQ_CI(M)] = pack_f16x2(u[2 * RTQ_CI(M)], u[2 * RTQ_CI(M) + 1]); });
  flip_signs<D>(h, s, lane);
  // own row into LDS (the code block has been read), then coalesced chunks out
  wait_lds_reads();
  lds_sync();
  uint4* yt = y + (size_t)row0 * CPR;
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

// d = 256: the two-lanes-per-vector tiles of rtq_pair.hpp with B-bit codes
// and the lambda, over a contiguous [n, 256] tensor.
template <int G, int ROT, int B>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 8))) void fwd_ext_pair_kernel(
    const uint4* __restrict__ x, uint4* __restrict__ codes, uint8_t* __restrict__ scales,
    const uint32_t* __restrict__ lam, uint32_t n, SeedRule sr, SignTable tb) {
  __shared__ uint4 lds[16 * 33];
  fwd_pair_tile<G, ROT, TileRows, B>(x, codes, scales, tile_rows(n, sr, tb), lds, threadIdx.x, lam);
}

// Three waves per SIMD, one kernel per lambda case (inv_pair_tile's LAM).
template <int G, int ROT, int B, bool LAM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void inv_ext_pair_kernel(
    const uint4* __restrict__ codes, const uint8_t* __restrict__ scales, uint4* __restrict__ y,
    const uint32_t* __restrict__ lam, uint32_t n, SeedRule sr, SignTable tb) {
  __shared__ uint4 lds[32 * 17];
  __shared__ __attribute__((aligned(16))) float inv_lam[LAM ? kPairLambdaFloats : 2];
  inv_pair_tile<G, ROT, TileRows, B, LAM>(codes, scales, y, tile_rows(n, sr, tb), lds, threadIdx.x, lam, inv_lam);
}

template <int ROT, int B>
KernelFn find_ext_bits(bool fwd, int d, int g, bool lam) {
#define RTQ_EXT_CASE(DD, GG)                                                           \
  if (d == DD && g == GG)                                                              \
    return fwd ? reinterpret_cast<KernelFn>(&fwd_ext_kernel<DD, GG, ROT, B>)           \
               : reinterpret_cast<KernelFn>(&inv_ext_kernel<DD, GG, ROT, B>);
  RTQ_EXT_CASE(64, 32) RTQ_EXT_CASE(64, 64)
  RTQ_EXT_CASE(128, 32) RTQ_EXT_CASE(128, 64) RTQ_EXT_CASE(128, 128)
#undef RTQ_EXT_CASE
#define RTQ_EXT_PAIR_CASE(GG)                                                          \
  if (d == 256 && g == GG)                                                             \
    return fwd ? reinterpret_cast<KernelFn>(&fwd_ext_pair_kernel<GG, ROT, B>)          \
           : lam ? reinterpret_cast<KernelFn>(&inv_ext_pair_kernel<GG, ROT, B, true>)  \
                 : reinterpret_cast<KernelFn>(&inv_ext_pair_kernel<GG, ROT, B, false>);
  RTQ_EXT_PAIR_CASE(32) RTQ_EXT_PAIR_CASE(64) RTQ_EXT_PAIR_CASE(128) RTQ_EXT_PAIR_CASE(256)
#undef RTQ_EXT_PAIR_CASE
  return nullptr;
}

template <int ROT>
KernelFn find_ext(bool fwd, int d, int g, int bits, bool lam) {
  switch (bits) {
    case 3: return find_ext_bits<ROT, 3>(fwd, d, g, lam);
    case 4: return find_ext_bits<ROT, 4>(fwd, d, g, lam);
    case 6: return find_ext_bits<ROT, 6>(fwd, d, g, lam);
    case 8: return find_ext_bits<ROT, 8>(fwd, d, g, lam);
    default: return nullptr;
  }
}

// Forward (in0 = x, out0 = codes, out1 = scales) or inverse (in0 = codes,
// in1 = scales, out0 = y) with `bits`-bit codes and an optional lambda.
rtq_status run_ext(bool fwd, int rot, const void* in0, const void* in1, void* out0, void* out1, const void* lam,
                   int64_t n, int32_t d, int32_t g, int32_t bits, uint64_t seed, int64_t rps, int32_t period,
                   hipStream_t stream) {
  if (n < 0 || rps < 0 || period < 0) return RTQ_ERR_INVALID_ARG;
  const rtq_status shape = check_shape(d, g);
  if (shape != RTQ_OK) return shape;
  KernelFn fn = rot == kSRFT ? find_ext<kSRFT>(fwd, d, g, bits, lam != nullptr)
                              : find_ext<kSRHT>(fwd, d, g, bits, lam != nullptr);
  if (!fn) return RTQ_ERR_UNSUPPORTED;
  // 4 bits with lambda below d = 256: the int4 tiles with the lambda multiply
  // (16-byte code moves, the int4 packer), which write the same bytes
  const KernelFn lane_lambda = bits == 4 && lam ? find_lane_lambda_kernel(fwd, rot, d, g) : nullptr;
  if (lane_lambda) fn = lane_lambda;
  if (n == 0) return RTQ_OK;
  if (n > kMaxRows) return RTQ_ERR_INVALID_ARG;
  const void* a = in0;
  const void* b = fwd ? out0 : in1;
  const void* c = fwd ? out1 : out0;
  if (!a || !b || !c || !aligned16(a) || !aligned16(b) || !aligned16(c)) return RTQ_ERR_INVALID_ARG;
  if (lam && !aligned16(lam)) return RTQ_ERR_INVALID_ARG;
  const int64_t fp16_bytes = n * 2 * d, code_bytes = n * d * bits / 8, scale_bytes = n * 2 * (d / g);
  if (fwd) {
    if (ranges_overlap(in0, fp16_bytes, out0, code_bytes) || ranges_overlap(in0, fp16_bytes, out1, scale_bytes) ||
        ranges_overlap(out0, code_bytes, out1, scale_bytes) || (lam && ranges_overlap(lam, 2 * d, out0, code_bytes)) ||
        (lam && ranges_overlap(lam, 2 * d, out1, scale_bytes)))
      return RTQ_ERR_INVALID_ARG;
  } else {
    if (ranges_overlap(out0, fp16_bytes, in0, code_bytes) || ranges_overlap(out0, fp16_bytes, in1, scale_bytes) ||
        (lam && ranges_overlap(lam, 2 * d, out0, fp16_bytes)))
      return RTQ_ERR_INVALID_ARG;
  }
  uint32_t n32 = (uint32_t)n;
  SeedRule sr = make_seed_rule(seed, rps, period, n);
  const uint32_t* l = static_cast<const uint32_t*>(lam);
  const int vpt = d == 256 ? 32 : 64;  // rows per tile
  const int64_t tiles = (n + vpt - 1) / vpt;
  SignTable tb;  // the d = 256 and lane-lambda kernels take the sign table as a last argument
  if (d == 256 || lane_lambda) fill_sign_table(tb, sr, n, d);
  if (fwd) {
    const void* x = in0;
    void* codes = out0;
    void* scales = out1;
    void* kargs[] = {&x, &codes, &scales, &l, &n32, &sr, &tb};
    return launch(fn, tiles, kargs, stream);
  }
  const void* codes = in0;
  const void* scales = in1;
  void* y = out0;
  void* kargs[] = {&codes, &scales, &y, &l, &n32, &sr, &tb};
  return launch(fn, tiles, kargs, stream);
}

}  // namespace rtq

#define RTQ_API extern "C" __attribute__((visibility("default")))

RTQ_API rtq_status srft_quant_fwd_ext(const void* x_f16, void* codes_u8, void* scales_f16, int64_t n, int32_t d,
                                      int32_t group, int32_t bits, const void* lambda_f16, uint64_t seed,
                                      int64_t rows_per_seed, int32_t seed_period, hipStream_t stream) {
  return rtq::run_ext(true, rtq::kSRFT, x_f16, nullptr, codes_u8, scales_f16, lambda_f16, n, d, group, bits, seed,
                      rows_per_seed, seed_period, stream);
}

RTQ_API rtq_status srht_quant_fwd_ext(const void* x_f16, void* codes_u8, void* scales_f16, int64_t n, int32_t d,
                                      int32_t group, int32_t bits, const void* lambda_f16, uint64_t seed,
                                      int64_t rows_per_seed, int32_t seed_period, hipStream_t stream) {
  return rtq::run_ext(true, rtq::kSRHT, x_f16, nullptr, codes_u8, scales_f16, lambda_f16, n, d, group, bits, seed,
                      rows_per_seed, seed_period, stream);
}

RTQ_API rtq_status srft_dequant_inv_ext(const void* codes_u8, const void* scales_f16, void* y_f16, int64_t n,
                                        int32_t d, int32_t group, int32_t bits, const void* lambda_f16,
                                        uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                        hipStream_t stream) {
  return rtq::run_ext(false, rtq::kSRFT, codes_u8, scales_f16, y_f16, nullptr, lambda_f16, n, d, group, bits, seed,
                      rows_per_seed, seed_period, stream);
}

RTQ_API rtq_status srht_dequant_inv_ext(const void* codes_u8, const void* scales_f16, void* y_f16, int64_t n,
                                        int32_t d, int32_t group, int32_t bits, const void* lambda_f16,
                                        uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                        hipStream_t stream) {
  return rtq::run_ext(false, rtq::kSRHT, codes_u8, scales_f16, y_f16, nullptr, lambda_f16, n, d, group, bits, seed,
                      rows_per_seed, seed_period, stream);
}

