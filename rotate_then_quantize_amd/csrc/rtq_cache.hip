// rtq_cache.hip -- the in-place append of new tokens into a strided cache and
// the row-mapped inverse that refreshes a dequantized fp16 copy of the
// cache (d = 64 / 128 / 256), and their C ABI entry points (include/rtq.h).
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
// Cache blocks addressed by strides (d = 64 / 128): the in-place append of new
// tokens and the row-mapped inverse that refreshes a dequantized fp16 mirror
// of the cache ("Quantization Speed Is Often a Kernel Problem", "First, the
// 17%": the dequantized prefix is kept between steps, the newest tokens stay
// in fp16, and the prefix is refreshed when that window fills).  One lane per
// row, 64 rows per wave; each lane reads or writes its own cache row.
// ---------------------------------------------------------------------------

// Row i of a block [layers][2][streams][n] lives at cache row
// l*sl + kv*skv + s*ss + (t0 + j)*st.
struct RowMap {
  int64_t sl, skv, ss, st;
  uint32_t t0, n, streams;
  Div32 by_n, by_streams;
};

__device__ __forceinline__ int64_t map_row(const RowMap& m, uint32_t i) {
  const uint32_t q1 = div32(i, m.by_n), j = i - q1 * m.n;
  const uint32_t q2 = div32(q1, m.by_streams), s = q1 - q2 * m.streams;
  return (int64_t)(q2 >> 1) * m.sl + (int64_t)(q2 & 1u) * m.skv + (int64_t)s * m.ss + (int64_t)(m.t0 + j) * m.st;
}

// The cache's seed rule on 64-bit row indices.
struct RowSeeds {
  uint64_t seed;
  int64_t rps;
  int32_t period;
};

// Quantize rows 0 .. n-1 of x (a contiguous [layers][2][streams][n_tokens][d]
// block) into the cache rows map_row(i).
template <int D, int G, int ROT>
__global__ __launch_bounds__(64) void fwd_mapped_kernel(const uint4* __restrict__ x, uint4* __restrict__ codes,
                                                        uint8_t* __restrict__ scales, uint32_t n, RowMap m,
                                                        RowSeeds rs) {
  constexpr int CPR = D / 8;
  constexpr int CW = D / 32;
  __shared__ uint4 buf[64 * CPR];
  const int lane = threadIdx.x;
  const uint32_t row0 = blockIdx.x * 64u;
  const int rows = (int)(n - row0 < 64u ? n - row0 : 64u);
  load_tile_to_lds<CPR>(x + (size_t)row0 * CPR, rows, buf, lane);
  const int64_t dst = map_row(m, row0 + (uint32_t)(lane < rows ? lane : rows - 1));
  const uint64_t s = row_seed(rs.seed, dst, rs.rps, rs.period);
  wait_vmcnt<0>();
  lds_sync();
  uint32_t h[D / 2];
  read_own_row<CPR>(buf, lane, h);
  flip_signs<D>(h, s, lane);
  uint32_t cw[D / 8], sb[D / G];
  quantize_row<D, G, ROT>(h, cw, sb);
  if (lane < rows) {
    // ordinary (cached) stores: each lane writes its own row in pieces, and
    // L2 merges the pieces of a line before it goes to HBM
    uint4* c = codes + dst * CW;
    sfor<CW>([&](auto C) {
      constexpr int k = RTQ_CI(C);
      c[k] = make_uint4(cw[4 * k], cw[4 * k + 1], cw[4 * k + 2], cw[4 * k + 3]);
    });
    uint8_t* srow = scales + dst * (2 * D / G);
    if constexpr (D / G == 1) {
      *reinterpret_cast<uint16_t*>(srow) = (uint16_t)sb[0];
    } else if constexpr (D / G == 2) {
      *reinterpret_cast<uint32_t*>(srow) = sb[0] | (sb[1] << 16);
    } else {
      *reinterpret_cast<uint2*>(srow) = make_uint2(sb[0] | (sb[1] << 16), sb[2] | (sb[3] << 16));
    }
  }
}

// Dequantize the cache rows map_row(i), i < n, into the same rows of y (an
// fp16 mirror of the cache).
template <int D, int G, int ROT>
__global__ __launch_bounds__(64) void inv_mapped_kernel(const uint4* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales, uint4* __restrict__ y,
                                                        uint32_t n, RowMap m, RowSeeds rs) {
  constexpr int CPR = D / 8;
  constexpr int CW = D / 32;
  const int lane = threadIdx.x;
  const uint32_t row0 = blockIdx.x * 64u;
  const int rows = (int)(n - row0 < 64u ? n - row0 : 64u);
  const int64_t src = map_row(m, row0 + (uint32_t)(lane < rows ? lane : rows - 1));
  uint32_t cw[D / 8], sb[D / G];
  sfor<CW>([&](auto C) {
    constexpr int k = RTQ_CI(C);
    const uint4 q = codes[src * CW + k];
    cw[4 * k] = q.x;
    cw[4 * k + 1] = q.y;
    cw[4 * k + 2] = q.z;
    cw[4 * k + 3] = q.w;
  });
  load_row_scales<D, G>(scales + src * (2 * D / G), 0u, sb);
  const uint64_t s = row_seed(rs.seed, src, rs.rps, rs.period);
  uint32_t h[D / 2];
  if constexpr (ROT == kSRFT) {
    float z[D];
    dequant_unpack<D, G>(cw, sb, HartleyIn<D>::value, z);
    srft_inv_hartley_packed<D>(z, h);
  } else {
    float u[D];
    dequant_unpack<D, G>(cw, sb, InvSqrt<D>::value, u);
    fwht_f32<D>(u);
    sfor<D / 2>([&](auto M) { h[RTQ_CI(M)] = pack_f16x2(u[2 * RTQ_CI(M)], u[2 * RTQ_CI(M) + 1]); });
  }
  flip_signs<D>(h, s, lane);
  if (lane < rows) {
    uint4* out = y + src * CPR;  // ordinary stores, merged per line in L2
    sfor<CPR>([&](auto C) {
      constexpr int k = RTQ_CI(C);
      out[k] = make_uint4(h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]);
    });
  }
}

// d = 256 (two lanes per vector, rtq_pair.hpp): tile row rl is row row0 + rl
// of the block, at cache row map_row(row0 + rl) with that row's own seed.
// The tile counts as uniform when every row's seed is the first row's.
struct MappedTileRows {
  uint32_t row0;
  int rows;
  bool uniform;
  uint64_t seed0;  // seed of the tile's first row
  const RowMap& m;
  const RowSeeds& rs;
  static constexpr bool kStreamStores = false;  // scattered rows: let L2 merge the pieces
  __device__ uint4 uniform_masks(uint32_t k) const { return chunk_sign_masks(seed0, k); }
  __device__ uint4 row_masks(int rl, uint32_t k) const {
    return chunk_sign_masks(row_seed(rs.seed, (int64_t)cache_row(rl), rs.rps, rs.period), k);
  }
  __device__ size_t cache_row(int rl) const { return (size_t)map_row(m, row0 + (uint32_t)rl); }
  __device__ uint4* y_chunk(uint4* y, int rl, uint32_t k) const { return y + cache_row(rl) * 32 + k; }
};

__device__ __forceinline__ MappedTileRows mapped_tile_rows(uint32_t n, const RowMap& m, const RowSeeds& rs) {
  const uint32_t row0 = blockIdx.x * 32u;
  const int rows = (int)(n - row0 < 32u ? n - row0 : 32u);
  const int lane = threadIdx.x & 31;
  const uint64_t s = row_seed(rs.seed, map_row(m, row0 + (uint32_t)(lane < rows ? lane : rows - 1)), rs.rps, rs.period);
  const uint64_t s0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(s >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)s);
  const bool uniform = __ballot(s != s0) == 0;
  return MappedTileRows{row0, rows, uniform, s0, m, rs};
}

// Three waves per SIMD, as the plain forward.
template <int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void fwd_mapped_pair_kernel(
    const uint4* __restrict__ x, uint4* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t n, RowMap m,
    RowSeeds rs) {
  __shared__ uint4 lds[16 * 33];
  fwd_pair_tile<G, ROT>(x, codes, scales, mapped_tile_rows(n, m, rs), lds, threadIdx.x);
}

// Three waves per SIMD, as the plain inverse.
template <int G, int ROT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3, 8))) void inv_mapped_pair_kernel(
    const uint4* __restrict__ codes, const uint8_t* __restrict__ scales, uint4* __restrict__ y, uint32_t n, RowMap m,
    RowSeeds rs) {
  __shared__ uint4 lds[32 * 17];
  inv_pair_tile<G, ROT>(codes, scales, y, mapped_tile_rows(n, m, rs), lds, threadIdx.x);
}

template <int ROT>
KernelFn find_mapped(bool fwd, int d, int g) {
#define RTQ_MAPPED_CASE(DD, GG)                                                        \
  if (d == DD && g == GG)                                                              \
    return fwd ? reinterpret_cast<KernelFn>(&fwd_mapped_kernel<DD, GG, ROT>)           \
               : reinterpret_cast<KernelFn>(&inv_mapped_kernel<DD, GG, ROT>);
  RTQ_MAPPED_CASE(64, 32) RTQ_MAPPED_CASE(64, 64)
  RTQ_MAPPED_CASE(128, 32) RTQ_MAPPED_CASE(128, 64) RTQ_MAPPED_CASE(128, 128)
#undef RTQ_MAPPED_CASE
#define RTQ_MAPPED_PAIR_CASE(GG)                                                       \
  if (d == 256 && g == GG)                                                             \
    return fwd ? reinterpret_cast<KernelFn>(&fwd_mapped_pair_kernel<GG, ROT>)          \
               : reinterpret_cast<KernelFn>(&inv_mapped_pair_kernel<GG, ROT>);
  RTQ_MAPPED_PAIR_CASE(32) RTQ_MAPPED_PAIR_CASE(64) RTQ_MAPPED_PAIR_CASE(128) RTQ_MAPPED_PAIR_CASE(256)
#undef RTQ_MAPPED_PAIR_CASE
  return nullptr;
}

inline bool overlaps128(const void* a, __int128 na, const void* b, __int128 nb) {
  const __int128 a0 = (__int128)(uintptr_t)a, b0 = (__int128)(uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Append (fwd: in0 = x, out0 = codes, out1 = scales) or row-mapped inverse
// (in0 = codes, in1 = scales, out0 = y) over tokens t0 .. t0+ntok-1 of every
// (layer, kv, stream).
rtq_status run_mapped(bool fwd, int rot, const void* in0, const void* in1, void* out0, void* out1, int32_t layers,
                      int32_t streams, int32_t t0, int32_t ntok, int32_t d, int32_t g, const int64_t (&st)[4],
                      uint64_t seed, int64_t rps, int32_t period, hipStream_t stream) {
  if (layers < 0 || streams < 0 || t0 < 0 || ntok < 0 || rps < 0 || period < 0) return RTQ_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (st[i] < 0) return RTQ_ERR_INVALID_ARG;
  const rtq_status shape = check_shape(d, g);
  if (shape != RTQ_OK) return shape;
  const KernelFn fn = rot == kSRFT ? find_mapped<kSRFT>(fwd, d, g) : find_mapped<kSRHT>(fwd, d, g);
  if (!fn) return RTQ_ERR_UNSUPPORTED;
  const int64_t n = (int64_t)layers * 2 * streams * ntok;
  if (n == 0) return RTQ_OK;
  if (n > kMaxRows || (int64_t)t0 + ntok > 0x7fffffff) return RTQ_ERR_INVALID_ARG;
  const void* a = in0;
  const void* b = fwd ? out0 : in1;
  const void* c = fwd ? out1 : out0;
  if (!a || !b || !c || !aligned16(a) || !aligned16(b) || !aligned16(c)) return RTQ_ERR_INVALID_ARG;
  const __int128 max_row = (__int128)(layers - 1) * st[0] + st[1] + (__int128)(streams - 1) * st[2] +
                           ((__int128)t0 + ntok - 1) * st[3];
  if (max_row >= ((__int128)1 << 56)) return RTQ_ERR_INVALID_ARG;
  const __int128 code_bytes = (max_row + 1) * (d / 2), scale_bytes = (max_row + 1) * 2 * (d / g);
  if (fwd) {
    const __int128 x_bytes = (__int128)n * 2 * d;
    if (overlaps128(in0, x_bytes, out0, code_bytes) || overlaps128(in0, x_bytes, out1, scale_bytes) ||
        overlaps128(out0, code_bytes, out1, scale_bytes))
      return RTQ_ERR_INVALID_ARG;
  } else {
    const __int128 y_bytes = (max_row + 1) * 2 * d;
    if (overlaps128(out0, y_bytes, in0, code_bytes) || overlaps128(out0, y_bytes, in1, scale_bytes))
      return RTQ_ERR_INVALID_ARG;
  }
  RowMap m;
  m.sl = st[0];
  m.skv = st[1];
  m.ss = st[2];
  m.st = st[3];
  m.t0 = (uint32_t)t0;
  m.n = (uint32_t)ntok;
  m.streams = (uint32_t)streams;
  m.by_n = make_div32((uint32_t)ntok);
  m.by_streams = make_div32((uint32_t)streams);
  RowSeeds rs;
  rs.seed = seed;
  rs.rps = rps;
  rs.period = period;
  uint32_t n32 = (uint32_t)n;
  const int vpt = d == 256 ? 32 : 64;  // rows per tile
  const int64_t tiles = (n + vpt - 1) / vpt;
  if (fwd) {
    const void* x = in0;
    void* codes = out0;
    void* scales = out1;
    void* kargs[] = {&x, &codes, &scales, &n32, &m, &rs};
    return launch(fn, tiles, kargs, stream);
  }
  const void* codes = in0;
  const void* scales = in1;
  void* y = out0;
  void* kargs[] = {&codes, &scales, &y, &n32, &m, &rs};
  return launch(fn, tiles, kargs, stream);
}

}  // namespace rtq

#define RTQ_API extern "C" __attribute__((visibility("default")))

#define RTQ_MAPPED_API(NAME, A0, A1, A2)                                                          \
  RTQ_API rtq_status NAME(A0, A1, A2, int32_t layers, int32_t streams, int32_t t0, int32_t n_tokens, int32_t d,  \
                          int32_t group, int64_t stride_layer, int64_t stride_kv, int64_t stride_stream,          \
                          int64_t stride_token, uint64_t seed, int64_t rows_per_seed, int32_t seed_period,        \
                          hipStream_t stream)

RTQ_MAPPED_API(srft_quant_append, const void* x_f16, void* codes_u8, void* scales_f16) {
  const int64_t st[4] = {stride_layer, stride_kv, stride_stream, stride_token};
  return rtq::run_mapped(true, rtq::kSRFT, x_f16, nullptr, codes_u8, scales_f16, layers, streams, t0, n_tokens, d,
                         group, st, seed, rows_per_seed, seed_period, stream);
}

RTQ_MAPPED_API(srht_quant_append, const void* x_f16, void* codes_u8, void* scales_f16) {
  const int64_t st[4] = {stride_layer, stride_kv, stride_stream, stride_token};
  return rtq::run_mapped(true, rtq::kSRHT, x_f16, nullptr, codes_u8, scales_f16, layers, streams, t0, n_tokens, d,
                         group, st, seed, rows_per_seed, seed_period, stream);
}

RTQ_MAPPED_API(srft_dequant_rows, const void* codes_u8, const void* scales_f16, void* y_f16) {
  const int64_t st[4] = {stride_layer, stride_kv, stride_stream, stride_token};
  return rtq::run_mapped(false, rtq::kSRFT, codes_u8, scales_f16, y_f16, nullptr, layers, streams, t0, n_tokens, d,
                         group, st, seed, rows_per_seed, seed_period, stream);
}

RTQ_MAPPED_API(srht_dequant_rows, const void* codes_u8, const void* scales_f16, void* y_f16) {
  const int64_t st[4] = {stride_layer, stride_kv, stride_stream, stride_token};
  return rtq::run_mapped(false, rtq::kSRHT, codes_u8, scales_f16, y_f16, nullptr, layers, streams, t0, n_tokens, d,
                         group, st, seed, rows_per_seed, seed_period, stream);
}

#undef RTQ_MAPPED_API

