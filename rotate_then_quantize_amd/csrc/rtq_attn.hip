// rtq_attn.hip -- one decode step of attention that reads the int4 rotated
// K/V cache directly (MI355X, gfx950), and its C ABI entry points.
//
// The method stores every K/V vector rotated and int4-quantized and
// dequantizes and rotates it back when attention reads it ("Quantization
// Speed Is Often a Kernel Problem", "First, the 17%").  Here the dequantize
// happens in registers inside the attention kernel, so no fp16 K/V ever
// lands in HBM: a separate dequantize pass would write and re-read the fp16
// cache and give back the bandwidth the int4 codes save ("Day 9 -
// Quantization: Shrink the Bytes Themselves", "Dequantization Must Fuse into
// the Kernel"; "Chapter 25 - Quantization: The Hardware View", "The
// Dequant/Requant Tax").  Per-group scales split each dot product into
// blocks that are scaled one by one and summed in higher precision (same
// chapter, "Granularity: Per-Tensor vs Per-Channel vs Per-Group"): here one
// fp32 scaling per 32-dim group of q.k.
//
// R is orthogonal and each stream's keys share one sign vector D_K (values
// one D_V), so with y = R D_K q and z_t = the dequantized rotated key,
//   q . k_t = y . z_t   and   sum_t p_t v_t = D_V R^T (sum_t p_t z^V_t).
// The kernel rotates each query once, runs softmax attention in the rotated
// domain, and rotates one output vector back per query, instead of
// inverse-rotating every cached vector.
//
// Mapping to CDNA4 (d = 64 / 128 / 256; q_per_kv <= 8):
//   * One workgroup of 4 waves per (layer, stream); the waves split the
//     stream's tokens into 32-token chunks and merge their softmax partials
//     in LDS.  Workgroup ids are remapped so that each XCD works through one
//     contiguous range of (layer, stream) pairs.  With few pairs and a
//     caller workspace, a stream's chunks are spread over several workgroups
//     whose partials the last one to finish merges (the online-softmax merge
//     again).
//   * Each chunk's code and scale rows arrive by direct-to-LDS loads
//     (global_load_lds) into a ring of ring_slots(d) chunk buffers per wave,
//     filled ahead of the chunk being computed.  Rows may sit anywhere (the
//     cache layout is given by strides).
//   * q.k is a [16 tokens x 32 dims] x [32 dims x 16 columns] MFMA
//     (v_mfma_f32_16x16x32_f16) per group of 32 dims.  The A operand is the
//     exact int4 code value as fp16 (no scale), so each group's partial dot
//     product is scaled by its fp16 scale in fp32 afterwards.  The query
//     operand carries the rotated query split into an fp16 high part
//     (columns 0..7) and low part (columns 8..15); one DPP add merges them,
//     so scores keep about 22 bits.
//   * p.v runs as O^T = V^T P^T per 16 output dims (v_mfma_f32_16x16x32_f16
//     over 32 tokens), with V decoded as fp16 (q * s / 16: the 1/16 keeps
//     every value finite for any fp16 scale) and P in fp16.  The P operand
//     is the q.k result layout itself, and O^T columns are queries, so the
//     online-softmax rescale stays in the lane that owns the query.
//   * int4 -> fp16 takes one v_bitop3 per pair of codes (mask, bias and
//     fp16 exponent at once) and one packed fp16 add or fma.
//   * The method keeps the newest tokens in fp16, unquantized ("First, the
//     17%").  The _window entry points take those tokens too: after the int4
//     part is merged, the workgroup scores the window in the original domain
//     and joins it to the same softmax with the online-softmax merge.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "rtq.h"
#include "rtq_device.hpp"
#include "rtq_mem.hpp"

namespace rtq {
namespace attn {

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

// Waves per workgroup, which split a stream's tokens into as many parts.
// (Two waves at d = 128 ran 10% faster on the Qwen2.5-1.5B cache, 234-240
// against 260-264 us, since the lead wave's query and output transforms then
// leave one wave waiting instead of three.  Each wave's accumulators then
// sum twice as many tokens against one running max, and the fp16 rounding of
// weights and values lands differently: on a test cache with outlier
// channels, where the output cancels terms 24 times its size, one element
// moved 8% past the parity bound.  Kept at 4 until that bound is derived
// from the fp16 operands instead of fixed.)
__host__ __device__ constexpr int waves_per_stream(int) { return 4; }
constexpr int kMaxWavesPerStream = 4;
constexpr int kChunk = 32;     // tokens per chunk (one p.v k-step)
// Chunk buffers per wave (one fewer chunks in flight) and the waves per SIMD
// the register allocation targets, by head dimension.  d = 128: two slots
// (41 KB of LDS per workgroup) and three waves per SIMD, so three
// workgroups share a CU; against three slots (60 KB, two workgroups per CU)
// this took 226 instead of 256 us on the Qwen2.5-1.5B decode cache, the
// third resident wave hiding more of each chunk's load and LDS latency than
// the second chunk in flight did.  d = 64: three slots at two waves (the
// compiler stays at 138 VGPRs, so three waves per SIMD run anyway).  d = 256:
// two slots (three would leave room for one workgroup per CU) at two waves.
__host__ __device__ constexpr int ring_slots(int d) { return d == 64 ? 3 : 2; }
__host__ __device__ constexpr int waves_per_eu(int d) { return d == 128 ? 3 : 2; }
constexpr int kMaxQ = 8;       // query heads per K/V head
constexpr float kNegBig = -1.0e30f;  // running-max start: finite, below any score
constexpr float kVShift = 0.0625f;   // V is decoded as q * s / 16
constexpr float kRescaleSlack = 8.0f;  // base-2 headroom of the running softmax max

struct Params {
  const uint4* q;        // [layers][streams][q_per_kv][d] fp16
  const uint8_t* codes;  // rows of d/2 bytes
  const uint8_t* scales; // rows of 2*d/group bytes
  uint4* out;            // like q
  int64_t stride_layer, stride_kv, stride_stream, stride_token;  // in rows
  uint64_t seed;
  int64_t rows_per_seed;
  int32_t seed_period;
  int32_t streams, tokens, q_per_kv;
  float qscale;  // softmax_scale * log2(e): scores come out in base-2 units
  // Token splits per (layer, stream): splits > 1 spreads a stream's chunks
  // over that many workgroups, which leave unnormalized partials in part and
  // count in count; the last one to finish merges them.
  int32_t splits;
  float* part;      // [pairs][splits][PartFloats]
  uint32_t* count;  // [pairs], zero between calls
  // fp16 window of each stream's newest tokens, unquantized and in the
  // original domain: [layers][K, V][streams][win_cap][d], or null.
  const uint4* win;
  int32_t win_cap, win_tokens;
};

constexpr int kMaxWindow = 64;  // window tokens per stream

// Floats of one split's partial: the unnormalized output sum of each query
// (q_per_kv rows of d), then its running max and its softmax denominator.
__host__ __device__ constexpr int64_t part_floats(int g, int d) { return ((int64_t)g * (d + 2) + 3) & ~(int64_t)3; }

template <int D, int GR>
struct Cfg {
  static constexpr int WAVES = waves_per_stream(D);
  static constexpr int BUFS = ring_slots(D);  // ring slots per wave
  static constexpr int KS = D / 32;       // q.k k-steps = 16-byte pieces per code row
  static constexpr int NT = D / 16;       // p.v output tiles of 16 dims
  static constexpr int RB = D / 2;        // code bytes per row
  static constexpr int SPR = D / GR;      // scales per row
  static constexpr int SLOT = 2 * SPR > 4 ? 2 * SPR : 4;  // LDS bytes per token of scales
  static constexpr int CODE_BYTES = kChunk * RB;
  static constexpr int SCALE_BYTES = kChunk * SLOT;
  static constexpr int BUF = 2 * CODE_BYTES + 2 * SCALE_BYTES;  // K codes, V codes, K scales, V scales
  static constexpr int CODE_DMA = CODE_BYTES / 1024;             // 16-byte loads per chunk per K or V
  static constexpr int NDMA = 2 * CODE_DMA + (SLOT == 8 ? 2 : 1);
  static constexpr int QROW = D + 4;  // fp32 row stride of the query / output staging
  static constexpr int SLOT_ARRAY = WAVES * BUF;  // one ring slot of every wave
  static constexpr int COMBINE = WAVES * kMaxQ * QROW * 4 + 2 * WAVES * kMaxQ * 4;
  static_assert(COMBINE <= SLOT_ARRAY, "the merge area fits in ring slot 0");
  static_assert(GR >= 32 && D % GR == 0, "groups of at least 32 values");
  // d = 256: the whole workgroup rotates the queries and outputs (TPC
  // threads per coordinate, each for kMaxQ / TPC queries), in a work area
  // that aliases the last ring slot, which is free before its first chunk is
  // issued and after the last one: the query stage [kMaxQ][QROW], the
  // transposed vectors [D][kMaxQ] and the twiddles [D].
  static constexpr bool DENSE_ROT = D == 256;
  static constexpr int WORK_SLOT = BUFS - 1;
  static constexpr int TPC = 64 * WAVES / D;
  static constexpr int ROT_AREA = kMaxQ * QROW * 4 + D * kMaxQ * 4 + D * 8;
  static_assert(!DENSE_ROT || (ROT_AREA <= SLOT_ARRAY && D * TPC == 64 * WAVES && (TPC == 1 || TPC == 2)),
                "the rotation area needs a free ring slot and one or two threads per coordinate");
};

// Token row r of a chunk sits in LDS row lrow(r) (an involution), and 16-byte
// piece k of LDS row L in slot k ^ swz(L).  For d = 128 and d = 256 this
// makes both the q.k reads (16 rows x 4 lanes) and the p.v reads (4 rows x
// 16 lanes) hit 64 distinct banks.  At d = 256 (128-byte rows, two rows per
// 64 banks) the p.v rows 4h + c get alternating parity from lrow, and the
// two rows of one parity get slot ranges 4 apart from swz.
template <int D>
__device__ __forceinline__ int lrow(int r) {
  if constexpr (D == 256) return r ^ ((r >> 2) & 1);
  else if constexpr (D == 128) return r ^ ((r >> 2) & 3);
  else return r;
}
template <int D>
__device__ __forceinline__ int swz(int lr) {
  if constexpr (D == 256) return (lr >> 1) & 7;
  else if constexpr (D == 128) return (lr >> 2) & 3;
  else return (lr >> 3) & 1;
}

__device__ __forceinline__ f16x2_t as_h2(uint32_t w) { return __builtin_bit_cast(f16x2_t, w); }
__device__ __forceinline__ uint32_t as_u32(f16x2_t h) { return __builtin_bit_cast(uint32_t, h); }

// Codes K and K+4 of a code word (low and high half of the result) as exact
// fp16 integers in [-8, 7].  K even: mask bits 4K'..4K'+3 of each half into
// the fp16 mantissa under the exponent of 1024 with the sign bit of the code
// flipped (one v_bitop3), giving 1032 + q; subtract 1032.  K odd: the code
// sits 4 bits higher, giving 1152 + 16 q; scale by 1/16 and subtract 72.
// (The key operand at d = 256, where key_pair's bias registers would spill.)
template <int K>
__device__ __forceinline__ f16x2_t code_pair(uint32_t w) {
  const uint32_t x = K >= 2 ? w >> 8 : w;
  if constexpr ((K & 1) == 0) {
    return as_h2((x & 0x000f000fu) ^ 0x64086408u) + (f16x2_t){(_Float16)-1032.0f, (_Float16)-1032.0f};
  } else {
    return __builtin_elementwise_fma(as_h2((x & 0x00f000f0u) ^ 0x64806480u),
                                     (f16x2_t){(_Float16)0.0625f, (_Float16)0.0625f},
                                     (f16x2_t){(_Float16)-72.0f, (_Float16)-72.0f});
  }
}

// Codes K and K+4 of a key code word as the fp16 subnormals (q + 8) 2^-24,
// times 16 for odd K (the code sits 4 bits higher): one v_bitop3 each (mask
// and flip of the code's sign bit), the shift by 8 shared by K = 2 and 3.
// The q.k operand of odd-K dims carries the matching 1/16, and the bias 8
// enters the MFMA accumulator as its start value (key_bias), so the q.k
// MFMA sums (q + 8) y and starts from -8 sum(y): scores come out times 2^-24.
template <int K>
__device__ __forceinline__ f16x2_t key_pair(uint32_t w) {
  const uint32_t x = K >= 2 ? w >> 8 : w;
  if constexpr ((K & 1) == 0) return as_h2((x & 0x000f000fu) ^ 0x00080008u);
  else return as_h2((x & 0x00f000f0u) ^ 0x00800080u);
}

// Codes K and K+4 of a value code word as exact fp16 q / 16: the code under
// the exponent of 1024 (1032 + q, K even) or of 1024 with the code 4 bits up
// (1152 + 16 q, K odd), then one packed fma with 1/16 and -64.5 or with 1/256
// and -4.5 (every step exact in fp16).
template <int K>
__device__ __forceinline__ f16x2_t value_pair16(uint32_t w) {
  const uint32_t x = K >= 2 ? w >> 8 : w;
  if constexpr ((K & 1) == 0) {
    return __builtin_elementwise_fma(as_h2((x & 0x000f000fu) ^ 0x64086408u),
                                     (f16x2_t){(_Float16)0.0625f, (_Float16)0.0625f},
                                     (f16x2_t){(_Float16)-64.5f, (_Float16)-64.5f});
  } else {
    return __builtin_elementwise_fma(as_h2((x & 0x00f000f0u) ^ 0x64806480u),
                                     (f16x2_t){(_Float16)0.00390625f, (_Float16)0.00390625f},
                                     (f16x2_t){(_Float16)-4.5f, (_Float16)-4.5f});
  }
}

// a - (half SEL of h as fp16), in fp32 (one v_fma_mix_f32; exact when that
// half is a rounding of a)
template <int SEL>
__device__ __forceinline__ float residual_of_half(float a, uint32_t h) {
  float r;
  if constexpr (SEL == 0) asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(a));
  else asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(a));
  return r;
}

// max of three floats (v_max3_f32 written out: fmaxf adds a quieting
// v_max_f32 x, x before every operand the compiler cannot prove canonical,
// and the lane-swap results below are such operands; scores are never
// signalling NaNs)
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// half SEL of w (fp16) times b plus c, in fp32 (one v_fma_mix_f32).  Plain
// code, not inline asm: b is an MFMA result, and the compiler inserts the wait
// states between an MFMA and a VALU read of its result only for instructions
// it can see.
template <int SEL>
__device__ __forceinline__ float half_fma(uint32_t w, float b, float c) {
  return __builtin_fmaf((float)as_h2(w)[SEL], b, c);
}

__device__ __forceinline__ f16x8_t pack8(f16x2_t a, f16x2_t b, f16x2_t c, f16x2_t d) {
  const u32x4v_t w = {as_u32(a), as_u32(b), as_u32(c), as_u32(d)};
  return __builtin_bit_cast(f16x8_t, w);
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

__device__ __forceinline__ f32x4_t mfma(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// x + (x of the lane 8 places further in the same row of 16 lanes).
__device__ __forceinline__ float add_ror8(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false);
  return x + __int_as_float(y);
}

// Max of x over lanes n, n + 16, n + 32, n + 48 (the four lane groups that
// hold one query column), with the gfx950 lane-swap instructions: swapping
// x with itself across 16-lane rows and then across 32-lane halves.
__device__ __forceinline__ float max_over_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max3f(__uint_as_float(a[0]), __uint_as_float(a[1]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3f(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[1]));
}

// Sum of x over lanes n, n + 16, n + 32, n + 48 (the same lane swaps).
__device__ __forceinline__ float sum_over_row_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Device-scope (all XCDs) store and load of one float of a split partial.
__device__ __forceinline__ void publish(float* a, float v) {
  __hip_atomic_store(a, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float collect(const float* a) {
  return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t seed_of_row(const Params& p, int64_t row) {
  return row_seed(p.seed, row, p.rows_per_seed, p.seed_period);
}

// Sign masks of one seed for the D/2 packed pairs, the same in every lane.
template <int D>
__device__ __forceinline__ void wave_sign_masks(uint64_t s, int lane, uint32_t (&m)[D / 2]) {
  sfor<D / 64>([&](auto Q) {
    constexpr int q = RTQ_CI(Q);
    const uint64_t bits = __ballot(sign_bit(s, (uint32_t)(64 * q + lane)));
    sfor<32>([&](auto M) {
      const uint32_t v = (uint32_t)(bits >> (2 * RTQ_CI(M))) & 3u;
      m[32 * q + RTQ_CI(M)] = (v * 0x40008000u) & 0x80008000u;
    });
  });
}

// ---------------------------------------------------------------------------
// d = 256: the queries are rotated and the outputs rotated back by the whole
// workgroup, each thread computing one coordinate of the queries as a direct
// sum over the d inputs, where one lane per vector would need 256 fp32
// registers.  This runs once per stream and step, about 2k instructions per
// thread.  (The code also takes two threads per coordinate, each for half the
// queries, as d = 128 would need; at d = 128 that measured slower than the
// lead wave's per-lane transforms, 288 against 270-280 us on the Qwen2.5-1.5B
// cache.)  Vectors sit transposed in LDS, v[n * kMaxQ + g], so each term's
// reads are one broadcast.
// ---------------------------------------------------------------------------

struct Twiddle256 {
  float c[256], s[256];  // cos(2 pi m / 256), sin(2 pi m / 256)
};
consteval Twiddle256 make_twiddle256() {
  Twiddle256 t{};
  for (int m = 0; m < 256; ++m) {
    t.c[m] = (float)cos2pi(m, 256);
    t.s[m] = (float)sin2pi(m, 256);
  }
  return t;
}
__constant__ Twiddle256 kTwiddle256 = make_twiddle256();

template <int NQ>
__device__ __forceinline__ void load_column(const float* v, int n, float (&a)[NQ]) {
  const float4 x = *reinterpret_cast<const float4*>(v + n * kMaxQ);
  a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
  if constexpr (NQ == 8) {
    const float4 y = *reinterpret_cast<const float4*>(v + n * kMaxQ + 4);
    a[4] = y.x; a[5] = y.y; a[6] = y.z; a[7] = y.w;
  }
}

// Twiddle m of a length-D transform, (cos, sin)(2 pi m / D), from the
// 256-entry table.
template <int D>
__device__ __forceinline__ float2 twiddle(int m) {
  return make_float2(kTwiddle256.c[m * (256 / D)], kTwiddle256.s[m * (256 / D)]);
}

// z[g] = coordinate t of R v_g for NQ vectors (v: the transposed vectors,
// first of the NQ queries at v[0]): the packed orthonormal real DFT
// (z_0 = X_0 / sqrt(D), z_{2k-1} = sqrt2 Re X_k / sqrt(D), z_{2k} =
// sqrt2 Im X_k / sqrt(D), z_{D-1} = X_{D/2} / sqrt(D)) for SRFT, H v / sqrt(D)
// for SRHT.
template <int D, int ROT, int NQ>
__device__ __forceinline__ void dense_forward(const float* v, const float2* tw, int t, float (&z)[NQ]) {
  float acc[NQ];
  sfor<NQ>([&](auto G) { acc[RTQ_CI(G)] = 0.0f; });
  if constexpr (ROT == 0) {
    const int k = (t + 1) >> 1;
    const bool im = t > 0 && t < D - 1 && (t & 1) == 0;  // X_k = sum v_n (cos - i sin)(2 pi k n / D)
    int idx = 0;
#pragma unroll 4
    for (int n = 0; n < D; ++n) {
      const float2 w = tw[idx];
      const float c = im ? -w.y : w.x;
      float a[NQ];
      load_column<NQ>(v, n, a);
      sfor<NQ>([&](auto G) { acc[RTQ_CI(G)] = __builtin_fmaf(c, a[RTQ_CI(G)], acc[RTQ_CI(G)]); });
      idx = (idx + k) & (D - 1);
    }
    constexpr float n_end = (float)(1.0 / csqrt((double)D)), n_mid = (float)(csqrt(2.0 / (double)D));
    const float norm = (t == 0 || t == D - 1) ? n_end : n_mid;
    sfor<NQ>([&](auto G) { z[RTQ_CI(G)] = acc[RTQ_CI(G)] * norm; });
  } else {
#pragma unroll 4
    for (int n = 0; n < D; ++n) {
      const float c = (__builtin_popcount(t & n) & 1) ? -1.0f : 1.0f;  // H[t][n]
      float a[NQ];
      load_column<NQ>(v, n, a);
      sfor<NQ>([&](auto G) { acc[RTQ_CI(G)] = __builtin_fmaf(c, a[RTQ_CI(G)], acc[RTQ_CI(G)]); });
    }
    sfor<NQ>([&](auto G) { z[RTQ_CI(G)] = acc[RTQ_CI(G)] * InvSqrt<D>::value; });
  }
}

// u[g] = element t of R^T z_g: the orthonormal inverse real DFT of the
// unpacked bins for SRFT, H z / sqrt(D) for SRHT.
template <int D, int ROT, int NQ>
__device__ __forceinline__ void dense_inverse(const float* z, const float2* tw, int t, float (&u)[NQ]) {
  if constexpr (ROT == 0) {
    float a0[NQ], a1[NQ], acc[NQ];
    load_column<NQ>(z, 0, a0);
    load_column<NQ>(z, D - 1, a1);
    const float alt = (t & 1) ? -1.0f : 1.0f;  // cos(pi t)
    sfor<NQ>([&](auto G) { acc[RTQ_CI(G)] = 0.0f; });
    int idx = t;
#pragma unroll 4
    for (int k = 1; k < D / 2; ++k) {
      const float2 w = tw[idx];
      float re[NQ], im[NQ];
      load_column<NQ>(z, 2 * k - 1, re);
      load_column<NQ>(z, 2 * k, im);
      sfor<NQ>([&](auto G) {
        constexpr int g = RTQ_CI(G);
        acc[g] = __builtin_fmaf(w.x, re[g], __builtin_fmaf(-w.y, im[g], acc[g]));
      });
      idx = (idx + t) & (D - 1);
    }
    constexpr float r2 = (float)csqrt(2.0);
    sfor<NQ>([&](auto G) {
      constexpr int g = RTQ_CI(G);
      u[g] = __builtin_fmaf(r2, acc[g], __builtin_fmaf(alt, a1[g], a0[g])) * InvSqrt<D>::value;
    });
  } else {
    dense_forward<D, 1, NQ>(z, tw, t, u);  // H / sqrt(D) is its own inverse
  }
}

// One direct-to-LDS load (nt): lane i's BYTES bytes from g land at LDS byte
// lds + BYTES * i.  Written as inline asm so that the compiler, which cannot
// tell the ring slots apart, does not add a full vmcnt wait before every LDS
// read; the kernel waits for each chunk itself (wait_vmcnt).  The asm has no
// register outputs.
// A 2-byte load fills the whole 4-byte slot of its lane (zero-extended).
template <int BYTES>
__device__ __forceinline__ void dma_to_lds(const void* g, const void* lds) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);  // wave-uniform
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(m), "v"(g) : "memory", "m0");
  else if constexpr (BYTES == 4)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off nt" ::"s"(m), "v"(g) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_ushort %1, off nt" ::"s"(m), "v"(g) : "memory", "m0");
}

// Dense prologue (d = 128, 256), every thread: the stream's G queries,
// sign-flipped with the key signs, go transposed into the work area (element
// n of queries 4h' .. 4h' + 3 by thread n + D h'); the TPC threads of
// coordinate c compute it for their share of the queries, scaled by qscale;
// then each query is scaled by the power of two 2^-e that puts its largest
// entry in [2^13, 2^14) and stored to the stage [kMaxQ][D + 4].
template <int D, int ROT>
__device__ __forceinline__ void dense_queries(const Params& p, int64_t qrow, uint64_t seed_k, int G, uint8_t* area,
                                              float* stage, int* qexp) {
  constexpr int TPC = 64 * waves_per_stream(D) / D, NQ = kMaxQ / TPC;
  __shared__ uint32_t amax_bits[kMaxQ];
  const int t = threadIdx.x, c = t % D, g0 = (t / D) * NQ;
  float* vt = reinterpret_cast<float*>(area + kMaxQ * (D + 4) * 4);
  float2* tw = reinterpret_cast<float2*>(vt + D * kMaxQ);
  const _Float16* q16 = reinterpret_cast<const _Float16*>(p.q);
  const float sg = sign_bit(seed_k, (uint32_t)c) ? -1.0f : 1.0f;
  float col[NQ];
  sfor<NQ>([&](auto Gi) {
    const int g = g0 + RTQ_CI(Gi);
    col[RTQ_CI(Gi)] = g < G ? sg * (float)q16[(qrow + g) * D + c] : 0.0f;
  });
  *reinterpret_cast<float4*>(vt + c * kMaxQ + g0) = make_float4(col[0], col[1], col[2], col[3]);
  if constexpr (NQ == 8) *reinterpret_cast<float4*>(vt + c * kMaxQ + 4) = make_float4(col[4], col[5], col[6], col[7]);
  if (ROT == 0 && t < D) tw[t] = twiddle<D>(t);
  if (t < kMaxQ) amax_bits[t] = 0u;
  __syncthreads();
  float z[NQ];
  if (g0 < G) {
    if (NQ == 8 && G <= 4) {
      float z4[4];
      dense_forward<D, ROT, 4>(vt, tw, c, z4);
      sfor<NQ>([&](auto Gi) { z[RTQ_CI(Gi)] = RTQ_CI(Gi) < 4 ? z4[RTQ_CI(Gi) & 3] : 0.0f; });
    } else {
      dense_forward<D, ROT, NQ>(vt + g0, tw, c, z);
    }
    sfor<NQ>([&](auto Gi) {
      const int g = g0 + RTQ_CI(Gi);
      z[RTQ_CI(Gi)] *= p.qscale;
      if (g < G)
        __hip_atomic_fetch_max(&amax_bits[g], __float_as_uint(fabsf(z[RTQ_CI(Gi)])), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    });
  }
  __syncthreads();
  if (g0 < G) {
    sfor<NQ>([&](auto Gi) {
      const int g = g0 + RTQ_CI(Gi);
      const float amax = __uint_as_float(amax_bits[g]);
      const int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 14 : 0;
      stage[g * (D + 4) + c] = __builtin_ldexpf(z[RTQ_CI(Gi)], -e);
      if (c == g) qexp[g] = e;
    });
  }
}

// Direct-to-LDS loads of chunk tokens tok0 .. tok0+31 (tokens past the end
// reload the last token; their scores are masked).
template <int D, int GR>
__device__ __forceinline__ void issue_chunk(const Params& p, int64_t row_k, int64_t row_v, int tok0, uint8_t* buf,
                                            int lane) {
  using C = Cfg<D, GR>;
  constexpr int PPR = C::RB / 16;  // pieces per row
  constexpr int RPI = 64 / PPR;    // LDS rows per load instruction
  const int last = p.tokens - 1;
  sfor<C::CODE_DMA>([&](auto I) {
    const int lr = RTQ_CI(I) * RPI + lane / PPR;
    const int r = lrow<D>(lr);
    const int piece = (lane % PPR) ^ swz<D>(lr);
    const int t = tok0 + r < last ? tok0 + r : last;
    const int64_t off = (int64_t)t * p.stride_token;
    const uint8_t* gk = p.codes + (row_k + off) * C::RB + 16 * piece;
    const uint8_t* gv = p.codes + (row_v + off) * C::RB + 16 * piece;
    dma_to_lds<16>(gk, buf + RTQ_CI(I) * 1024);
    dma_to_lds<16>(gv, buf + C::CODE_BYTES + RTQ_CI(I) * 1024);
  });
  uint8_t* sb = buf + 2 * C::CODE_BYTES;
  if constexpr (C::SLOT == 16) {
    // 16 bytes per token: lanes 0..31 keys, 32..63 values, one load each
    const int r = lane & 31;
    const int t = tok0 + r < last ? tok0 + r : last;
    const int64_t row = (lane < 32 ? row_k : row_v) + (int64_t)t * p.stride_token;
    dma_to_lds<16>(p.scales + row * 16, sb);
  } else if constexpr (C::SLOT == 8) {
    // 8 bytes per token: lane l loads word l & 1 of token l / 2
    const int t = tok0 + lane / 2 < last ? tok0 + lane / 2 : last;
    const int64_t off = (int64_t)t * p.stride_token;
    dma_to_lds<4>(p.scales + (row_k + off) * 8 + 4 * (lane & 1), sb);
    dma_to_lds<4>(p.scales + (row_v + off) * 8 + 4 * (lane & 1), sb + C::SCALE_BYTES);
  } else {
    // one 4-byte slot per token (2 or 4 bytes of scales): lanes 0..31 keys, 32..63 values
    const int r = lane & 31;
    const int t = tok0 + r < last ? tok0 + r : last;
    const int64_t row = (lane < 32 ? row_k : row_v) + (int64_t)t * p.stride_token;
    dma_to_lds<2 * C::SPR>(p.scales + row * (2 * C::SPR), sb);
  }
}

// DPP lane moves: x of another lane of the same row of 16.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// op over each aligned group of N lanes (N = 8, 16, 32 or 64), in every lane
// of the group: quad swaps, then the mirror of each 8 and of each 16 lanes,
// then the 16- and 32-lane swaps.  Every lane of the wave must be active.
template <int N, class Op>
__device__ __forceinline__ float reduce_lanes(float x, Op op) {
  static_assert(N == 8 || N == 16 || N == 32 || N == 64, "lane groups of 8 to 64");
  x = op(x, dpp<0xB1>(x));   // quad_perm 1,0,3,2
  x = op(x, dpp<0x4E>(x));   // quad_perm 2,3,0,1
  x = op(x, dpp<0x141>(x));  // row_half_mirror: lane i <-> 7 - i
  if constexpr (N >= 16) x = op(x, dpp<0x140>(x));  // row_mirror: lane i <-> 15 - i
  if constexpr (N >= 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  if constexpr (N >= 64) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = op(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  return x;
}
struct AddOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};
struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

// LDS of the window part: the weights [kMaxWindow][kMaxQ] and coef[kMaxQ]
// (in ring slot 0), and the partial value sums of every token phase
// [planes][kMaxQ][D], whose plane 0 becomes the window output ows[g][D].
template <int D>
struct WindowLds {
  static constexpr int PAIRS = D / 2;               // 4-byte dim pairs per row
  static constexpr int PHASES = 64 * waves_per_stream(D) / PAIRS;  // token phases of the value loop
  static constexpr int PLANES = PAIRS < 64 ? waves_per_stream(D) : PHASES;  // d = 64: one per wave
  static constexpr int WEIGHT_BYTES = 4096;
  static_assert((kMaxWindow * kMaxQ + kMaxQ) * 4 <= WEIGHT_BYTES, "weights and coef fit 4 KB");
  static constexpr int RED_BYTES = PLANES * kMaxQ * D * 4;
};

// The fp16 window's share of one softmax over the int4 tokens and the
// window tokens, by the whole workgroup.  Scores: lanes hold 16-byte pieces
// of the window key rows (a wave's loads cover consecutive rows) and dot them
// with the same pieces of every query; a row's pieces are summed over its
// lanes.  Softmax: one wave per query merges the window scores with the int4
// part's running max mq and denominator lq (the online-softmax merge).
// Values: each thread owns a dim pair and one token phase (coalesced rows),
// sums weight * value for every query, and the phases are summed through
// LDS.  Leaves coef[g] (the weight of the normalized int4 output) and
// ows[g * D + dim] (the window's part of the output, multiplied by the value
// sign of dim, since the output is sign-flipped as a whole at the end).
// Scores are in base-2 units like the int4 part's.  The window's K, V and
// query loads (WindowRegs) are all issued before the first use, so the part
// costs one memory round trip, which the caller can start early.
template <int D>
struct WindowRegs {
  using WL = WindowLds<D>;
  static constexpr int CPR = D / 8;                    // 16-byte pieces per row
  static constexpr int RPW = 64 / CPR;                 // rows per wave per key load
  static constexpr int RPG = RPW * waves_per_stream(D);  // rows per workgroup per key load
  static constexpr int NK = kMaxWindow / RPG;          // key loads per thread
  static constexpr int NV = kMaxWindow / WL::PHASES;   // value loads per thread
  uint4 qv[kMaxQ], kv[NK];
  uint32_t vv[NV];

  __device__ __forceinline__ void load(const Params& p, int64_t wrow_k, int64_t wrow_v, int64_t qrow, int G) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, W = p.win_tokens;
    const int c = lane % CPR, r0 = w * RPW + lane / CPR;
    const int pr = t % WL::PAIRS, ph = t / WL::PAIRS;
    const uint32_t* wv = reinterpret_cast<const uint32_t*>(p.win) + wrow_v * WL::PAIRS;
    sfor<kMaxQ>([&](auto I) {
      if (RTQ_CI(I) < G) qv[RTQ_CI(I)] = p.q[(qrow + RTQ_CI(I)) * CPR + c];
    });
    sfor<NK>([&](auto I) {
      const int j = r0 + RTQ_CI(I) * RPG;
      kv[RTQ_CI(I)] = j < W ? p.win[(wrow_k + j) * CPR + c] : make_uint4(0, 0, 0, 0);
    });
    sfor<NV>([&](auto I) {
      const int j = ph + RTQ_CI(I) * WL::PHASES;
      vv[RTQ_CI(I)] = j < W ? wv[(int64_t)j * WL::PAIRS + pr] : 0u;
    });
  }
};

template <int D>
__device__ __forceinline__ void window_part(const Params& p, const WindowRegs<D>& r, int G, uint64_t seed_v,
                                            const float* mq, const float* lq, float* wts, float* coef, float* red) {
  using WL = WindowLds<D>;
  using WR = WindowRegs<D>;
  constexpr int CPR = WR::CPR, RPG = WR::RPG, NK = WR::NK, NV = WR::NV;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, W = p.win_tokens;
  const int c = lane % CPR, r0 = w * WR::RPW + lane / CPR;
  const int pr = t % WL::PAIRS, ph = t / WL::PAIRS;
  const uint4* qv = r.qv;
  const uint4* kv = r.kv;
  const uint32_t* vv = r.vv;

  // scores of every (window token, query)
  sfor<NK>([&](auto I) {
    if (RTQ_CI(I) * RPG < W) {
      const int j = r0 + RTQ_CI(I) * RPG;
      const uint4 k = kv[RTQ_CI(I)];
      sfor<kMaxQ>([&](auto Gi) {
        constexpr int g = RTQ_CI(Gi);
        if (g < G) {
          const uint4 a = qv[g];
          float acc = __builtin_amdgcn_fdot2(as_h2(a.x), as_h2(k.x), 0.0f, false);
          acc = __builtin_amdgcn_fdot2(as_h2(a.y), as_h2(k.y), acc, false);
          acc = __builtin_amdgcn_fdot2(as_h2(a.z), as_h2(k.z), acc, false);
          acc = __builtin_amdgcn_fdot2(as_h2(a.w), as_h2(k.w), acc, false);
          acc = reduce_lanes<CPR>(acc, AddOp{});
          if (c == 0 && j < W) wts[j * kMaxQ + g] = acc * p.qscale;
        }
      });
    }
  });
  __syncthreads();

  // softmax over the int4 part and the window, one wave per query; the
  // weights of rows past the window become 0
  for (int g = w; g < G; g += waves_per_stream(D)) {
    const float sc = lane < W ? wts[lane * kMaxQ + g] : kNegBig;
    const float m = fmaxf(mq[g], reduce_lanes<64>(sc, MaxOp{}));
    const float fr = __builtin_amdgcn_exp2f(mq[g] - m);  // 0 when there is no int4 token
    const float e = lane < W ? __builtin_amdgcn_exp2f(sc - m) : 0.0f;
    const float inv = 1.0f / __builtin_fmaf(fr, lq[g], reduce_lanes<64>(e, AddOp{}));
    wts[lane * kMaxQ + g] = e * inv;
    if (lane == 0) coef[g] = fr * lq[g] * inv;
  }
  __syncthreads();

  // the weighted values: dims 2 pr, 2 pr + 1 of every query, over this phase's tokens
  float acc[kMaxQ][2];
  sfor<kMaxQ>([&](auto Gi) { acc[RTQ_CI(Gi)][0] = acc[RTQ_CI(Gi)][1] = 0.0f; });
  sfor<NV>([&](auto I) {
    if (RTQ_CI(I) * WL::PHASES < W) {
      const int j = ph + RTQ_CI(I) * WL::PHASES;  // < kMaxWindow
      const float4 wa = *reinterpret_cast<const float4*>(wts + j * kMaxQ);
      const float4 wb = *reinterpret_cast<const float4*>(wts + j * kMaxQ + 4);
      const float wg[kMaxQ] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
      const f16x2_t v = as_h2(vv[RTQ_CI(I)]);
      const float v0 = (float)v[0], v1 = (float)v[1];
      sfor<kMaxQ>([&](auto Gi) {
        constexpr int g = RTQ_CI(Gi);
        if (g < G) {
          acc[g][0] = __builtin_fmaf(wg[g], v0, acc[g][0]);
          acc[g][1] = __builtin_fmaf(wg[g], v1, acc[g][1]);
        }
      });
    }
  });
  int plane = ph;
  if constexpr (WL::PAIRS < 64) {
    // d = 64: the wave's two phases (lanes 0-31, 32-63) are summed here
    sfor<kMaxQ>([&](auto Gi) {
      sfor<2>([&](auto E) {
        const float x = acc[RTQ_CI(Gi)][RTQ_CI(E)];
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        acc[RTQ_CI(Gi)][RTQ_CI(E)] = __uint_as_float(a[0]) + __uint_as_float(a[1]);
      });
    });
    plane = w;
  }
  if (WL::PAIRS >= 64 || lane < 32) {
    sfor<kMaxQ>([&](auto Gi) {
      constexpr int g = RTQ_CI(Gi);
      if (g < G)
        *reinterpret_cast<float2*>(red + (plane * kMaxQ + g) * D + 2 * pr) = make_float2(acc[g][0], acc[g][1]);
    });
  }
  __syncthreads();
  for (int idx = t; idx < G * D; idx += 64 * waves_per_stream(D)) {
    const int g = idx / D, dim = idx - g * D;
    float sum = 0.0f;
    sfor<WL::PLANES>([&](auto P) { sum += red[(RTQ_CI(P) * kMaxQ + g) * D + dim]; });
    red[g * D + dim] = sign_bit(seed_v, (uint32_t)dim) ? -sum : sum;  // plane 0 becomes ows
  }
  __syncthreads();
}

// This lane's source addresses for token 0 of a chunk (the same pieces as
// issue_chunk), so that a full chunk's loads cost one 64-bit add each: chunk
// tok0 reads base + tok0 * (bytes per token step).  Only a stream's last,
// partial chunk goes through issue_chunk's clamped addressing.
template <int D, int GR>
struct ChunkSources {
  using C = Cfg<D, GR>;
  static constexpr int NS = C::SLOT == 8 ? 2 : 1;  // scale loads per chunk
  const uint8_t* k[C::CODE_DMA];
  const uint8_t* v[C::CODE_DMA];
  const uint8_t* s[NS];
  int64_t code_step, scale_step;  // bytes per token

  __device__ __forceinline__ ChunkSources(const Params& p, int64_t row_k, int64_t row_v, int lane) {
    constexpr int PPR = C::RB / 16, RPI = 64 / PPR;
    sfor<C::CODE_DMA>([&](auto I) {
      const int lr = RTQ_CI(I) * RPI + lane / PPR;
      const int r = lrow<D>(lr);
      const int piece = (lane % PPR) ^ swz<D>(lr);
      const int64_t off = (int64_t)r * p.stride_token;
      k[RTQ_CI(I)] = p.codes + (row_k + off) * C::RB + 16 * piece;
      v[RTQ_CI(I)] = p.codes + (row_v + off) * C::RB + 16 * piece;
    });
    if constexpr (C::SLOT == 16) {
      s[0] = p.scales + ((lane < 32 ? row_k : row_v) + (int64_t)(lane & 31) * p.stride_token) * 16;
    } else if constexpr (C::SLOT == 8) {
      const int64_t off = (int64_t)(lane / 2) * p.stride_token;
      s[0] = p.scales + (row_k + off) * 8 + 4 * (lane & 1);
      s[1] = p.scales + (row_v + off) * 8 + 4 * (lane & 1);
    } else {
      s[0] = p.scales + ((lane < 32 ? row_k : row_v) + (int64_t)(lane & 31) * p.stride_token) * (2 * C::SPR);
    }
    code_step = p.stride_token * C::RB;
    scale_step = p.stride_token * 2 * C::SPR;
  }

  // Direct-to-LDS loads of the full chunk of tokens tok0 .. tok0 + 31.
  __device__ __forceinline__ void issue(int tok0, uint8_t* buf) const {
    const int64_t dc = (int64_t)tok0 * code_step, ds = (int64_t)tok0 * scale_step;
    sfor<C::CODE_DMA>([&](auto I) {
      dma_to_lds<16>(k[RTQ_CI(I)] + dc, buf + RTQ_CI(I) * 1024);
      dma_to_lds<16>(v[RTQ_CI(I)] + dc, buf + C::CODE_BYTES + RTQ_CI(I) * 1024);
    });
    uint8_t* sb = buf + 2 * C::CODE_BYTES;
    if constexpr (C::SLOT == 16) {
      dma_to_lds<16>(s[0] + ds, sb);
    } else if constexpr (C::SLOT == 8) {
      dma_to_lds<4>(s[0] + ds, sb);
      dma_to_lds<4>(s[1] + ds, sb + C::SCALE_BYTES);
    } else {
      dma_to_lds<2 * C::SPR>(s[0] + ds, sb);
    }
  }
};

template <int D, int GR, int ROT>
__global__ void __launch_bounds__(64 * waves_per_stream(D)) __attribute__((amdgpu_waves_per_eu(waves_per_eu(D), 8)))
attn_decode_kernel(Params p) {
  using C = Cfg<D, GR>;
  constexpr int kWaves = C::WAVES, kStreams = 1;
  // Three ring slots as three LDS arrays: the compiler then tells the
  // direct-to-LDS loads of one slot from the reads of another and waits only
  // for the chunk being read.
  __shared__ __attribute__((aligned(16))) uint8_t slot0[C::SLOT_ARRAY];
  __shared__ __attribute__((aligned(16))) uint8_t slot1[C::SLOT_ARRAY];
  __shared__ __attribute__((aligned(16))) uint8_t slot2[C::BUFS > 2 ? C::SLOT_ARRAY : 16];
  // query in, output out (d = 256: in the work area of ring slot 1)
  __shared__ __attribute__((aligned(16))) float stage_arr[C::DENSE_ROT ? 4 : kStreams * kMaxQ * C::QROW];
  __shared__ int qexp_all[kStreams * kMaxQ];
  uint8_t* const work = C::WORK_SLOT == 1 ? slot1 : slot2;  // the dense rotations' area (last ring slot)
  float* const stage_all = C::DENSE_ROT ? reinterpret_cast<float*>(work) : stage_arr;
  float* const vt_all = reinterpret_cast<float*>(work + kMaxQ * C::QROW * 4);  // dense: [D][kMaxQ]

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n = lane & 15, h = lane >> 4;
  const int G = p.q_per_kv, T = p.tokens;
  // Workgroups go to the 8 XCDs round-robin (id b to XCD b % 8).  Give XCD x
  // one contiguous range of work items (a layer's stream pairs in order), so
  // the workgroups running together on an XCD read neighbouring streams, whose
  // scale rows share 128-byte lines in a time-major cache, through one L2.
  const int nwg = gridDim.x, b = blockIdx.x;
  const int per = nwg >> 3, extra = nwg & 7, x = b & 7;
  const int item = x * per + (x < extra ? x : extra) + (b >> 3);
  const int pair = item / p.splits, split = item - pair * p.splits;  // a pair's splits are neighbours
  const int pairs_per_layer = (p.streams + kStreams - 1) / kStreams;
  const int layer = pair / pairs_per_layer;
  const int sw = w / kWaves, part_w = w % kWaves;  // stream of the wave, token part
  const int stream = (pair - layer * pairs_per_layer) * kStreams + sw;
  const bool active = stream < p.streams;
  const int64_t row_k = (int64_t)layer * p.stride_layer + (int64_t)stream * p.stride_stream;
  const int64_t row_v = row_k + p.stride_kv;
  const int64_t qrow = ((int64_t)layer * p.streams + stream) * G;  // first query row of this stream
  float* const stage = stage_all + sw * kMaxQ * C::QROW;
  int* const qexp = qexp_all + sw * kMaxQ;

  // this workgroup's chunks (its split of the stream), then this wave's part of them
  const int64_t nchunks = active ? (T + kChunk - 1) / kChunk : 0;
  const int s_begin = (int)(split * nchunks / p.splits), s_len = (int)((split + 1) * nchunks / p.splits) - s_begin;
  const int c_begin = s_begin + part_w * s_len / kWaves;
  const int c_end = s_begin + (part_w + 1) * s_len / kWaves;
  const bool lead = active && part_w == 0;  // rotates the stream's queries and outputs

  // ---- prologue: queries (lead waves) and the first two chunks (every wave) ----
  uint4 qv[C::DENSE_ROT ? 1 : D / 8];
  if constexpr (!C::DENSE_ROT) {
    if (lead && lane < G) {
      const uint4* src = p.q + (qrow + lane) * (D / 8);
      sfor<D / 8>([&](auto I) { qv[RTQ_CI(I)] = src[RTQ_CI(I)]; });
    }
  }
  const ChunkSources<D, GR> src(p, row_k, row_v, lane);
  // a chunk is full unless it holds the stream's last token
  auto load_chunk = [&](int c, uint8_t* dst) {
    if ((c + 1) * kChunk <= T) src.issue(c * kChunk, dst);
    else issue_chunk<D, GR>(p, row_k, row_v, c * kChunk, dst, lane);
  };
  if (c_begin < c_end) load_chunk(c_begin, slot0 + w * C::BUF);
  if (C::BUFS > 2 && c_begin + 1 < c_end)
    load_chunk(c_begin + 1, slot1 + w * C::BUF);
  if constexpr (C::DENSE_ROT) {
    dense_queries<D, ROT>(p, qrow, seed_of_row(p, row_k), G, work, stage, qexp);
  } else if (lead) {
    uint32_t mk[D / 2];
    wave_sign_masks<D>(seed_of_row(p, row_k), lane, mk);
    if (lane < G) {
      uint32_t hq[D / 2];
      sfor<D / 8>([&](auto I) {
        constexpr int i = RTQ_CI(I);
        hq[4 * i] = qv[i].x ^ mk[4 * i];
        hq[4 * i + 1] = qv[i].y ^ mk[4 * i + 1];
        hq[4 * i + 2] = qv[i].z ^ mk[4 * i + 2];
        hq[4 * i + 3] = qv[i].w ^ mk[4 * i + 3];
      });
      float y[D];
      float sc;
      if constexpr (ROT == 0) {
        srft_fwd_unscaled<D>(hq, y);
        sc = SrftScale<D>::value * p.qscale;
      } else {
        fwht_from_f16<D>(hq, y);
        sc = InvSqrt<D>::value * p.qscale;
      }
      float amax = 0.0f;
      sfor<D>([&](auto I) { amax = fmaxf(amax, fabsf(y[RTQ_CI(I)])); });
      amax *= sc;  // the largest entry of y * sc (rounding is monotonic)
      // scale the query by 2^-e so that its largest entry lies in [2^13, 2^14):
      // the fp16 high part cannot overflow and the low part keeps its bits.
      // y * (sc 2^-e) is (y * sc) 2^-e exactly: one multiply per entry.
      const int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 14 : 0;
      const float f = __builtin_ldexpf(sc, -e);
      float* dst = stage + lane * C::QROW;
      sfor<D / 4>([&](auto I) {
        constexpr int i = RTQ_CI(I);
        *reinterpret_cast<float4*>(dst + 4 * i) = make_float4(y[4 * i] * f, y[4 * i + 1] * f, y[4 * i + 2] * f,
                                                              y[4 * i + 3] * f);
      });
      qexp[lane] = e;
    }
  }
  __syncthreads();

  // q.k B operand, k-step j: column n < 8 holds the fp16 high part of query
  // n, column n + 8 its low part; lane group h supplies dims
  // 32j + 8h + {v, v + 4} as pair v (the order key_pair produces).
  // Pair v of odd v meets key codes held 16 times larger (key_pair), so it
  // carries 1/16 (exact: a power of two).  key_bias[gi]: the MFMA start
  // value of score group gi in this lane's column, -8 2^-24 times the sum of
  // the column's query parts over the group's dims (key_pair's bias).
  constexpr bool kBiasedKeys = D <= 128;  // key_pair (else code_pair and no bias)
  f16x8_t bq[C::KS];
  float key_bias[C::SPR];
  {
    const int g = n & 7;
    const bool valid = g < G;
    const float* src = stage + g * C::QROW;
    float part_sum[C::KS];
    const f16x2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    sfor<C::KS>([&](auto J) {
      constexpr int j = RTQ_CI(J);
      uint32_t wds[4];
      float ps = 0.0f;
      const float4 lo4 = valid ? *reinterpret_cast<const float4*>(src + 32 * j + 8 * h) : make_float4(0, 0, 0, 0);
      const float4 hi4 = valid ? *reinterpret_cast<const float4*>(src + 32 * j + 8 * h + 4) : make_float4(0, 0, 0, 0);
      const float av[4] = {lo4.x, lo4.y, lo4.z, lo4.w}, bv[4] = {hi4.x, hi4.y, hi4.z, hi4.w};
      sfor<4>([&](auto V) {
        constexpr int v = RTQ_CI(V);
        // the high parts (a, b) and the residuals a - high, b - high (exact in
        // fp32: one v_fma_mix each), both rounded to fp16 pairs
        const float a = av[v], b = bv[v];
        const uint32_t hp = pack_f16x2(a, b);
        const uint32_t lp = pack_f16x2(residual_of_half<0>(a, hp), residual_of_half<1>(b, hp));
        uint32_t x = n < 8 ? hp : lp;
        ps = __builtin_amdgcn_fdot2(as_h2(x), ones, ps, false);
        if constexpr (kBiasedKeys && (v & 1)) x = as_u32(as_h2(x) * (f16x2_t){(_Float16)0.0625f, (_Float16)0.0625f});
        wds[v] = x;
      });
      bq[j] = pack8(as_h2(wds[0]), as_h2(wds[1]), as_h2(wds[2]), as_h2(wds[3]));
      part_sum[j] = kBiasedKeys ? sum_over_row_groups(ps) : 0.0f;
    });
    sfor<C::SPR>([&](auto GI) {
      constexpr int gi = RTQ_CI(GI), per = GR / 32;
      float t = 0.0f;
      sfor<per>([&](auto JJ) { t += part_sum[gi * per + RTQ_CI(JJ)]; });
      key_bias[gi] = kBiasedKeys ? t * -4.76837158203125e-7f : 0.0f;  // -8 * 2^-24
    });
  }
  // 2^e of the query of this lane's column (its stage row was scaled by 2^-e).
  // Columns without a query have a zero operand: their scores are 0, their
  // softmax stays finite and nothing reads their outputs, so they need no
  // mask; lanes n + 8 hold copies of columns n < 8 (add_ror8).
  const float my_scale =
      __builtin_ldexpf(1.0f, ((n & 7) < G ? qexp[n & 7] : 0) + (kBiasedKeys ? 24 : 0));  // key_pair's 2^-24 too
  const bool q_lane = n < G;  // lanes whose outputs are merged
  if constexpr (C::DENSE_ROT) __syncthreads();  // the stage in the work slot is read; the ring may refill it

  f32x4_t acc[C::NT];
  sfor<C::NT>([&](auto I) { acc[RTQ_CI(I)] = (f32x4_t){0.0f, 0.0f, 0.0f, 0.0f}; });
  float m_run = kNegBig, l_run = 0.0f;

  // p.v A operand: lane n reads code word dw of each token row (and word
  // dw + 16 at d = 256); tile i covers dims 8n + i (d = 128), 128 (i / 8) +
  // 8n + i % 8 (d = 256), or 8(n & 7) + 4(n >> 3) + i (d = 64).
  constexpr int WH = D == 256 ? 2 : 1;  // code words per lane and token row
  const int dw = D == 64 ? (n & 7) : n;
  const uint32_t vsel = (D == 64 && n >= 8) ? 0x07060302u : 0x05040100u;

  // one chunk in ring slot B (chunk c - c_begin lives in slot (c - c_begin) % BUFS);
  // BUFS - 1 chunks are in flight while one is computed
  auto chunk = [&](auto B, int c) {
    constexpr int NB = C::BUFS;
    constexpr int b = RTQ_CI(B);
    constexpr int nb = (b + NB - 1) % NB;  // slot of chunk c + NB - 1
    uint8_t* const buf = b == 0 ? slot0 + w * C::BUF : b == 1 ? slot1 + w * C::BUF : slot2 + w * C::BUF;
    uint8_t* const next = nb == 0 ? slot0 + w * C::BUF : nb == 1 ? slot1 + w * C::BUF : slot2 + w * C::BUF;
    if (NB > 2 && c + 1 < c_end) wait_vmcnt<C::NDMA>();
    else wait_vmcnt<0>();
    lds_sync();
    if (c + NB - 1 < c_end) load_chunk(c + NB - 1, next);
    const uint8_t* kc = buf;
    const uint8_t* vc = buf + C::CODE_BYTES;
    const uint8_t* ks = buf + 2 * C::CODE_BYTES;
    const uint8_t* vs = ks + C::SCALE_BYTES;
    const int tok0 = c * kChunk;
    const bool full = tok0 + kChunk <= T;

    // ---- scores of tokens 16 tau + 4h + r (column n) ----
    float sc[2][4];
    sfor<2>([&](auto TAU) {
      constexpr int tau = RTQ_CI(TAU);
      const int lr = lrow<D>(16 * tau + n);
      const uint8_t* rowp = kc + lr * C::RB + 4 * h;
      const int sw = swz<D>(lr);
      uint32_t kw[C::KS];
      sfor<C::KS>([&](auto J) { kw[RTQ_CI(J)] = *reinterpret_cast<const uint32_t*>(rowp + 16 * (RTQ_CI(J) ^ sw)); });
      constexpr int SW = C::SLOT / 4;  // scale words per token
      uint32_t sk[4 * SW];             // tokens 16 tau + 4h + r: words SW r .. SW r + SW - 1
      sfor<SW>([&](auto Q) {
        const uint4 a = *reinterpret_cast<const uint4*>(ks + C::SLOT * (16 * tau + 4 * h) + 16 * RTQ_CI(Q));
        sk[4 * RTQ_CI(Q)] = a.x; sk[4 * RTQ_CI(Q) + 1] = a.y; sk[4 * RTQ_CI(Q) + 2] = a.z; sk[4 * RTQ_CI(Q) + 3] = a.w;
      });
      f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
      sfor<C::SPR>([&](auto GI) {
        constexpr int gi = RTQ_CI(GI);
        f32x4_t part = {key_bias[gi], key_bias[gi], key_bias[gi], key_bias[gi]};
        sfor<GR / 32>([&](auto JJ) {
          constexpr int j = gi * (GR / 32) + RTQ_CI(JJ);
          const uint32_t x = kw[j];
          if constexpr (kBiasedKeys)
            part = mfma(pack8(key_pair<0>(x), key_pair<1>(x), key_pair<2>(x), key_pair<3>(x)), bq[j], part);
          else
            part = mfma(pack8(code_pair<0>(x), code_pair<1>(x), code_pair<2>(x), code_pair<3>(x)), bq[j], part);
        });
        sfor<4>([&](auto R) {
          constexpr int r = RTQ_CI(R);
          s[r] = half_fma<gi & 1>(sk[SW * r + (gi >> 1)], part[r], s[r]);
        });
      });
      // scores in units of 1 / my_scale (base-2 units once multiplied by it);
      // only a chunk that holds the stream's last token has tokens to mask
      sfor<4>([&](auto R) { sc[tau][RTQ_CI(R)] = add_ror8(s[RTQ_CI(R)]); });
      if (!full) {
        asm volatile("");  // a branch, not four selects on every chunk
        sfor<4>([&](auto R) {
          constexpr int r = RTQ_CI(R);
          if (tok0 + 16 * tau + 4 * h + r >= T) sc[tau][r] = -__builtin_inff();
        });
      }
    });

    // ---- online softmax (base 2) over the chunk, per query column ----
    // The running max moves only when a score passes it by more than 8
    // (weights stay <= 2^8, well inside fp16), so the accumulators are
    // rescaled a handful of times per stream instead of on most chunks.
    float cmax = max3f(max3f(sc[0][0], sc[0][1], sc[0][2]), max3f(sc[0][3], sc[1][0], sc[1][1]),
                       max3f(sc[1][2], sc[1][3], sc[1][3]));
    cmax = max_over_row_groups(cmax) * my_scale;  // the factor is a power of two: max and scaling commute
    const bool grow = cmax > m_run + kRescaleSlack;
    if (__ballot(grow)) {
      const float m_new = grow ? cmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      sfor<C::NT>([&](auto I) { acc[RTQ_CI(I)] *= alpha; });
      m_run = m_new;
    }
    float pr[2][4];
    sfor<2>([&](auto TAU) {
      sfor<4>([&](auto R) {
        pr[RTQ_CI(TAU)][RTQ_CI(R)] =
            __builtin_amdgcn_exp2f(__builtin_fmaf(sc[RTQ_CI(TAU)][RTQ_CI(R)], my_scale, -m_run));
      });
    });
    // P^T operand: element 4 tau + r = token 16 tau + 4h + r of query n.  The
    // denominator sums these fp16 weights themselves (v_dot2_f32_f16 with
    // (1, 1): exact), so numerator and denominator use the same weights.
    const f16x2_t p01 = {(_Float16)pr[0][0], (_Float16)pr[0][1]}, p23 = {(_Float16)pr[0][2], (_Float16)pr[0][3]};
    const f16x2_t p45 = {(_Float16)pr[1][0], (_Float16)pr[1][1]}, p67 = {(_Float16)pr[1][2], (_Float16)pr[1][3]};
    const f16x8_t pb = pack8(p01, p23, p45, p67);
    {
      const f16x2_t one = {(_Float16)1.0f, (_Float16)1.0f};
      float psum = __builtin_amdgcn_fdot2(p01, one, 0.0f, false);
      psum = __builtin_amdgcn_fdot2(p23, one, psum, false);
      psum = __builtin_amdgcn_fdot2(p45, one, psum, false);
      l_run += __builtin_amdgcn_fdot2(p67, one, psum, false);
    }

    // ---- values: V^T operand of tokens (a, b) = pair v of lane group h ----
    uint32_t ylo[WH][4], yhi[WH][4], s2[WH][4];
    sfor<4>([&](auto V) {
      constexpr int v = RTQ_CI(V);
      const int ta = 16 * (v >> 1) + 4 * h + 2 * (v & 1), tb = ta + 1;
      const int la = lrow<D>(ta), lb = lrow<D>(tb);
      sfor<WH>([&](auto HH) {
        constexpr int hh = RTQ_CI(HH);
        const int wd = dw + 16 * hh;
        const uint32_t xa = *reinterpret_cast<const uint32_t*>(vc + la * C::RB + 16 * ((wd >> 2) ^ swz<D>(la)) + 4 * (wd & 3));
        const uint32_t xb = *reinterpret_cast<const uint32_t*>(vc + lb * C::RB + 16 * ((wd >> 2) ^ swz<D>(lb)) + 4 * (wd & 3));
        if constexpr (D >= 128) {
          ylo[hh][v] = __builtin_amdgcn_perm(xb, xa, 0x05040100u);
          yhi[hh][v] = __builtin_amdgcn_perm(xb, xa, 0x07060302u);
        } else {
          ylo[hh][v] = __builtin_amdgcn_perm(xb, xa, vsel);
          yhi[hh][v] = ylo[hh][v];
        }
        const int vgi = (8 * wd) / GR;  // the scale group of those dims
        const uint16_t sa = *reinterpret_cast<const uint16_t*>(vs + C::SLOT * ta + 2 * vgi);
        const uint16_t sb2 = *reinterpret_cast<const uint16_t*>(vs + C::SLOT * tb + 2 * vgi);
        s2[hh][v] = (uint32_t)sa | ((uint32_t)sb2 << 16);  // value_pair16 carries the 1/16 of kVShift
      });
    });
    sfor<C::NT>([&](auto I) {
      constexpr int i = RTQ_CI(I);
      constexpr int k = i & 3, hh = i / 8;
      f16x2_t a[4];
      sfor<4>([&](auto V) {
        constexpr int v = RTQ_CI(V);
        const uint32_t y = (D >= 128 && (i & 4)) ? yhi[hh][v] : ylo[hh][v];
        a[v] = value_pair16<k>(y) * as_h2(s2[hh][v]);
      });
      acc[i] = mfma(pack8(a[0], a[1], a[2], a[3]), pb, acc[i]);
    });
  };
#pragma unroll 1
  for (int c = c_begin; c < c_end; c += C::BUFS) {
    chunk(ic<0>{}, c);
    if (c + 1 >= c_end) break;
    chunk(ic<1>{}, c + 1);
    if constexpr (C::BUFS > 2) {
      if (c + 2 >= c_end) break;
      chunk(ic<2>{}, c + 2);
    }
  }

  // The fp16 window's loads go out now when this workgroup is the only one
  // of its stream (their latency then overlaps the merge); with token splits
  // only the workgroup that merges them reads the window.
  const bool has_window = p.win != nullptr && p.win_tokens > 0;
  const int64_t wrow_k = ((int64_t)layer * 2 * p.streams + stream) * p.win_cap;
  const int64_t wrow_v = wrow_k + (int64_t)p.streams * p.win_cap;
  WindowRegs<D> wregs;
  if (has_window && p.splits == 1) wregs.load(p, wrow_k, wrow_v, qrow, G);

  // ---- merge the partials of each stream's waves ----
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  __syncthreads();  // every wave is done with its ring; the merge area aliases it
  float* ow = reinterpret_cast<float*>(slot0);                  // [kWaves][kMaxQ][QROW]
  float* mw = ow + kWaves * kMaxQ * C::QROW;                    // [kWaves][kMaxQ]
  float* lw = mw + kWaves * kMaxQ;                              // [kWaves][kMaxQ]
  if (q_lane) {
    if (h == 0) {
      mw[w * kMaxQ + n] = m_run;
      lw[w * kMaxQ + n] = l_run;
    }
    float* dst = ow + (w * kMaxQ + n) * C::QROW;
    sfor<C::NT>([&](auto I) {
      constexpr int i = RTQ_CI(I);
      sfor<4>([&](auto R) {
        constexpr int r = RTQ_CI(R);
        const int mrow = 4 * h + r;  // output row of the O^T tile = dim lane index
        const int dim = D == 64 ? 8 * (mrow & 7) + 4 * (mrow >> 3) + i : 128 * (i / 8) + 8 * mrow + i % 8;
        dst[dim] = acc[i][r];
      });
    });
  }
  __syncthreads();
  static_assert(kStreams == 1, "the split partials assume one stream per workgroup");
  // the merged output of query g, dim: the stage row (one lane per query
  // rotates it back), or at d = 256 the transposed work area
  // (the SRFT inverse below is srft_inv_hartley, whose input factor
  // 1/sqrt(2d) is folded in here)
  constexpr float kOutFold = (ROT == 0 && !C::DENSE_ROT) ? HartleyIn<D>::value : 1.0f;
  auto put_out = [&](int g, int dim, float val) {
    if constexpr (C::DENSE_ROT) vt_all[dim * kMaxQ + g] = val;
    else stage_all[g * C::QROW + dim] = val;
  };
  // the int4 part's running max and denominator per query (window merge)
  __shared__ float mq[kMaxQ], lq[kMaxQ];
  float* const mine = p.splits > 1 ? p.part + ((int64_t)pair * p.splits + split) * part_floats(G, D) : nullptr;
  for (int idx = threadIdx.x; idx < G * D; idx += 64 * kWaves) {
    const int g = idx / D, dim = idx % D;
    float mx = kNegBig;
    for (int ww = 0; ww < kWaves; ++ww) mx = fmaxf(mx, mw[ww * kMaxQ + g]);
    float num = 0.0f, den = 0.0f;
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = __builtin_amdgcn_exp2f(mw[ww * kMaxQ + g] - mx);
      den = __builtin_fmaf(f, lw[ww * kMaxQ + g], den);
      num = __builtin_fmaf(f, ow[(ww * kMaxQ + g) * C::QROW + dim], num);
    }
    if (p.splits == 1) {
      // den >= 1 when the stream has int4 tokens (the max score has weight 1)
      put_out(g, dim, den > 0.0f ? num * (kOutFold / kVShift) / den : 0.0f);
      if (dim == 0) {
        mq[g] = mx;
        lq[g] = den;
      }
    } else {
      publish(mine + idx, num);
      if (dim == 0) {
        publish(mine + G * D + g, mx);
        publish(mine + G * D + G + g, den);
      }
    }
  }
  if (p.splits > 1) {
    // Publish this split's partial; the workgroup that completes the count
    // merges all of them (no workgroup ever waits for another).
    // The partials are agent-scope relaxed atomics: global accesses with sc1,
    // coherent across the XCDs' L2 caches (LLVM AMDGPUUsage, memory model for
    // GFX942).  An agent-scope release would add an L2 writeback and an
    // acquire an L2 invalidate, which only ordinary (non-sc1) accesses need;
    // what remains of the release, waiting for the stores before the count
    // moves, is done here, and every read of a partial is an sc1 load issued
    // after the count's fetch_add has returned.
    __shared__ int is_last;
    wait_vmcnt<0>();  // this lane's partial stores are complete
    __syncthreads();
    if (threadIdx.x == 0)
      is_last = __hip_atomic_fetch_add(p.count + pair, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(p.splits - 1);
    __syncthreads();
    if (!is_last) return;
    const float* first = p.part + (int64_t)pair * p.splits * part_floats(G, D);
    for (int idx = threadIdx.x; idx < G * D; idx += 64 * kWaves) {
      const int g = idx / D, dim = idx % D;
      float mx = kNegBig;
      for (int sp = 0; sp < p.splits; ++sp) mx = fmaxf(mx, collect(first + sp * part_floats(G, D) + G * D + g));
      float num = 0.0f, den = 0.0f;
      for (int sp = 0; sp < p.splits; ++sp) {
        const float* ps = first + sp * part_floats(G, D);
        const float f = __builtin_amdgcn_exp2f(collect(ps + G * D + g) - mx);
        den = __builtin_fmaf(f, collect(ps + G * D + G + g), den);
        num = __builtin_fmaf(f, collect(ps + idx), num);
      }
      put_out(g, dim, den > 0.0f ? num * (kOutFold / kVShift) / den : 0.0f);
      if (dim == 0) {
        mq[g] = mx;
        lq[g] = den;
      }
    }
    if (threadIdx.x == 0) __hip_atomic_store(p.count + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();

  // ---- the fp16 window's part (the merge area of ring slot 0 is free now) ----
  // weights and coef at the start of ring slot 0; the phase sums after them
  // at d = 256 (ring slot 1 holds the rotation area there), else in ring slot 1
  using WL = WindowLds<D>;
  float* const wsc = reinterpret_cast<float*>(slot0);     // [kMaxWindow][kMaxQ] weights
  float* const coef = wsc + kMaxWindow * kMaxQ;            // [kMaxQ]
  float* const ows = reinterpret_cast<float*>(C::WORK_SLOT == 1 ? slot0 + WL::WEIGHT_BYTES : slot1);  // [kMaxQ][D]
  static_assert((C::DENSE_ROT && C::WORK_SLOT == 1) ? WL::WEIGHT_BYTES + WL::RED_BYTES <= C::SLOT_ARRAY
                             : WL::WEIGHT_BYTES <= C::SLOT_ARRAY && WL::RED_BYTES <= C::SLOT_ARRAY,
                "the window area fits the free ring slots");
  if (has_window) {
    if (p.splits > 1) wregs.load(p, wrow_k, wrow_v, qrow, G);
    window_part<D>(p, wregs, G, seed_of_row(p, row_v), mq, lq, wsc, coef, ows);
  }

  // ---- rotate the outputs back: o = D_V R^T o_rot ----
  if constexpr (C::DENSE_ROT) {
    constexpr int NQ = kMaxQ / C::TPC;
    const int t = threadIdx.x, c = t % D, g0 = (t / D) * NQ;
    float2* tw = reinterpret_cast<float2*>(vt_all + D * kMaxQ);
    if (ROT == 0 && t < D) tw[t] = twiddle<D>(t);
    __syncthreads();
    const float sv = sign_bit(seed_of_row(p, row_v), (uint32_t)c) ? -1.0f : 1.0f;
    _Float16* o16 = reinterpret_cast<_Float16*>(p.out);
    auto store = [&](int g, float u) {
      if (has_window) u = __builtin_fmaf(coef[g], u, ows[g * D + c]);
      o16[(qrow + g) * D + c] = (_Float16)(sv * u);
    };
    if (g0 < G) {
      if (NQ == 8 && G <= 4) {
        float u[4];
        dense_inverse<D, ROT, 4>(vt_all, tw, c, u);
        sfor<4>([&](auto Gi) {
          if (RTQ_CI(Gi) < G) store(RTQ_CI(Gi), u[RTQ_CI(Gi)]);
        });
      } else {
        float u[NQ];
        dense_inverse<D, ROT, NQ>(vt_all + g0, tw, c, u);
        sfor<NQ>([&](auto Gi) {
          if (g0 + RTQ_CI(Gi) < G) store(g0 + RTQ_CI(Gi), u[RTQ_CI(Gi)]);
        });
      }
    }
  } else if (lead) {
    uint32_t mvs[D / 2];
    wave_sign_masks<D>(seed_of_row(p, row_v), lane, mvs);
    if (lane < G) {
      float z[D], u[D];
      const float* src = stage + lane * C::QROW;
      sfor<D / 4>([&](auto I) {
        constexpr int i = RTQ_CI(I);
        const float4 f = *reinterpret_cast<const float4*>(src + 4 * i);
        z[4 * i] = f.x; z[4 * i + 1] = f.y; z[4 * i + 2] = f.z; z[4 * i + 3] = f.w;
      });
      if constexpr (ROT == 0) {
        srft_inv_hartley<D>(z, u);
      } else {
        fwht_f32<D>(z);
        sfor<D>([&](auto I) { u[RTQ_CI(I)] = z[RTQ_CI(I)] * InvSqrt<D>::value; });
      }
      if (has_window) {
        const float a = coef[lane];
        const float* wrow = ows + lane * D;
        sfor<D / 4>([&](auto I) {
          constexpr int i = RTQ_CI(I);
          const float4 f = *reinterpret_cast<const float4*>(wrow + 4 * i);
          u[4 * i] = __builtin_fmaf(a, u[4 * i], f.x);
          u[4 * i + 1] = __builtin_fmaf(a, u[4 * i + 1], f.y);
          u[4 * i + 2] = __builtin_fmaf(a, u[4 * i + 2], f.z);
          u[4 * i + 3] = __builtin_fmaf(a, u[4 * i + 3], f.w);
        });
      }
      uint4* dst = p.out + (qrow + lane) * (D / 8);
      sfor<D / 8>([&](auto I) {
        constexpr int i = RTQ_CI(I);
        dst[i] = make_uint4(pack_f16x2(u[8 * i], u[8 * i + 1]) ^ mvs[4 * i],
                            pack_f16x2(u[8 * i + 2], u[8 * i + 3]) ^ mvs[4 * i + 1],
                            pack_f16x2(u[8 * i + 4], u[8 * i + 5]) ^ mvs[4 * i + 2],
                            pack_f16x2(u[8 * i + 6], u[8 * i + 7]) ^ mvs[4 * i + 3]);
      });
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

using KernelFn = const void*;


template <int ROT>
KernelFn find_kernel(int d, int g) {
#define RTQ_ATTN_CASE(DD, GG) \
  if (d == DD && g == GG) return reinterpret_cast<KernelFn>(&attn_decode_kernel<DD, GG, ROT>);
  RTQ_ATTN_CASE(64, 32) RTQ_ATTN_CASE(64, 64)
  RTQ_ATTN_CASE(128, 32) RTQ_ATTN_CASE(128, 64) RTQ_ATTN_CASE(128, 128)
  RTQ_ATTN_CASE(256, 32) RTQ_ATTN_CASE(256, 64) RTQ_ATTN_CASE(256, 128) RTQ_ATTN_CASE(256, 256)
#undef RTQ_ATTN_CASE
  return nullptr;
}

// Block index of a row under the seed rule, before the modulo.
inline int64_t block_of(int64_t row, int64_t rps) { return rps ? row / rps : 0; }

// True when every token of every (layer, kv, stream) has the seed of its
// token 0, so one sign vector serves the whole key (or value) sequence.
bool seeds_constant(int64_t layers, int64_t streams, int64_t tokens, const int64_t (&st)[4], int64_t rps,
                    int32_t period) {
  if (rps == 0 || period == 1 || tokens == 1) return true;
  // each token step moves a whole number of seed periods
  if (st[3] % rps == 0 && period != 0 && (st[3] / rps) % period == 0) return true;
  for (int64_t l = 0; l < layers; ++l)
    for (int64_t kv = 0; kv < 2; ++kv)
      for (int64_t s = 0; s < streams; ++s) {
        const int64_t r0 = l * st[0] + kv * st[1] + s * st[2];
        if (block_of(r0, rps) != block_of(r0 + (tokens - 1) * st[3], rps)) return false;
      }
  return true;
}

// Token splits.  Two workgroups per CU, 512 on MI355X's 256 CUs, is what
// every head dimension holds (d = 64 and 128 hold three).  Fewer (layer,
// stream) pairs leave CUs idle, so each stream's chunks are spread over as
// many workgroups as fit in that one round (at least kMinChunksPerSplit
// chunks each).  More splits measured slower, each workgroup paying its own
// query rotation and merge: counting three per CU gives the SmolLM2-360M
// cache four splits instead of three, 22.9-23.1 against 21.7-21.9 us.
constexpr int64_t kResidentWorkgroups = 512;
constexpr int64_t kMinChunksPerSplit = 8;
constexpr int64_t kMaxSplits = 64;

int choose_splits(int64_t pairs, int64_t tokens) {
  if (pairs <= 0 || 2 * pairs > kResidentWorkgroups) return 1;
  int64_t s = kResidentWorkgroups / pairs;
  const int64_t by_tokens = (tokens + kChunk - 1) / kChunk / kMinChunksPerSplit;
  if (s > by_tokens) s = by_tokens;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 2 ? 1 : (int)s;
}

// Workspace of a launch with `splits` splits: the per-pair counters (padded
// to 256 bytes), then the partials.
uint64_t workspace_bytes(int64_t pairs, int splits, int g, int d) {
  if (splits < 2) return 0;
  return (uint64_t)((pairs * 4 + 255) & ~(int64_t)255) + (uint64_t)pairs * splits * part_floats(g, d) * 4;
}

bool overlaps(const void* a, __int128 na, const void* b, __int128 nb) {
  const __int128 a0 = (__int128)(uintptr_t)a, b0 = (__int128)(uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

rtq_status scratch_on_current_device(hipStream_t stream, void** out);
extern const size_t kScratchBytesExtern;

// use_scratch: the split workspace is the library's static scratch (set up
// here, after every argument check), and workspace must be null.
rtq_status run(int rot, const void* q, const void* codes, const void* scales, void* out, int32_t layers,
               int32_t streams, int32_t tokens, int32_t q_per_kv, int32_t d, int32_t group, const int64_t (&st)[4],
               uint64_t seed, int64_t rps, int32_t period, float softmax_scale, const void* win, int32_t win_cap,
               int32_t win_tokens, void* workspace, size_t workspace_size, hipStream_t stream,
               bool use_scratch = false) {
  if (layers < 0 || streams < 0 || rps < 0 || period < 0) return RTQ_ERR_INVALID_ARG;
  for (int i = 0; i < 4; ++i)
    if (st[i] < 0) return RTQ_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale) || softmax_scale > 3.0e38f || softmax_scale < -3.0e38f)
    return RTQ_ERR_INVALID_ARG;
  // One stream per workgroup.  (Two adjacent streams per 8-wave workgroup,
  // to share the 128-byte lines of a time-major cache, measured slower: 537
  // vs 414 us on the Qwen2.5-1.5B decode cache, as the whole CU then waits
  // at the workgroup's barriers.)
  const KernelFn fn = rot == 0 ? find_kernel<0>(d, group) : find_kernel<1>(d, group);
  if (!fn) return RTQ_ERR_UNSUPPORTED;
  if (q_per_kv < 1) return RTQ_ERR_INVALID_ARG;
  if (q_per_kv > kMaxQ) return RTQ_ERR_UNSUPPORTED;
  if (win_tokens < 0 || win_cap < 0 || (win == nullptr && win_tokens != 0)) return RTQ_ERR_INVALID_ARG;
  if (win_tokens > kMaxWindow) return RTQ_ERR_UNSUPPORTED;
  if (win_tokens > win_cap || (win != nullptr && !aligned16(win))) return RTQ_ERR_INVALID_ARG;
  if (layers == 0 || streams == 0) return RTQ_OK;
  // the int4 prefix may be empty only when the window holds the tokens
  if (tokens < (win_tokens > 0 ? 0 : 1) || tokens > 0x7fffff00) return RTQ_ERR_INVALID_ARG;
  const int64_t wgs = (int64_t)layers * streams;
  if (wgs > 0x7fffffff) return RTQ_ERR_INVALID_ARG;
  if (!q || !codes || !scales || !out) return RTQ_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(codes) || !aligned16(scales) || !aligned16(out)) return RTQ_ERR_INVALID_ARG;
  if ((workspace == nullptr) != (workspace_size == 0) || !aligned16(workspace)) return RTQ_ERR_INVALID_ARG;
  // largest row the kernel reads, in 128-bit arithmetic (none without int4 tokens)
  const __int128 max_row = tokens == 0 ? -1 : (__int128)(layers - 1) * st[0] + st[1] +
                                                  (__int128)(streams - 1) * st[2] + (__int128)(tokens - 1) * st[3];
  if (max_row >= ((__int128)1 << 56)) return RTQ_ERR_INVALID_ARG;
  if (tokens > 0 && !seeds_constant(layers, streams, tokens, st, rps, period)) return RTQ_ERR_INVALID_ARG;
  const __int128 qo_bytes = (__int128)layers * streams * q_per_kv * d * 2;
  const __int128 code_bytes = (max_row + 1) * (d / 2), scale_bytes = (max_row + 1) * 2 * (d / group);
  const __int128 win_bytes = win_tokens > 0 ? (__int128)layers * 2 * streams * win_cap * d * 2 : 0;
  if (win_tokens > 0 && (overlaps(out, qo_bytes, win, win_bytes) ||
                         (workspace && overlaps(workspace, workspace_size, win, win_bytes))))
    return RTQ_ERR_INVALID_ARG;
  if (overlaps(out, qo_bytes, q, qo_bytes) || overlaps(out, qo_bytes, codes, code_bytes) ||
      overlaps(out, qo_bytes, scales, scale_bytes))
    return RTQ_ERR_INVALID_ARG;
  if (workspace && (overlaps(workspace, workspace_size, q, qo_bytes) || overlaps(workspace, workspace_size, out, qo_bytes) ||
                    overlaps(workspace, workspace_size, codes, code_bytes) ||
                    overlaps(workspace, workspace_size, scales, scale_bytes)))
    return RTQ_ERR_INVALID_ARG;
  if (use_scratch) {
    if (workspace != nullptr) return RTQ_ERR_INVALID_ARG;
    const rtq_status s = scratch_on_current_device(stream, &workspace);
    if (s != RTQ_OK) return s;
    workspace_size = kScratchBytesExtern;
  }
  // as many splits as the policy asks for and the workspace holds
  int splits = workspace ? choose_splits(wgs, tokens) : 1;
  while (splits > 1 && (workspace_bytes(wgs, splits, q_per_kv, d) > workspace_size || wgs * splits > 0x7fffffff))
    --splits;
  Params p;
  p.q = static_cast<const uint4*>(q);
  p.codes = static_cast<const uint8_t*>(codes);
  p.scales = static_cast<const uint8_t*>(scales);
  p.out = static_cast<uint4*>(out);
  p.stride_layer = st[0];
  p.stride_kv = st[1];
  p.stride_stream = st[2];
  p.stride_token = st[3];
  p.seed = seed;
  p.rows_per_seed = rps;
  p.seed_period = period;
  p.streams = streams;
  p.tokens = tokens;
  p.q_per_kv = q_per_kv;
  p.qscale = (float)((double)softmax_scale * 1.4426950408889634074);
  p.splits = splits;
  p.count = splits > 1 ? static_cast<uint32_t*>(workspace) : nullptr;
  p.part = splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ((wgs * 4 + 255) & ~(int64_t)255))
                      : nullptr;
  p.win = win_tokens > 0 ? static_cast<const uint4*>(win) : nullptr;
  p.win_cap = win_cap;
  p.win_tokens = win_tokens;
  void* kargs[] = {&p};
  const hipError_t e =
      hipLaunchKernel(fn, dim3((unsigned)(wgs * splits)), dim3(64 * waves_per_stream(d)), kargs, 0, stream);
  return e == hipSuccess ? RTQ_OK : RTQ_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Scratch of srft_attn_decode_noalloc: the split workspace in a file-scope
// device array, for callers that cannot allocate.
// ---------------------------------------------------------------------------

// The largest workspace the split policy asks for: splits happen only with
// at most kResidentWorkgroups / 2 (layer, stream) pairs (counters padded to
// 256 bytes), and pairs * splits <= kResidentWorkgroups partials of at most
// kMaxQ queries at d = 256.
constexpr size_t kScratchBytes =
    (size_t)(((kResidentWorkgroups / 2) * 4 + 255) & ~(int64_t)255) +
    (size_t)kResidentWorkgroups * (size_t)part_floats(kMaxQ, 256) * 4;
static_assert(kScratchBytes == 4228096, "4 MiB + 8 KiB");
const size_t kScratchBytesExtern = kScratchBytes;

// Each GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device, once set up

__global__ void zero_words(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// The device address of `scratch` on the current device.  The first call on
// a device looks it up (the array's name is a host-side stand-in, not a
// device address) and clears it with a kernel on `stream` (not a memset, so
// that a graph capture records a kernel node).
rtq_status scratch_on_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return RTQ_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return RTQ_ERR_HIP;
    hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, stream, static_cast<uint4*>(ptr), kScratchBytes / 16);
    if (hipGetLastError() != hipSuccess) return RTQ_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return RTQ_OK;
}

}  // namespace attn
}  // namespace rtq

#define RTQ_API extern "C" __attribute__((visibility("default")))

RTQ_API rtq_status srft_attn_decode(const void* q_f16, const void* codes_u8, const void* scales_f16, void* out_f16,
                                    int32_t layers, int32_t streams, int32_t tokens, int32_t q_per_kv, int32_t d,
                                    int32_t group, int64_t stride_layer, int64_t stride_kv, int64_t stride_stream,
                                    int64_t stride_token, uint64_t seed, int64_t rows_per_seed,
                                    int32_t seed_period, float softmax_scale, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  const int64_t st[4] = {stride_layer, stride_kv, stride_stream, stride_token};
  return rtq::attn::run(0, q_f16, codes_u8, scales_f16, out_f16, layers, streams, tokens, q_per_kv, d, group, st,
                        seed, rows_per_seed, seed_period, softmax_scale, nullptr, 0, 0, workspace, workspace_bytes,
                        stream);
}

RTQ_API rtq_status srft_attn_decode_window(const void* q_f16, const void* codes_u8, const void* scales_f16,
                                           void* out_f16, int32_t layers, int32_t streams, int32_t tokens,
                                           int32_t q_per_kv, int32_t d, int32_t group, int64_t stride_layer,
                                           int64_t stride_kv, int64_t stride_stream, int64_t stride_token,
                                           uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                           float softmax_scale, const void* window_f16, int32_t window_capacity,
                                           int32_t window_tokens, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  const int64_t st[4] = {stride_layer, stride_kv, stride_stream, stride_token};
  return rtq::attn::run(0, q_f16, codes_u8, scales_f16, out_f16, layers, streams, tokens, q_per_kv, d, group, st,
                        seed, rows_per_seed, seed_period, softmax_scale, window_f16, window_capacity, window_tokens,
                        workspace, workspace_bytes, stream);
}

RTQ_API rtq_status srht_attn_decode(const void* q_f16, const void* codes_u8, const void* scales_f16, void* out_f16,
                                    int32_t layers, int32_t streams, int32_t tokens, int32_t q_per_kv, int32_t d,
                                    int32_t group, int64_t stride_layer, int64_t stride_kv, int64_t stride_stream,
                                    int64_t stride_token, uint64_t seed, int64_t rows_per_seed,
                                    int32_t seed_period, float softmax_scale, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  const int64_t st[4] = {stride_layer, stride_kv, stride_stream, stride_token};
  return rtq::attn::run(1, q_f16, codes_u8, scales_f16, out_f16, layers, streams, tokens, q_per_kv, d, group, st,
                        seed, rows_per_seed, seed_period, softmax_scale, nullptr, 0, 0, workspace, workspace_bytes,
                        stream);
}

RTQ_API rtq_status srht_attn_decode_window(const void* q_f16, const void* codes_u8, const void* scales_f16,
                                           void* out_f16, int32_t layers, int32_t streams, int32_t tokens,
                                           int32_t q_per_kv, int32_t d, int32_t group, int64_t stride_layer,
                                           int64_t stride_kv, int64_t stride_stream, int64_t stride_token,
                                           uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                           float softmax_scale, const void* window_f16, int32_t window_capacity,
                                           int32_t window_tokens, void* workspace, size_t workspace_bytes,
                                           hipStream_t stream) {
  const int64_t st[4] = {stride_layer, stride_kv, stride_stream, stride_token};
  return rtq::attn::run(1, q_f16, codes_u8, scales_f16, out_f16, layers, streams, tokens, q_per_kv, d, group, st,
                        seed, rows_per_seed, seed_period, softmax_scale, window_f16, window_capacity, window_tokens,
                        workspace, workspace_bytes, stream);
}

RTQ_API size_t rtq_attn_workspace_bytes(int32_t layers, int32_t streams, int32_t tokens, int32_t q_per_kv,
                                        int32_t d) {
  if (layers <= 0 || streams <= 0 || tokens < 1 || q_per_kv < 1 || q_per_kv > rtq::attn::kMaxQ || d <= 0)
    return 0;
  const int64_t pairs = (int64_t)layers * streams;
  if (pairs > 0x7fffffff) return 0;
  int splits = rtq::attn::choose_splits(pairs, tokens);
  while (splits > 1 && pairs * splits > 0x7fffffff) --splits;
  return (size_t)rtq::attn::workspace_bytes(pairs, splits, q_per_kv, d);
}

RTQ_API rtq_status srft_attn_decode_noalloc(const void* q_f16, const void* codes_u8, const void* scales_f16,
                                            void* out_f16, int32_t layers, int32_t streams, int32_t tokens,
                                            int32_t q_per_kv, int32_t d, int32_t group, int64_t stride_layer,
                                            int64_t stride_kv, int64_t stride_stream, int64_t stride_token,
                                            uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                            float softmax_scale, hipStream_t stream) {
  // the split plan's workspace must fit the scratch (by construction every plan does)
  if (rtq_attn_workspace_bytes(layers, streams, tokens, q_per_kv, d) > rtq::attn::kScratchBytes)
    return RTQ_ERR_UNSUPPORTED;
  const int64_t st[4] = {stride_layer, stride_kv, stride_stream, stride_token};
  return rtq::attn::run(0, q_f16, codes_u8, scales_f16, out_f16, layers, streams, tokens, q_per_kv, d, group, st,
                        seed, rows_per_seed, seed_period, softmax_scale, nullptr, 0, 0, nullptr, 0, stream,
                        /*use_scratch=*/true);
}
