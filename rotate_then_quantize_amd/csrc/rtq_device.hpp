// rtq_device.hpp -- register-resident building blocks for the fused
// rotate-then-quantize kernels on CDNA4 (gfx950, wave64).
//
// Every transform here works on one K/V vector held entirely in the registers
// of one lane (d <= 128) or of two lanes (d = 256), with compile-time
// register indices: no LDS, no cross-lane traffic and no loops at run time.
//
// Method sources (page title, section):
//   "Quantization Speed Is Often a Kernel Problem", "First, the 17%":
//     K/V vectors are rotated before int4 quantization and un-rotated after
//     dequantization; SRFT flips signs with a seeded +-1 vector and then takes
//     a real FFT (inverse: real inverse FFT); the Hadamard variant (SRHT) is
//     the control.
//   same page, "Fusing four steps into two kernels is not enough": forward =
//     rotate + quantize in one kernel, inverse = dequantize + inverse-rotate
//     in one kernel; one absmax scale per group of 32 values.
//   "Day 9 - Quantization: Shrink the Bytes Themselves", "What Quantization
//     Is, Mathematically" / "How Many Numbers Should One Scale Cover":
//     symmetric int4, scale = absmax / 8, scales stored as fp16.
//   "Chapter 25 - Quantization: The Hardware View", "Kernels: Marlin,
//     CUTLASS, and Why INT4 Packing Needs Special Code": two int4 per byte,
//     w0 in the low nibble.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rtq {

// ---------------------------------------------------------------------------
// Compile-time helpers
// ---------------------------------------------------------------------------

template <int... Is> struct iseq {};
template <int N, int... Is> struct make_iseq : make_iseq<N - 1, N - 1, Is...> {};
template <int... Is> struct make_iseq<0, Is...> { using type = iseq<Is...>; };
template <int I> struct ic { static constexpr int value = I; };

template <typename F, int... Is>
__device__ __forceinline__ void sfor_impl(F& f, iseq<Is...>) {
  (f(ic<Is>{}), ...);
}
// Unrolled loop whose index is a compile-time constant: f(ic<0>{}) .. f(ic<N-1>{}).
template <int N, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  sfor_impl(f, typename make_iseq<N>::type{});
}
#define RTQ_CI(x) (decltype(x)::value)

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }
constexpr int bitrev(int x, int bits) {
  int r = 0;
  for (int i = 0; i < bits; ++i) r = (r << 1) | ((x >> i) & 1);
  return r;
}

// cos(2*pi*t/n) and sin(2*pi*t/n) in double at compile time: exact integer
// reduction of the angle to [0, pi/4], then Taylor series.  consteval: these
// must never run on the GPU.
constexpr double kPi = 3.141592653589793238462643383279502884;
consteval double taylor_sin(double x) {
  double x2 = x * x, term = x, sum = x;
  for (int k = 1; k < 16; ++k) {
    term *= -x2 / ((2.0 * k) * (2.0 * k + 1.0));
    sum += term;
  }
  return sum;
}
consteval double taylor_cos(double x) {
  double x2 = x * x, term = 1.0, sum = 1.0;
  for (int k = 1; k < 16; ++k) {
    term *= -x2 / ((2.0 * k - 1.0) * (2.0 * k));
    sum += term;
  }
  return sum;
}
consteval double cos2pi(long long t, long long n) {
  t %= n;
  if (t < 0) t += n;
  const long long q = (4 * t) / n;      // quadrant
  const long long r = 4 * t - q * n;    // angle inside the quadrant = (pi/2) r / n
  double c, s;
  if (2 * r <= n) {
    const double phi = (kPi / 2.0) * (double)r / (double)n;
    c = taylor_cos(phi);
    s = taylor_sin(phi);
  } else {
    const double psi = (kPi / 2.0) * (double)(n - r) / (double)n;
    c = taylor_sin(psi);
    s = taylor_cos(psi);
  }
  switch (q) {
    case 0: return c;
    case 1: return -s;
    case 2: return -c;
    default: return s;
  }
}
consteval double sin2pi(long long t, long long n) { return cos2pi(4 * t - n, 4 * n); }
consteval double csqrt(double x) {
  double r = x > 1.0 ? x : 1.0;
  for (int i = 0; i < 200; ++i) r = 0.5 * (r + x / r);
  return r;
}

// ---------------------------------------------------------------------------
// fp16 and bit helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float lo_f(uint32_t w) {
  return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu)));
}
__device__ __forceinline__ float hi_f(uint32_t w) {
  return __half2float(__ushort_as_half((unsigned short)(w >> 16)));
}
// Two floats to packed fp16 (round to nearest even): low half = a.
// (v_cvt_pk_f16_f32 written out: left to itself the compiler fuses an fma
// that feeds the conversion into v_fma_mix{lo,hi}_f16, which issue at half
// rate.)
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  uint32_t r;
  asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// fp16 + fp16 and fp16 - fp16 into fp32 with one v_fma_mix_f32 each (the sum
// of two fp16 values is exact in fp32).  SEL_A / SEL_B pick the half (0 = low,
// 1 = high) of each packed operand.
template <int SEL_A, int SEL_B>
__device__ __forceinline__ float mix_add(uint32_t a, uint32_t b) {
  float r;
  if constexpr (SEL_A == 0 && SEL_B == 0)
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
  else if constexpr (SEL_A == 1 && SEL_B == 1)
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
  else if constexpr (SEL_A == 0 && SEL_B == 1)
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
// a - b
template <int SEL_A, int SEL_B>
__device__ __forceinline__ float mix_sub(uint32_t a, uint32_t b) {
  float r;
  if constexpr (SEL_A == 0 && SEL_B == 0)
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[0,0,0] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(b), "v"(a));
  else if constexpr (SEL_A == 1 && SEL_B == 1)
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(b), "v"(a));
  else if constexpr (SEL_A == 0 && SEL_B == 1)
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(b), "v"(a));
  else
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[0,0,1] op_sel_hi:[1,0,1]" : "=v"(r) : "v"(b), "v"(a));
  return r;
}

// Nibble order of a 32-bit word reversed (nibble i <-> nibble 7-i).
__device__ __forceinline__ uint32_t nibble_reverse(uint32_t x) {
  x = __builtin_amdgcn_perm(x, x, 0x00010203u);  // byte reverse
  return ((x >> 4) & 0x0f0f0f0fu) | ((x << 4) & 0xf0f0f0f0u);
}

// ---------------------------------------------------------------------------
// Sign pattern: SplitMix64 (Steele, Lea & Flood 2014).  Output i (0-based) of
// the stream started at state S is mix(S + (i+1)*gamma); the sign of element i
// is -1 iff its bit 63 is set.  The final xor-shift of the mixer leaves bit 63
// unchanged, so it is skipped.
// ---------------------------------------------------------------------------

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

__host__ __device__ __forceinline__ uint32_t sign_bit(uint64_t seed, uint32_t i) {
  uint64_t z = seed + (uint64_t)(i + 1u) * kGamma;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)(z >> 63);
}

// XOR masks that flip the fp16 sign bits of elements 8k .. 8k+7 (four packed
// pairs, low half = even element).
__device__ __forceinline__ uint4 chunk_sign_masks(uint64_t seed, uint32_t k) {
  uint32_t m[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t e = 8u * k + 2u * t;
    m[t] = (sign_bit(seed, e) << 15) | (sign_bit(seed, e + 1u) << 31);
  }
  return make_uint4(m[0], m[1], m[2], m[3]);
}

__device__ __forceinline__ uint64_t row_seed(uint64_t seed, int64_t row, int64_t rows_per_seed,
                                             int32_t seed_period) {
  if (rows_per_seed == 0) return seed;
  uint64_t block = (uint64_t)(row / rows_per_seed);
  if (seed_period != 0) block %= (uint64_t)seed_period;
  return seed + block;
}

__device__ __forceinline__ uint4 xor4(uint4 a, uint4 b) {
  return make_uint4(a.x ^ b.x, a.y ^ b.y, a.z ^ b.z, a.w ^ b.w);
}

// ---------------------------------------------------------------------------
// Complex radix-2 FFT (decimation in time), forward sign exp(-2 pi i / L).
// ---------------------------------------------------------------------------

// (a, b) <- (a + w b, a - w b), w = exp(-2 pi i J / L).
template <int J, int L>
__device__ __forceinline__ void bfly(float& ar, float& ai, float& br, float& bi) {
  if constexpr (J == 0) {
    const float tr = ar - br, ti = ai - bi;
    ar = ar + br;
    ai = ai + bi;
    br = tr;
    bi = ti;
  } else if constexpr (4 * J == L) {  // w = -i, w b = (bi, -br)
    const float tr = ar - bi, ti = ai + br;
    ar = ar + bi;
    ai = ai - br;
    br = tr;
    bi = ti;
  } else {
    constexpr float c = (float)cos2pi(J, L);
    constexpr float s = (float)sin2pi(J, L);
    // w b = (c br + s bi) + i (c bi - s br)
    const float pr = __builtin_fmaf(c, br, __builtin_fmaf(s, bi, ar));
    const float pi = __builtin_fmaf(c, bi, __builtin_fmaf(-s, br, ai));
    br = __builtin_fmaf(2.0f, ar, -pr);
    bi = __builtin_fmaf(2.0f, ai, -pi);
    ar = pr;
    ai = pi;
  }
}

// Stages of length 4 .. M on data already in bit-reversed order after stage 1.
template <int M>
__device__ __forceinline__ void fft_stages_from4(float (&re)[M], float (&im)[M]) {
  constexpr int LOG = ilog2(M);
  sfor<LOG - 1>([&](auto S) {
    constexpr int len = 4 << RTQ_CI(S);
    constexpr int half = len / 2;
    sfor<M / len>([&](auto B) {
      sfor<half>([&](auto J) {
        constexpr int p = RTQ_CI(B) * len + RTQ_CI(J);
        bfly<RTQ_CI(J), len>(re[p], im[p], re[p + half], im[p + half]);
      });
    });
  });
}

// W = DFT_M(x), x_m = xr[m] + i xi[m] (fp32, natural order in and out; the
// bit reversal is register renaming only).
template <int M>
__device__ __forceinline__ void cfft_f32(const float (&xr)[M], const float (&xi)[M], float (&re)[M],
                                         float (&im)[M]) {
  constexpr int LOG = ilog2(M);
  sfor<M / 2>([&](auto I) {
    constexpr int i = RTQ_CI(I);
    constexpr int e = bitrev(2 * i, LOG);
    re[2 * i] = xr[e] + xr[e + M / 2];
    im[2 * i] = xi[e] + xi[e + M / 2];
    re[2 * i + 1] = xr[e] - xr[e + M / 2];
    im[2 * i + 1] = xi[e] - xi[e + M / 2];
  });
  fft_stages_from4<M>(re, im);
}

// ---------------------------------------------------------------------------
// Real-input DFT by even/odd recursion (decimation in time on real data).
//
//   X_k = sum_n u_n exp(-2 pi i k n / N),  k = 0 .. N/2 (unnormalized).
// With E, O the real DFTs of the even and odd samples (length N/2):
//   X_k = E_k + w^k O_k  and  X_{N/2-k} = conj(E_k - w^k O_k),  k = 0 .. N/4,
// where E_0, O_0, E_{N/4}, O_{N/4} are real.  Each bin pair costs six FMAs:
// X_k from two fused multiply-adds per component, X_{N/2-k} as 2E - X_k.
// The recursion ends at N = 4, whose first add/sub layer reads the fp16
// samples directly (v_fma_mix).  Samples u_j live in packed pairs, u_j = half
// (j % 2) of h[j / 2]; this call transforms u_{OFF}, u_{OFF+S}, ... .
// ---------------------------------------------------------------------------

template <int N, int S, int OFF, int H>
__device__ __forceinline__ void rdft(const uint32_t (&h)[H], float (&xr)[N / 2 + 1], float (&xi)[N / 2 + 1]) {
  if constexpr (N == 4) {
    constexpr int a = OFF, b = OFF + S, c = OFF + 2 * S, d = OFF + 3 * S;
    static_assert((a & 1) == (c & 1) && (b & 1) == (d & 1), "leaf pairs share a half");
    const float t0 = mix_add<a & 1, c & 1>(h[a / 2], h[c / 2]);
    const float t1 = mix_sub<a & 1, c & 1>(h[a / 2], h[c / 2]);
    const float t2 = mix_add<b & 1, d & 1>(h[b / 2], h[d / 2]);
    const float t3 = mix_sub<b & 1, d & 1>(h[b / 2], h[d / 2]);
    xr[0] = t0 + t2;
    xr[2] = t0 - t2;
    xr[1] = t1;
    xi[1] = -t3;
    xi[0] = 0.0f;
    xi[2] = 0.0f;
  } else {
    float er[N / 4 + 1], ei[N / 4 + 1], orr[N / 4 + 1], oi[N / 4 + 1];
    rdft<N / 2, 2 * S, OFF, H>(h, er, ei);
    rdft<N / 2, 2 * S, OFF + S, H>(h, orr, oi);
    xr[0] = er[0] + orr[0];
    xi[0] = 0.0f;
    xr[N / 2] = er[0] - orr[0];
    xi[N / 2] = 0.0f;
    xr[N / 4] = er[N / 4];  // w^{N/4} = -i and E, O are real there
    xi[N / 4] = -orr[N / 4];
    sfor<N / 4 - 1>([&](auto K) {
      constexpr int k = RTQ_CI(K) + 1;
      constexpr float c = (float)cos2pi(k, N), s = (float)sin2pi(k, N);  // w^k = c - i s
      xr[k] = __builtin_fmaf(c, orr[k], __builtin_fmaf(s, oi[k], er[k]));
      xi[k] = __builtin_fmaf(c, oi[k], __builtin_fmaf(-s, orr[k], ei[k]));
      xr[N / 2 - k] = __builtin_fmaf(2.0f, er[k], -xr[k]);
      xi[N / 2 - k] = __builtin_fmaf(-2.0f, ei[k], xi[k]);
    });
  }
}

// The same recursion on fp32 samples g_{OFF}, g_{OFF+S}, ... (the leaf adds
// and subtracts fp32 values).
template <int N, int S, int OFF, int L>
__device__ __forceinline__ void rdft_f32(const float (&g)[L], float (&xr)[N / 2 + 1], float (&xi)[N / 2 + 1]) {
  if constexpr (N == 4) {
    constexpr int a = OFF, b = OFF + S, c = OFF + 2 * S, d = OFF + 3 * S;
    const float t0 = g[a] + g[c], t1 = g[a] - g[c], t2 = g[b] + g[d], t3 = g[b] - g[d];
    xr[0] = t0 + t2;
    xr[2] = t0 - t2;
    xr[1] = t1;
    xi[1] = -t3;
    xi[0] = 0.0f;
    xi[2] = 0.0f;
  } else {
    float er[N / 4 + 1], ei[N / 4 + 1], orr[N / 4 + 1], oi[N / 4 + 1];
    rdft_f32<N / 2, 2 * S, OFF, L>(g, er, ei);
    rdft_f32<N / 2, 2 * S, OFF + S, L>(g, orr, oi);
    xr[0] = er[0] + orr[0];
    xi[0] = 0.0f;
    xr[N / 2] = er[0] - orr[0];
    xi[N / 2] = 0.0f;
    xr[N / 4] = er[N / 4];
    xi[N / 4] = -orr[N / 4];
    sfor<N / 4 - 1>([&](auto K) {
      constexpr int k = RTQ_CI(K) + 1;
      constexpr float c = (float)cos2pi(k, N), s = (float)sin2pi(k, N);
      xr[k] = __builtin_fmaf(c, orr[k], __builtin_fmaf(s, oi[k], er[k]));
      xi[k] = __builtin_fmaf(c, oi[k], __builtin_fmaf(-s, orr[k], ei[k]));
      xr[N / 2 - k] = __builtin_fmaf(2.0f, er[k], -xr[k]);
      xi[N / 2 - k] = __builtin_fmaf(-2.0f, ei[k], xi[k]);
    });
  }
}

// Packed orthonormal SRFT of length D (one lane), returned divided by
// sqrt(2/D): the quantizer multiplies it back (zs = SrftScale<D>), so the
// interior bins cost nothing extra and only the two real end bins (scale
// 1/sqrt(D) = sqrt(2/D) / sqrt(2)) take a multiply.
template <int D> struct SrftScale { static constexpr float value = (float)csqrt(2.0 / (double)D); };

template <int D>
__device__ __forceinline__ void srft_fwd_unscaled(const uint32_t (&h)[D / 2], float (&z)[D]) {
  constexpr int M = D / 2;
  float xr[M + 1], xi[M + 1];
  rdft<D, 1, 0, D / 2>(h, xr, xi);
  constexpr float r2 = (float)(1.0 / csqrt(2.0));
  z[0] = xr[0] * r2;
  sfor<M - 1>([&](auto K) {
    constexpr int k = RTQ_CI(K) + 1;
    z[2 * k - 1] = xr[k];
    z[2 * k] = xi[k];
  });
  z[D - 1] = xr[M] * r2;
}

// ---------------------------------------------------------------------------
// Real DFT of length D = 2M from one complex DFT of length M.
// ---------------------------------------------------------------------------

// Scale sets for the real-DFT bins: bin 0 is multiplied by S0, bin M by SM,
// bins 1..M-1 by SI.
template <int D>
struct OrthoPacked {  // the packed orthonormal rfft: z[0]=X0, ..., sqrt2 on interior bins
  static constexpr double s0 = 1.0 / csqrt((double)D);
  static constexpr double sm = 1.0 / csqrt((double)D);
  static constexpr double si = csqrt(2.0 / (double)D);
};

// Bins U_k (k = 0..M) of the real fp32 sequence u:
// U_k = sum_n u_n exp(-2 pi i k n / D), scaled per SC.  With
// W = DFT_M(u_{2m} + i u_{2m+1}):
//   U_k = (W_k + conj W_{M-k})/2 - (i/2) exp(-2 pi i k / D) (W_k - conj W_{M-k}).
// (The fp16-input path of the fused kernels is rdft above; this one serves
// inputs already in fp32, such as lambda-weighted vectors.)
template <int D, class SC>
__device__ __forceinline__ void rfft_bins(const float (&u)[D], float (&ur)[D / 2 + 1], float (&ui)[D / 2 + 1]) {
  constexpr int M = D / 2;
  float xr[M], xi[M];
  sfor<M>([&](auto I) {
    xr[RTQ_CI(I)] = u[2 * RTQ_CI(I)];
    xi[RTQ_CI(I)] = u[2 * RTQ_CI(I) + 1];
  });
  float re[M], im[M];
  cfft_f32<M>(xr, xi, re, im);
  constexpr float s0 = (float)SC::s0, sm = (float)SC::sm, si = (float)SC::si;
  ur[0] = s0 * (re[0] + im[0]);
  ui[0] = 0.0f;
  ur[M] = sm * (re[0] - im[0]);
  ui[M] = 0.0f;
  ur[M / 2] = si * re[M / 2];
  ui[M / 2] = -si * im[M / 2];
  sfor<M / 2 - 1>([&](auto K) {
    constexpr int k = RTQ_CI(K) + 1;
    constexpr float hh = (float)(SC::si * 0.5);
    constexpr float a = (float)(SC::si * 0.5 * sin2pi(k, D));  // (si/2) * i * w^k = a + i b
    constexpr float b = (float)(SC::si * 0.5 * cos2pi(k, D));
    const float Ar = re[k] + re[M - k], Ai = im[k] - im[M - k];
    const float Br = re[k] - re[M - k], Bi = im[k] + im[M - k];
    const float Qr = __builtin_fmaf(a, Br, -b * Bi);
    const float Qi = __builtin_fmaf(a, Bi, b * Br);
    ur[k] = __builtin_fmaf(hh, Ar, -Qr);
    ui[k] = __builtin_fmaf(hh, Ai, -Qi);
    ur[M - k] = __builtin_fmaf(hh, Ar, Qr);
    ui[M - k] = -__builtin_fmaf(hh, Ai, Qi);
  });
}

// z = R u for the packed orthonormal SRFT of length D (D <= 128, one lane),
// u in fp32.
template <int D>
__device__ __forceinline__ void srft_fwd(const float (&u)[D], float (&z)[D]) {
  constexpr int M = D / 2;
  float ur[M + 1], ui[M + 1];
  rfft_bins<D, OrthoPacked<D>>(u, ur, ui);
  z[0] = ur[0];
  sfor<M - 1>([&](auto K) {
    constexpr int k = RTQ_CI(K) + 1;
    z[2 * k - 1] = ur[k];
    z[2 * k] = ui[k];
  });
  z[D - 1] = ur[M];
}

// u = KAPPA * R^T z for the packed orthonormal SRFT of length D (the
// orthonormal irfft of the unpacked bins, times KAPPA).  Computed as
// u_{2n} + i u_{2n+1} = conj(DFT_M(V))_n with V built from z.
template <int D, class KAPPA>
__device__ __forceinline__ void srft_inv(const float (&z)[D], float (&u)[D]) {
  constexpr int M = D / 2;
  constexpr double cout = KAPPA::value / (csqrt(2.0) * csqrt((double)D));
  float vr[M], vi[M];
  {
    constexpr float c = (float)(cout * csqrt(2.0));
    vr[0] = c * (z[0] + z[D - 1]);
    vi[0] = c * (z[D - 1] - z[0]);
    constexpr float c2 = (float)(cout * 2.0);
    vr[M / 2] = c2 * z[M - 1];
    vi[M / 2] = c2 * z[M];
  }
  sfor<M / 2 - 1>([&](auto K) {
    constexpr int k = RTQ_CI(K) + 1;
    constexpr float co = (float)cout;
    constexpr float ms = (float)(-cout * sin2pi(k, D));  // cout * i * w^-k = ms + i mc'
    constexpr float mc = (float)(cout * cos2pi(k, D));
    const float Ar = z[2 * k - 1] + z[2 * (M - k) - 1], Ai = z[2 * k] - z[2 * (M - k)];
    const float Br = z[2 * k - 1] - z[2 * (M - k) - 1], Bi = z[2 * k] + z[2 * (M - k)];
    const float Qr = __builtin_fmaf(ms, Br, -mc * Bi);
    const float Qi = __builtin_fmaf(mc, Br, ms * Bi);
    vr[k] = __builtin_fmaf(co, Ar, Qr);
    vi[k] = -__builtin_fmaf(co, Ai, Qi);
    vr[M - k] = __builtin_fmaf(co, Ar, -Qr);
    vi[M - k] = __builtin_fmaf(co, Ai, -Qi);
  });
  float wr[M], wi[M];
  cfft_f32<M>(vr, vi, wr, wi);
  sfor<M>([&](auto N) {
    constexpr int m = RTQ_CI(N);
    u[2 * m] = wr[m];
    u[2 * m + 1] = -wi[m];
  });
}

// The discrete Hartley transform u_n = sum_m g_m (cos + sin)(2 pi m n / D)
// of D real samples, from the real DFTs E and O (length D/2) of the even
// and odd samples.  With G = DFT(g), u_n = Re G_n - Im G_n and u_{D-n} =
// Re G_n + Im G_n; the last even/odd step of the real DFT and this
// combination fold together: with A = Re E_k - Im E_k, B = Re E_k + Im E_k
// and w^k = c - i s,
//   u_k       = A + (c + s) Re O_k + (s - c) Im O_k,
//   u_{D-k}   = B + (c - s) Re O_k + (c + s) Im O_k,
//   u_{D/2-k} = 2 B - u_{D-k},   u_{D/2+k} = 2 A - u_k,
// eight operations per four samples (k = 1 .. D/4 - 1); k = 0 and D/4 take
// the sums and differences of the real end bins.
template <int D>
__device__ __forceinline__ void hartley_f32(const float (&g)[D], float (&u)[D]) {
  constexpr int M = D / 2, Q = D / 4;
  float er[Q + 1], ei[Q + 1], orr[Q + 1], oi[Q + 1];
  rdft_f32<M, 2, 0, D>(g, er, ei);
  rdft_f32<M, 2, 1, D>(g, orr, oi);
  u[0] = er[0] + orr[0];
  u[M] = er[0] - orr[0];
  u[Q] = er[Q] + orr[Q];  // G_{D/4} = E_{D/4} - i O_{D/4}, both real
  u[D - Q] = er[Q] - orr[Q];
  sfor<Q - 1>([&](auto K) {
    constexpr int k = RTQ_CI(K) + 1;
    constexpr double c = cos2pi(k, D), s = sin2pi(k, D);
    constexpr float cps = (float)(c + s), smc = (float)(s - c), cms = (float)(c - s);
    const float A = er[k] - ei[k], B = er[k] + ei[k];
    u[k] = __builtin_fmaf(cps, orr[k], __builtin_fmaf(smc, oi[k], A));
    u[D - k] = __builtin_fmaf(cms, orr[k], __builtin_fmaf(cps, oi[k], B));
    u[M - k] = __builtin_fmaf(2.0f, B, -u[D - k]);
    u[M + k] = __builtin_fmaf(2.0f, A, -u[k]);
  });
}

// Step of hartley_f32 that forms sample n (0 for the end bins).
template <int D>
constexpr int hartley_step(int n) {
  constexpr int M = D / 2, Q = D / 4;
  if (n == 0 || n == M || n == Q || n == D - Q) return 0;
  if (n < Q) return n;           // u_k
  if (n < M) return M - n;       // u_{M-k}
  if (n < D - Q) return n - M;   // u_{M+k}
  return D - n;                  // u_{D-k}
}

// hartley_f32 with the samples rounded to fp16 pairs, hw[m] = (u_{2m},
// u_{2m+1}), each pair as soon as the step that completes it has run, so
// that few unpacked samples are live at once.  Weighted: sample n is first
// multiplied by w[n] (w 8-byte aligned).
template <int D, bool Weighted = false>
__device__ __forceinline__ void hartley_f32_packed(const float (&g)[D], uint32_t (&hw)[D / 2],
                                                   const float* w = nullptr) {
  constexpr int M = D / 2, Q = D / 4;
  float er[Q + 1], ei[Q + 1], orr[Q + 1], oi[Q + 1];
  rdft_f32<M, 2, 0, D>(g, er, ei);
  rdft_f32<M, 2, 1, D>(g, orr, oi);
  float u[D];
  auto pack_done = [&](auto K) {
    constexpr int k = RTQ_CI(K);
    sfor<M>([&](auto W) {
      constexpr int m = RTQ_CI(W);
      constexpr int t0 = hartley_step<D>(2 * m), t1 = hartley_step<D>(2 * m + 1);
      if constexpr ((t0 > t1 ? t0 : t1) == k) {
        if constexpr (Weighted) {
          const float2 q = *reinterpret_cast<const float2*>(w + 2 * m);
          hw[m] = pack_f16x2(u[2 * m] * q.x, u[2 * m + 1] * q.y);
        } else {
          hw[m] = pack_f16x2(u[2 * m], u[2 * m + 1]);
        }
      }
    });
  };
  u[0] = er[0] + orr[0];
  u[M] = er[0] - orr[0];
  u[Q] = er[Q] + orr[Q];
  u[D - Q] = er[Q] - orr[Q];
  pack_done(ic<0>{});
  sfor<Q - 1>([&](auto K) {
    constexpr int k = RTQ_CI(K) + 1;
    constexpr double c = cos2pi(k, D), s = sin2pi(k, D);
    constexpr float cps = (float)(c + s), smc = (float)(s - c), cms = (float)(c - s);
    const float A = er[k] - ei[k], B = er[k] + ei[k];
    u[k] = __builtin_fmaf(cps, orr[k], __builtin_fmaf(smc, oi[k], A));
    u[D - k] = __builtin_fmaf(cms, orr[k], __builtin_fmaf(cps, oi[k], B));
    u[M - k] = __builtin_fmaf(2.0f, B, -u[D - k]);
    u[M + k] = __builtin_fmaf(2.0f, A, -u[k]);
    pack_done(ic<k>{});
  });
}

// u = sqrt2 * R^T z for the packed orthonormal SRFT of length D (the
// srft_inv<D, Sqrt2> result), given yk = z / sqrt(D) (the caller folds that
// factor into its dequantization), through the Hartley transform: with
// g_0 = sqrt2 yk_0, g_{D/2} = sqrt2 yk_{D-1}, g_m = yk_{2m-1} - yk_{2m} and
// g_{D-m} = yk_{2m-1} + yk_{2m} (m = 1 .. D/2-1), the inverse is
// sum_m g_m (cos + sin)(2 pi m n / D) (hartley_f32).  This costs about the
// forward recursion plus one operation per coordinate, against the complex
// FFT of length D/2 plus its pre-processing for srft_inv.
template <int D>
__device__ __forceinline__ void srft_inv_hartley(const float (&yk)[D], float (&u)[D]) {
  constexpr int M = D / 2;
  constexpr float sq2 = 1.41421356237309504880f;
  float g[D];
  g[0] = sq2 * yk[0];
  g[M] = sq2 * yk[D - 1];
  sfor<M - 1>([&](auto K) {
    constexpr int m = RTQ_CI(K) + 1;
    g[m] = yk[2 * m - 1] - yk[2 * m];
    g[D - m] = yk[2 * m - 1] + yk[2 * m];
  });
  hartley_f32<D>(g, u);
}

// srft_inv_hartley with the samples rounded to fp16 pairs (hartley_f32_packed).
template <int D>
__device__ __forceinline__ void srft_inv_hartley_packed(const float (&yk)[D], uint32_t (&hw)[D / 2]) {
  constexpr int M = D / 2;
  constexpr float sq2 = 1.41421356237309504880f;
  float g[D];
  g[0] = sq2 * yk[0];
  g[M] = sq2 * yk[D - 1];
  sfor<M - 1>([&](auto K) {
    constexpr int m = RTQ_CI(K) + 1;
    g[m] = yk[2 * m - 1] - yk[2 * m];
    g[D - m] = yk[2 * m - 1] + yk[2 * m];
  });
  hartley_f32_packed<D>(g, hw);
}

// The factor on z for which srft_inv_hartley<D> returns u = R^T z.
template <int D> struct HartleyIn { static constexpr float value = (float)(1.0 / csqrt(2.0 * (double)D)); };

struct One { static constexpr double value = 1.0; };

// 1/sqrt(D) as a compile-time fp32 constant (the SRHT normalization).
template <int D> struct InvSqrt { static constexpr float value = (float)(1.0 / csqrt((double)D)); };
struct Sqrt2 { static constexpr double value = 1.4142135623730950488016887242097; };

// ---------------------------------------------------------------------------
// Walsh-Hadamard transform (Sylvester order), unnormalized.
// ---------------------------------------------------------------------------

template <int N>
__device__ __forceinline__ void fwht_stages_from2(float (&v)[N]) {
  constexpr int LOG = ilog2(N);
  sfor<LOG - 1>([&](auto S) {
    constexpr int h = 2 << RTQ_CI(S);
    sfor<N / (2 * h)>([&](auto B) {
      sfor<h>([&](auto J) {
        constexpr int p = RTQ_CI(B) * 2 * h + RTQ_CI(J);
        const float a = v[p], b = v[p + h];
        v[p] = a + b;
        v[p + h] = a - b;
      });
    });
  });
}

// y = H_N u, u_{2m} = lo(h[m]), u_{2m+1} = hi(h[m]).
template <int N>
__device__ __forceinline__ void fwht_from_f16(const uint32_t (&h)[N / 2], float (&y)[N]) {
  sfor<N / 2>([&](auto M) {
    constexpr int m = RTQ_CI(M);
    y[2 * m] = mix_add<0, 1>(h[m], h[m]);
    y[2 * m + 1] = mix_sub<0, 1>(h[m], h[m]);
  });
  fwht_stages_from2<N>(y);
}

// In place, fp32.
template <int N>
__device__ __forceinline__ void fwht_f32(float (&v)[N]) {
  sfor<N / 2>([&](auto M) {
    constexpr int m = RTQ_CI(M);
    const float a = v[2 * m], b = v[2 * m + 1];
    v[2 * m] = a + b;
    v[2 * m + 1] = a - b;
  });
  fwht_stages_from2<N>(v);
}

// ---------------------------------------------------------------------------
// Symmetric absmax int4 quantizer and nibble packing.
// ---------------------------------------------------------------------------

// Eight int4 codes of (z * inv) packed into one word: nibble i = code i, two's
// complement, q_i = clamp(rne(z_i * inv), -8, 7).  The rounding is
// fma(z_i, inv, 1.5 * 2^23): the fp32 result lies in [2^23, 2^24), where the
// spacing is 1, so the fma's single rounding is round-half-even of z_i * inv,
// v_med3 clamps it, and the low 4 bits of the pattern are q_i mod 16.
// (Forms that round z_i * inv + 248 with v_cvt_pk_u8_f32, or into an fp16
// half with v_fma_mix{lo,hi}_f16, take fewer instructions but are not
// faster: the first rounds twice, the second issues at half rate.)
__device__ __forceinline__ uint32_t pack8_int4(const float* z, float inv) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  uint32_t b[8];
  sfor<8>([&](auto I) {
    const float t = __builtin_fmaf(z[RTQ_CI(I)], inv, kMagic);
    b[RTQ_CI(I)] = __float_as_uint(__builtin_amdgcn_fmed3f(t, kMagic - 8.0f, kMagic + 7.0f));
  });
  // low bytes of the even codes -> e, of the odd codes -> o
  const uint32_t e = __builtin_amdgcn_perm(b[2], b[0], 0x0c0c0400u) | __builtin_amdgcn_perm(b[6], b[4], 0x04000c0cu);
  const uint32_t o = __builtin_amdgcn_perm(b[3], b[1], 0x0c0c0400u) | __builtin_amdgcn_perm(b[7], b[5], 0x04000c0cu);
  return (e & 0x0f0f0f0fu) | ((o << 4) & 0xf0f0f0f0u);
}

// Words Q .. Q + 3 of w count as computed here (an empty asm that claims to
// change them): later code cannot move their computation past this point.
template <int Q, int N>
__device__ __forceinline__ void pin_words(uint32_t (&w)[N]) {
  asm volatile("" : "+v"(w[Q]), "+v"(w[Q + 1]), "+v"(w[Q + 2]), "+v"(w[Q + 3]));
}

// One group (GI) of quantize_pack below.
template <int GI, int D, int G>
__device__ __forceinline__ void quantize_pack_group(const float (&z)[D], float zs, uint32_t (&cw)[D / 8],
                                                    uint32_t (&sb)[D / G]) {
  constexpr int g0 = GI * G;
  float a = 0.0f;
  sfor<G>([&](auto I) { a = fmaxf(a, fabsf(z[g0 + RTQ_CI(I)])); });
  a *= zs;
  uint32_t bits = __half_as_ushort(__float2half_rn(a * 0.125f));
  bits = bits < 0x7bffu ? bits : 0x7bffu;  // saturate (inf -> 65504)
  sb[GI] = bits;
  const float s = __half2float(__ushort_as_half((unsigned short)bits));
  const float inv = bits == 0u ? 0.0f : __builtin_amdgcn_rcpf(s) * zs;
  sfor<G / 8>([&](auto W) {
    constexpr int base = g0 + RTQ_CI(W) * 8;
    cw[base / 8] = pack8_int4(&z[base], inv);
  });
}

// Per group of G consecutive values of (zs * z): s = fp16_rne(absmax / 8)
// saturated at 65504; q = clamp(rne(zs * z / s), -8, 7), q = 0 when s == 0.
// Codes: cw[w] holds values 8w .. 8w+7, value 2i in the low nibble of byte i
// (pack8_int4).  quantize_pack_group does one group (GI) of this.
template <int D, int G>
__device__ __forceinline__ void quantize_pack(const float (&z)[D], float zs, uint32_t (&cw)[D / 8],
                                              uint32_t (&sb)[D / G]) {
  sfor<D / G>([&](auto GI) { quantize_pack_group<RTQ_CI(GI), D, G>(z, zs, cw, sb); });
}

// fp16 half SEL of a, times b, plus c, in fp32 with a single rounding.
template <int SEL>
__device__ __forceinline__ float mix_fma(uint32_t a, float b, float c) {
  float r;
  if constexpr (SEL == 0)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// z = s' * q for every value, s' = zs * s (inverse of quantize_pack's codes).
// Two codes at a time become an fp16 pair, biased to q + 8 by flipping the
// nibble's top bit and placed under a fixed fp16 exponent:
//   * nibbles j and j + 4 of a code word (values 8w + j, 8w + j + 4) with
//     j = 0 (and j = 2 after one 8-bit shift) sit in mantissa bits 0..3 of
//     the low and high halves under the exponent of 1024 (0x6400): each half
//     reads 1024 + 8 + q, and one v_fma_mix gives (1032 + q) s' - 1032 s';
//   * nibbles j = 1 (and 3) sit in mantissa bits 4..7 under the exponent of
//     16384 (0x7400), where the mantissa unit is 16: each half reads
//     16384 + 256 (q + 8), and (72 + q) (s' / 256) * 256 - 72 s' = s' q.
// One shift, four mask-and-bias operations and eight v_fma_mix per word.
// For a power-of-two zs every product and sum is exact in fp32.
template <int D, int G>
__device__ __forceinline__ void dequant_unpack(const uint32_t (&cw)[D / 8], const uint32_t (&sb)[D / G],
                                               float zs, float (&z)[D]) {
  sfor<D / G>([&](auto GI) {
    constexpr int g0 = RTQ_CI(GI) * G;
    const float s = __half2float(__ushort_as_half((unsigned short)sb[RTQ_CI(GI)])) * zs;
    const float c = -1032.0f * s;
    const float s16 = s * (1.0f / 256.0f), c16 = -72.0f * s;
    sfor<G / 8>([&](auto W) {
      constexpr int base = g0 + RTQ_CI(W) * 8;
      const uint32_t x = cw[base / 8], y = x >> 8;
      const uint32_t p0 = (x & 0x000f000fu) ^ 0x64086408u;  // nibbles 0 and 4
      const uint32_t p1 = (x & 0x00f000f0u) ^ 0x74807480u;  // nibbles 1 and 5
      const uint32_t p2 = (y & 0x000f000fu) ^ 0x64086408u;  // nibbles 2 and 6
      const uint32_t p3 = (y & 0x00f000f0u) ^ 0x74807480u;  // nibbles 3 and 7
      z[base + 0] = mix_fma<0>(p0, s, c);
      z[base + 4] = mix_fma<1>(p0, s, c);
      z[base + 1] = mix_fma<0>(p1, s16, c16);
      z[base + 5] = mix_fma<1>(p1, s16, c16);
      z[base + 2] = mix_fma<0>(p2, s, c);
      z[base + 6] = mix_fma<1>(p2, s, c);
      z[base + 3] = mix_fma<0>(p3, s16, c16);
      z[base + 7] = mix_fma<1>(p3, s16, c16);
    });
  });
}

// ---------------------------------------------------------------------------
// Other code widths: B-bit codes in a little-endian bit stream.
// ---------------------------------------------------------------------------

// Per group of G values of (zs * z): s = fp16_rne(absmax / 2^(B-1)) saturated
// at 65504, q = clamp(rne(zs * z / s), -2^(B-1), 2^(B-1) - 1) (q = 0 when
// s == 0).  Code i fills stream bits [i*B, (i+1)*B); word k of cw holds stream
// bits 32k .. 32k+31.  The rounding is quantize_pack's: the fma lands in
// [2^23, 2^24), where the low bits of the fp32 pattern are q mod 2^B.
template <int D, int G, int B>
__device__ __forceinline__ void quantize_pack_bits(const float (&z)[D], float zs, uint32_t (&cw)[D * B / 32],
                                                   uint32_t (&sb)[D / G]) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  constexpr float kLo = -(float)(1 << (B - 1)), kHi = (float)((1 << (B - 1)) - 1);
  constexpr float kInvRange = 1.0f / (float)(1 << (B - 1));
  constexpr uint32_t kMask = (1u << B) - 1u;
  sfor<D * B / 32>([&](auto K) { cw[RTQ_CI(K)] = 0u; });
  sfor<D / G>([&](auto GI) {
    constexpr int g0 = RTQ_CI(GI) * G;
    float a = 0.0f;
    sfor<G>([&](auto I) { a = fmaxf(a, fabsf(z[g0 + RTQ_CI(I)])); });
    a *= zs;
    uint32_t bits = __half_as_ushort(__float2half_rn(a * kInvRange));
    bits = bits < 0x7bffu ? bits : 0x7bffu;
    sb[RTQ_CI(GI)] = bits;
    const float s = __half2float(__ushort_as_half((unsigned short)bits));
    const float inv = bits == 0u ? 0.0f : __builtin_amdgcn_rcpf(s) * zs;
    sfor<G>([&](auto I) {
      constexpr int i = g0 + RTQ_CI(I);
      constexpr int pos = i * B, w = pos / 32, sh = pos % 32;
      const float t = __builtin_amdgcn_fmed3f(__builtin_fmaf(z[i], inv, kMagic), kMagic + kLo, kMagic + kHi);
      const uint32_t f = __float_as_uint(t) & kMask;
      cw[w] |= f << sh;
      if constexpr (sh + B > 32) cw[w + 1] |= f >> (32 - sh);
    });
  });
}

// z = s' * q for every value, s' = zs * s (inverse of quantize_pack_bits).
template <int D, int G, int B>
__device__ __forceinline__ void dequant_unpack_bits(const uint32_t (&cw)[D * B / 32], const uint32_t (&sb)[D / G],
                                                    float zs, float (&z)[D]) {
  sfor<D / G>([&](auto GI) {
    constexpr int g0 = RTQ_CI(GI) * G;
    const float s = __half2float(__ushort_as_half((unsigned short)sb[RTQ_CI(GI)])) * zs;
    sfor<G>([&](auto I) {
      constexpr int i = g0 + RTQ_CI(I);
      constexpr int pos = i * B, w = pos / 32, sh = pos % 32;
      uint32_t v = cw[w] >> sh;
      if constexpr (sh + B > 32) v |= cw[w + 1] << (32 - sh);
      const int q = (int)(v << (32 - B)) >> (32 - B);  // sign-extend the B-bit field
      z[i] = (float)q * s;
    });
  });
}

}  // namespace rtq
