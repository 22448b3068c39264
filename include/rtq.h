/*
 * rtq.h -- C ABI of the rotate-then-quantize int4 KV-cache library for
 * AMD MI355X (gfx950).
 *
 * The method: each K/V vector is rotated and stored as int4 codes with fp16
 * scales; reading the cache reverses both steps ("Quantization Speed Is
 * Often a Kernel Problem", section "First, the 17%").  The fused
 * form runs rotate + quantize as one kernel and dequantize + inverse-rotate
 * as another (same page, section "Fusing four steps into two kernels is not
 * enough").  Each entry point below is one such fused kernel launch.
 *
 * Common conventions
 * ------------------
 *  Layout (all row-major, contiguous, rows independent):
 *    x, y     : [n][d]      IEEE fp16 K/V vectors (2*d bytes per row)
 *    codes    : [n][d/2]    uint8; byte m of a row holds packed coordinate
 *                            2m in its low nibble and 2m+1 in its high nibble,
 *                            each a two's-complement int4 in [-8, 7] ("Chapter
 *                            25 - Quantization: The Hardware View", section
 *                            "Kernels: Marlin, CUTLASS, and Why INT4 Packing
 *                            Needs Special Code")
 *    scales   : [n][d/group] IEEE fp16; scale j of a row covers packed
 *                            coordinates [j*group, (j+1)*group)
 *  Shapes: d in {64, 128, 256}; group in {32, 64, 128, 256} with group <= d.
 *    group == d is the per-token recipe (one scale per vector).  Rows per
 *    call: 0 <= n <= 0xFFFFFF00 (row indices are 32-bit on the device); a
 *    larger n returns RTQ_ERR_INVALID_ARG.
 *  Signs: row r uses the sign vector of seed'(r) =
 *    seed + ((r / rows_per_seed) % seed_period)   (mod 2^64),
 *    where rows_per_seed == 0 means one seed for every row and
 *    seed_period == 0 means no modulo.  Sign i of seed S is -1 iff bit 63 of
 *    the (i+1)-th output of SplitMix64 (Steele, Lea & Flood 2014) started at
 *    state S is set.  The method page fixes only that the signs are a
 *    constant pseudo-random +-1 vector ("Quantization Speed Is Often a
 *    Kernel Problem", "First, the 17%").
 *  Pointers: device pointers (or any pointers the GPU can address), each
 *    16-byte aligned.  The caller owns every buffer; the library allocates
 *    no device memory and is thread-safe.  The only state kept between calls
 *    is a per-host-thread copy of the last sign table the host evaluated (a
 *    pure function of seed, d and the seed count), reused by later calls
 *    with the same seed.  Outputs must
 *    not overlap inputs.
 *  Stream: the work is enqueued asynchronously on `stream` (NULL = the
 *    default stream) and the call returns; results are visible after the
 *    stream is synchronized.
 *  Errors: all arguments are validated on the host before any HIP call; on
 *    error nothing is launched and nothing is written.  n == 0 returns RTQ_OK
 *    without touching any pointer.  A failed launch returns RTQ_ERR_HIP (the
 *    HIP error stays readable through hipGetLastError()).  Nothing throws.
 */
#ifndef RTQ_H
#define RTQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's own stream handle. */
typedef struct ihipStream_t* hipStream_t;

typedef enum rtq_status {
  RTQ_OK = 0,
  RTQ_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, overlap */
  RTQ_ERR_UNSUPPORTED = 2, /* (d, group) outside the supported set            */
  RTQ_ERR_HIP = 3          /* the HIP runtime reported an error at launch      */
} rtq_status;

/*
 * srft_quant_fwd -- fused forward step with the SRFT rotation.
 *
 * For each row r: u = D(seed'(r)) * x[r] (sign flip, which the SRFT applies
 * before its FFT: "Quantization Speed Is Often a Kernel Problem", "First, the
 * 17%"); z = R u, R = orthonormal real DFT (rfft) packed to d reals as
 *   z[0] = X_0, z[2k-1] = sqrt2*Re X_k, z[2k] = sqrt2*Im X_k (k=1..d/2-1),
 *   z[d-1] = X_{d/2},  X_k = d^-1/2 * sum_n u_n exp(-2 pi i k n / d);
 * then per group j: s_j = fp16_rne(max_i |z_i| / 8) (saturated at 65504),
 * q_i = clamp(round_half_even(z_i / s_j), -8, 7) (q = 0 when s_j == 0)
 * ("Day 9 - Quantization: Shrink the Bytes Themselves", sections "What
 * Quantization Is, Mathematically" and "How Many Numbers Should One Scale
 * Cover"); codes and scales are written in the layout above.
 *
 *   x_f16       in : [n][d] fp16
 *   codes_u8    out: [n][d/2] uint8
 *   scales_f16  out: [n][d/group] fp16
 * Rotated values are kept in fp32 inside the kernel and never stored.
 */
rtq_status srft_quant_fwd(const void* x_f16, void* codes_u8, void* scales_f16,
                          int64_t n, int32_t d, int32_t group, uint64_t seed,
                          int64_t rows_per_seed, int32_t seed_period,
                          hipStream_t stream);

/*
 * srft_dequant_inv -- fused inverse step with the SRFT rotation.
 *
 * For each row r: z_hat_i = s_j * q_i (sign-extended nibbles); u = R^T z_hat
 * (the orthonormal irfft of the unpacked bins); y[r] = fp16_rne(D(seed'(r)) * u)
 * ("Quantization Speed Is Often a Kernel Problem", "First, the 17%": the
 * inverse runs when the cache is read).
 *
 *   codes_u8    in : [n][d/2] uint8
 *   scales_f16  in : [n][d/group] fp16
 *   y_f16       out: [n][d] fp16
 */
rtq_status srft_dequant_inv(const void* codes_u8, const void* scales_f16, void* y_f16,
                            int64_t n, int32_t d, int32_t group, uint64_t seed,
                            int64_t rows_per_seed, int32_t seed_period,
                            hipStream_t stream);

/*
 * srht_quant_fwd / srht_dequant_inv -- the same two steps with the SRHT
 * control rotation ("Quantization Speed Is Often a Kernel Problem", "First,
 * the 17%": a sign-randomized Hadamard transform used as the control):
 * R = d^-1/2 * H_d, H[i][k] = (-1)^popcount(i & k) (Sylvester order).
 * R is symmetric, so the inverse applies the same transform.  Arguments,
 * layouts and errors are those of the SRFT entry points.
 */
rtq_status srht_quant_fwd(const void* x_f16, void* codes_u8, void* scales_f16,
                          int64_t n, int32_t d, int32_t group, uint64_t seed,
                          int64_t rows_per_seed, int32_t seed_period,
                          hipStream_t stream);

rtq_status srht_dequant_inv(const void* codes_u8, const void* scales_f16, void* y_f16,
                            int64_t n, int32_t d, int32_t group, uint64_t seed,
                            int64_t rows_per_seed, int32_t seed_period,
                            hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* rtq_status_string(rtq_status status);

#ifdef __cplusplus
}
#endif

#endif /* RTQ_H */
