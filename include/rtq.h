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

#include <stddef.h>
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

/*
 * srft_quant_fwd_ext / srht_quant_fwd_ext / srft_dequant_inv_ext /
 * srht_dequant_inv_ext -- the forward and inverse steps with other code widths
 * and an optional per-channel lambda.  The method page's fused recipe adds one
 * scale per channel to the per-group absmax, and its quality study runs 3-,
 * 4-, 6- and 8-bit codes ("Quantization Speed Is Often a Kernel Problem",
 * "First, the 17%"); the formulas below are this library's reading.
 *
 *   bits        : 3, 4, 6 or 8.  Group scale s_j = fp16_rne(absmax / 2^(bits-1))
 *                 (saturated at 65504), q = clamp(round_half_even(z / s_j),
 *                 -2^(bits-1), 2^(bits-1) - 1).
 *   codes_u8    : [n][d*bits/8] bytes.  The codes of a row form one bit
 *                 stream: code i fills stream bits [i*bits, (i+1)*bits), least
 *                 significant bit first, stream bit k being bit k%8 of byte
 *                 k/8; each field is two's complement.  bits = 4 gives the
 *                 nibble layout of the common conventions (and the same codes
 *                 as srft_quant_fwd when lambda_f16 is NULL).
 *   lambda_f16  : NULL, or d fp16 values (16-byte aligned), one per channel.
 *                 The forward rotates D * (lambda .* x) (the products are exact
 *                 in fp32); the inverse returns fp16(D * (R^T z_hat) ./ lambda).
 *                 Entries must be finite and nonzero.
 *   x_f16, y_f16, scales_f16, n, d, group, seed rule, stream: as for
 *                 srft_quant_fwd / srft_dequant_inv.
 * Supported: every (d, group) of the common conventions; other bits return
 * RTQ_ERR_UNSUPPORTED.  Errors otherwise as in the common conventions.
 */
rtq_status srft_quant_fwd_ext(const void* x_f16, void* codes_u8, void* scales_f16, int64_t n, int32_t d,
                              int32_t group, int32_t bits, const void* lambda_f16, uint64_t seed,
                              int64_t rows_per_seed, int32_t seed_period, hipStream_t stream);

rtq_status srht_quant_fwd_ext(const void* x_f16, void* codes_u8, void* scales_f16, int64_t n, int32_t d,
                              int32_t group, int32_t bits, const void* lambda_f16, uint64_t seed,
                              int64_t rows_per_seed, int32_t seed_period, hipStream_t stream);

rtq_status srft_dequant_inv_ext(const void* codes_u8, const void* scales_f16, void* y_f16, int64_t n, int32_t d,
                                int32_t group, int32_t bits, const void* lambda_f16, uint64_t seed,
                                int64_t rows_per_seed, int32_t seed_period, hipStream_t stream);

rtq_status srht_dequant_inv_ext(const void* codes_u8, const void* scales_f16, void* y_f16, int64_t n, int32_t d,
                                int32_t group, int32_t bits, const void* lambda_f16, uint64_t seed,
                                int64_t rows_per_seed, int32_t seed_period, hipStream_t stream);

/*
 * srft_quant_append / srht_quant_append -- the forward step written in place
 * into a cache whose rows are addressed by strides: the new tokens of every
 * layer, K/V and stream go straight to their cache rows.  With
 * srft_dequant_rows it maintains a dequantized fp16 copy of the cache prefix
 * between decode steps while the newest tokens stay in fp16 and are quantized
 * when that window fills ("Quantization Speed Is Often a Kernel Problem",
 * "First, the 17%").
 *
 *   x_f16       in : [layers][2][streams][n_tokens][d] fp16, contiguous
 *                    (index 0 / 1 of the second axis = keys / values)
 *   codes_u8    out: cache codes, rows of d/2 bytes
 *   scales_f16  out: cache scales, rows of d/group fp16
 * x[l][kv][s][j] goes to cache row
 *   l*stride_layer + kv*stride_kv + s*stride_stream + (t0 + j)*stride_token
 * and is rotated, quantized and packed exactly as srft_quant_fwd would do for
 * that row (its seed is the seed rule applied to that cache row).  Other rows
 * are not touched.  The strides must map distinct (layer, kv, stream, token)
 * to distinct rows.
 *
 * Supported: every (d, group) of the common conventions, else
 * RTQ_ERR_UNSUPPORTED.  layers, streams, t0, n_tokens, strides >= 0,
 * layers*2*streams*n_tokens <= 0xFFFFFF00, else RTQ_ERR_INVALID_ARG; an empty
 * block returns RTQ_OK.  The caller guarantees that the cache holds every row
 * the strides reach.  Pointers, streams and errors as in the common
 * conventions.
 */
rtq_status srft_quant_append(const void* x_f16, void* codes_u8, void* scales_f16, int32_t layers, int32_t streams,
                             int32_t t0, int32_t n_tokens, int32_t d, int32_t group, int64_t stride_layer,
                             int64_t stride_kv, int64_t stride_stream, int64_t stride_token, uint64_t seed,
                             int64_t rows_per_seed, int32_t seed_period, hipStream_t stream);

rtq_status srht_quant_append(const void* x_f16, void* codes_u8, void* scales_f16, int32_t layers, int32_t streams,
                             int32_t t0, int32_t n_tokens, int32_t d, int32_t group, int64_t stride_layer,
                             int64_t stride_kv, int64_t stride_stream, int64_t stride_token, uint64_t seed,
                             int64_t rows_per_seed, int32_t seed_period, hipStream_t stream);

/*
 * srft_dequant_rows / srht_dequant_rows -- the inverse step on the cache rows
 * of tokens t0 .. t0+n_tokens-1 of every (layer, K/V, stream), addressed as in
 * srft_quant_append, written to the same rows of y_f16 (an fp16 copy of the
 * cache with rows of d fp16): y[row] is what srft_dequant_inv gives for that
 * row.  Other rows of y are not touched.  Arguments, support and errors as
 * for srft_quant_append; y must not overlap the cache.
 */
rtq_status srft_dequant_rows(const void* codes_u8, const void* scales_f16, void* y_f16, int32_t layers,
                             int32_t streams, int32_t t0, int32_t n_tokens, int32_t d, int32_t group,
                             int64_t stride_layer, int64_t stride_kv, int64_t stride_stream, int64_t stride_token,
                             uint64_t seed, int64_t rows_per_seed, int32_t seed_period, hipStream_t stream);

rtq_status srht_dequant_rows(const void* codes_u8, const void* scales_f16, void* y_f16, int32_t layers,
                             int32_t streams, int32_t t0, int32_t n_tokens, int32_t d, int32_t group,
                             int64_t stride_layer, int64_t stride_kv, int64_t stride_stream, int64_t stride_token,
                             uint64_t seed, int64_t rows_per_seed, int32_t seed_period, hipStream_t stream);

/*
 * srft_attn_decode / srht_attn_decode -- one decode step of softmax attention
 * that reads the int4 cache written by srft_quant_fwd / srht_quant_fwd
 * directly: the cache is dequantized and rotated back when attention reads
 * it ("Quantization Speed Is Often a Kernel Problem", "First, the 17%"), here
 * inside the attention kernel, so no fp16 K/V is written to memory.
 *
 * For every layer l < layers, stream s < streams (a batch entry times a K/V
 * head) and query g < q_per_kv, with keys k_t and values v_t the dequantized,
 * inverse-rotated, sign-flipped rows (what *_dequant_inv returns before its
 * fp16 rounding) of tokens t < tokens:
 *   out[l][s][g] = fp16( sum_t w_t v_t ),
 *   w_t = exp(c_t - max c) / sum_t' exp(c_t' - max c),
 *   c_t = softmax_scale * (q[l][s][g] . k_t).
 * The kernel uses R's orthogonality: it rotates each query with the keys'
 * sign vector (q . k_t = (R D q) . z_t) and rotates the weighted sum of the
 * rotated values back once per query.
 *
 *   q_f16      in : [layers][streams][q_per_kv][d] fp16
 *   codes_u8   in : the cache codes, rows of d/2 bytes (layout as above)
 *   scales_f16 in : the cache scales, rows of d/group fp16
 *   out_f16    out: [layers][streams][q_per_kv][d] fp16
 *   Row of (layer l, kv, stream s, token t), kv = 0 for keys and 1 for values:
 *     l*stride_layer + kv*stride_kv + s*stride_stream + t*stride_token
 *   (a layer-major cache [layer][K,V][stream][token] of capacity C has
 *   strides (2*streams*C, streams*C, C, 1); a time-major one
 *   [token][layer][K,V][stream] has (2*streams, streams, 1, 2*layers*streams)).
 *   seed, rows_per_seed, seed_period: the rule the cache was written with.
 *   Every key row of one (layer, stream) must have the same seed, and every
 *   value row likewise (true for one seed per layer, or per layer and K/V);
 *   otherwise RTQ_ERR_INVALID_ARG.
 *
 * Supported: (d, group) in {(64,32), (64,64), (128,32), (128,64), (128,128),
 * (256,32), (256,64), (256,128), (256,256)} and 1 <= q_per_kv <= 8, else
 * RTQ_ERR_UNSUPPORTED.  tokens >= 1, strides >= 0,
 * layers * streams < 2^31, softmax_scale finite, else RTQ_ERR_INVALID_ARG; layers == 0
 * or streams == 0 returns RTQ_OK and touches nothing.  The caller guarantees
 * that the cache holds every row the strides reach; out must not overlap the
 * inputs.  Pointers, streams and error behaviour as in the common conventions.
 * Numerics: scores keep about 22 bits (fp16 hi/lo query, exact int4 keys,
 * fp32 scaling); values and softmax weights enter the weighted sum as fp16.
 *
 * Token splits (optional): with fewer (layer, stream) pairs than the GPU has
 * room for, the call can spread each stream's tokens over several
 * workgroups, which merge their softmax partials (running max, denominator,
 * unnormalized sum; the usual online-softmax merge) through a workspace:
 *   workspace       inout: caller-owned device memory, 16-byte aligned, of
 *                   workspace_bytes bytes; or NULL with workspace_bytes == 0
 *                   (then every stream runs in one workgroup).  It must be
 *                   zero-filled before its first use; every call that
 *                   completes leaves it ready for the next one.  Calls that
 *                   may run at the same time (other streams) need workspaces
 *                   of their own.  It must not overlap the other buffers.
 *   rtq_attn_workspace_bytes(layers, streams, tokens, q_per_kv, d) gives the
 *   size that allows every split the call would make (0: it would not split;
 *   0 also for invalid sizes).  A smaller workspace gives fewer splits.  The
 *   result does not depend on the split count beyond fp32 rounding.
 * workspace == NULL with workspace_bytes != 0 (or the reverse), or a
 * misaligned workspace: RTQ_ERR_INVALID_ARG.
 */
rtq_status srft_attn_decode(const void* q_f16, const void* codes_u8, const void* scales_f16, void* out_f16,
                            int32_t layers, int32_t streams, int32_t tokens, int32_t q_per_kv, int32_t d,
                            int32_t group, int64_t stride_layer, int64_t stride_kv, int64_t stride_stream,
                            int64_t stride_token, uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                            float softmax_scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

rtq_status srht_attn_decode(const void* q_f16, const void* codes_u8, const void* scales_f16, void* out_f16,
                            int32_t layers, int32_t streams, int32_t tokens, int32_t q_per_kv, int32_t d,
                            int32_t group, int64_t stride_layer, int64_t stride_kv, int64_t stride_stream,
                            int64_t stride_token, uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                            float softmax_scale, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * srft_attn_decode_window / srht_attn_decode_window -- the same decode step
 * over a cache whose newest tokens are still fp16: the method page's decode
 * cache keeps the newest tokens unquantized in a small window and quantizes
 * them only when it fills ("Quantization Speed Is Often a Kernel Problem",
 * "First, the 17%").  One softmax runs over the `tokens` int4 tokens of each
 * stream (as in srft_attn_decode) and its first `window_tokens` window
 * tokens, which come after them:
 *   out[l][s][g] = fp16( sum_t w_t v_t + sum_j w'_j wv_j ),  with the weights
 *   w, w' of one softmax over c_t = softmax_scale * (q . k_t) and
 *   c'_j = softmax_scale * (q . wk_j).
 *
 *   window_f16      in : [layers][2][streams][window_capacity][d] fp16, the
 *                        window keys (index 1 = 0) and values (1), in the
 *                        original domain (neither rotated nor sign-flipped);
 *                        16-byte aligned.  Slots past window_tokens are not read.
 *   window_capacity    : token slots per (layer, K/V, stream) of the window.
 *   window_tokens      : window tokens that count, 0 .. window_capacity.
 *   tokens             : may be 0 when window_tokens >= 1 (no int4 token yet).
 * Other arguments, workspace, supported shapes and errors as for
 * srft_attn_decode.  window_tokens > 64: RTQ_ERR_UNSUPPORTED; window_tokens >
 * window_capacity, a NULL window with window_tokens > 0, a misaligned window,
 * or out overlapping the window: RTQ_ERR_INVALID_ARG.  window_tokens == 0 is
 * srft_attn_decode.
 */
rtq_status srft_attn_decode_window(const void* q_f16, const void* codes_u8, const void* scales_f16,
                                   void* out_f16, int32_t layers, int32_t streams, int32_t tokens,
                                   int32_t q_per_kv, int32_t d, int32_t group, int64_t stride_layer,
                                   int64_t stride_kv, int64_t stride_stream, int64_t stride_token,
                                   uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                   float softmax_scale, const void* window_f16, int32_t window_capacity,
                                   int32_t window_tokens, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

rtq_status srht_attn_decode_window(const void* q_f16, const void* codes_u8, const void* scales_f16,
                                   void* out_f16, int32_t layers, int32_t streams, int32_t tokens,
                                   int32_t q_per_kv, int32_t d, int32_t group, int64_t stride_layer,
                                   int64_t stride_kv, int64_t stride_stream, int64_t stride_token,
                                   uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                   float softmax_scale, const void* window_f16, int32_t window_capacity,
                                   int32_t window_tokens, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream);

size_t rtq_attn_workspace_bytes(int32_t layers, int32_t streams, int32_t tokens, int32_t q_per_kv, int32_t d);

/*
 * srft_attn_decode_noalloc -- srft_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same computation, arguments, checks
 * and results as srft_attn_decode with a workspace of
 * rtq_attn_workspace_bytes(...) bytes, but the token-split workspace is a
 * static device array of the library (4,228,096 bytes: the largest one the
 * split policy asks for), so the caller passes none and nothing is
 * allocated, by the library or by the caller.
 *   Scratch: each GPU the library runs on holds its own copy until the
 *   process ends.  The first call on a device looks up its address and
 *   clears it with a kernel launched on `stream` (after the argument
 *   checks); every call that completes leaves it cleared again.
 *   Concurrency: every call on one GPU shares that GPU's scratch, so calls
 *   that may overlap in time on one GPU (other streams, other host threads)
 *   race and give wrong results; serialize them, or use srft_attn_decode
 *   with workspaces of their own.
 *   Errors: as srft_attn_decode; RTQ_ERR_HIP if the scratch cannot be set up
 *   on the current device; RTQ_ERR_UNSUPPORTED if a call's split plan needed
 *   more scratch than the array holds (none does under the current policy).
 */
rtq_status srft_attn_decode_noalloc(const void* q_f16, const void* codes_u8, const void* scales_f16, void* out_f16,
                                    int32_t layers, int32_t streams, int32_t tokens, int32_t q_per_kv, int32_t d,
                                    int32_t group, int64_t stride_layer, int64_t stride_kv, int64_t stride_stream,
                                    int64_t stride_token, uint64_t seed, int64_t rows_per_seed, int32_t seed_period,
                                    float softmax_scale, hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* rtq_status_string(rtq_status status);

#ifdef __cplusplus
}
#endif

#endif /* RTQ_H */
