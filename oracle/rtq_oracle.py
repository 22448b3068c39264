"""Plain fp64 CPU oracle for rotate-then-quantize int4 KV-cache compression.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or run anything in this package.  It shares no code, table,
constant generator or helper with the HIP library and imports nothing from it.

Everything here is written to be checked by eye against the source pages:
explicit O(d^2) matrices, scalar rounding rules, no blocking or fusion.

Sources (cited by page title and section):
  [P1] "Quantization Speed Is Often a Kernel Problem" -- the method page.
  [P3] "Day 9 - Quantization: Shrink the Bytes Themselves".
  [P4] "Quantization & Serving".
  [P5] "Chapter 25 - Quantization: The Hardware View".

What the pages fix and what is this oracle's reading where they leave a step open:
  * Each K/V vector is rotated, quantized to int4, and later dequantized and
    rotated back [P1, "First, the 17%"].
  * SRFT = flip signs with a constant pseudo-random +-1 vector, then take an FFT (rfft on the
    way in, irfft on the way out) [P1, "First, the 17%"].  Reading: the
    orthonormal real DFT, with the d/2+1 complex bins packed into d reals as
    [X0, sqrt2*Re X1, sqrt2*Im X1, ..., sqrt2*Im X_{d/2-1}, X_{d/2}].
  * SRHT = sign-randomized Hadamard transform, the control rotation
    [P1, "First, the 17%"].  Reading: (1/sqrt d) * Sylvester H_d.
  * Symmetric absmax quantization, zero point 0 [P3, "What Quantization Is,
    Mathematically"; P4].  Reading: scale = fp16(absmax / 8) (the int4
    worked examples on P3 divide by 8), code = clamp(round-half-even(z/s),
    -8, 7) (the clamp range of the symmetric quantizer code on P5, "Python:
    Quantize, Simulate the Integer GEMM, and Compute the Savings").
  * Scales are fp16 values [P3, "How Many Numbers Should One Scale Cover"];
    one absmax scale per group of consecutive values [P1, "Fusing four steps
    into two kernels is not enough"].
  * Two int4 codes per byte, w0 in the low nibble, w1 in the high nibble,
    read back as signed values [P5, "Kernels: Marlin, CUTLASS, and Why INT4
    Packing Needs Special Code"].  Reading: two's complement nibbles.
  * The +-1 vector: the pages do not say how it is drawn.  Reading: sign i of
    seed S is -1 iff bit 63 of the (i+1)-th output of the published SplitMix64
    generator (Steele, Lea, Flood 2014) started at state S is set; the seed of
    row r is S + ((r div rows_per_seed) mod seed_period), with 0 meaning
    "one seed for all rows" / "no modulo".
"""

from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1
SPLITMIX64_GAMMA = 0x9E3779B97F4A7C15
INT4_MIN = -8
INT4_MAX = 7
FP16_MAX = 65504.0

# ---------------------------------------------------------------------------
# Sign vector (the SRFT's +-1 sign flip, [P1, "First, the 17%"])
# ---------------------------------------------------------------------------


def splitmix64_stream(state: int, count: int) -> list[int]:
    """The first ``count`` outputs of SplitMix64 started at ``state``.

    Published generator (Steele, Lea & Flood, "Fast splittable pseudorandom
    number generators", OOPSLA 2014; Vigna's reference implementation): the
    state advances by the golden-ratio increment, and each output is the
    state passed through two xor-shift-multiply rounds and a final xor-shift.
    """
    out = []
    s = state & MASK64
    for _ in range(count):
        s = (s + SPLITMIX64_GAMMA) & MASK64
        z = s
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
        out.append(z ^ (z >> 31))
    return out


def sign_vector(seed: int, d: int) -> np.ndarray:
    """D in {+1,-1}^d for one seed: -1 where bit 63 of output i is set."""
    return np.array(
        [-1.0 if (o >> 63) & 1 else 1.0 for o in splitmix64_stream(seed, d)],
        dtype=np.float64,
    )


def row_seed(seed: int, row: int, rows_per_seed: int, seed_period: int) -> int:
    """Seed of row ``row``: seed + ((row // rows_per_seed) % seed_period).

    rows_per_seed == 0 means every row uses ``seed``; seed_period == 0 means
    the block index is not wrapped.  Arithmetic is modulo 2^64.
    """
    if rows_per_seed == 0:
        return seed & MASK64
    block = row // rows_per_seed
    if seed_period != 0:
        block %= seed_period
    return (seed + block) & MASK64


def sign_matrix(n: int, d: int, seed: int, rows_per_seed: int = 0,
                seed_period: int = 0, row0: int = 0, rows=None) -> np.ndarray:
    """[n, d] matrix of per-row sign vectors for rows row0 .. row0+n-1, or for
    the listed row indices when ``rows`` is given."""
    cache: dict[int, np.ndarray] = {}
    out = np.empty((n, d), dtype=np.float64)
    for i in range(n):
        s = row_seed(seed, row0 + i if rows is None else int(rows[i]), rows_per_seed, seed_period)
        if s not in cache:
            cache[s] = sign_vector(s, d)
        out[i] = cache[s]
    return out


# ---------------------------------------------------------------------------
# Rotations R (d x d, orthonormal)
# ---------------------------------------------------------------------------


def srft_matrix(d: int) -> np.ndarray:
    """Packed orthonormal real DFT, written out from its definition.

    X_k = (1/sqrt d) * sum_n u_n * exp(-2*pi*i*k*n/d), k = 0..d/2 (the rfft of
    [P1, "First, the 17%"] with orthonormal scaling).  Rows of R, in order:
      row 0        : X_0                      (real)
      row 2k-1     : sqrt(2) * Re X_k,  k = 1 .. d/2-1
      row 2k       : sqrt(2) * Im X_k,  k = 1 .. d/2-1
      row d-1      : X_{d/2}                  (real)
    The sqrt(2) on interior bins makes R^T R = I.
    """
    if d < 2 or d % 2:
        raise ValueError("d must be even and >= 2")
    n = np.arange(d)
    half = d // 2
    R = np.empty((d, d), dtype=np.float64)
    R[0, :] = 1.0 / math.sqrt(d)
    for k in range(1, half):
        # reduce k*n mod d before forming the angle to keep it small
        ang = 2.0 * math.pi * ((k * n) % d) / d
        R[2 * k - 1, :] = math.sqrt(2.0 / d) * np.cos(ang)
        R[2 * k, :] = -math.sqrt(2.0 / d) * np.sin(ang)
    R[d - 1, :] = np.where(n % 2 == 0, 1.0, -1.0) / math.sqrt(d)
    return R


def srht_matrix(d: int) -> np.ndarray:
    """(1/sqrt d) * H_d with H[i][k] = (-1)^popcount(i & k) (Sylvester order).

    The sign-randomized Hadamard control of [P1, "First, the 17%"].
    """
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    H = np.empty((d, d), dtype=np.float64)
    for i in range(d):
        for k in range(d):
            H[i, k] = -1.0 if bin(i & k).count("1") % 2 else 1.0
    return H / math.sqrt(d)


_MATRIX_CACHE: dict[tuple[str, int], np.ndarray] = {}


def rotation_matrix(rot: str, d: int) -> np.ndarray:
    key = (rot, d)
    if key not in _MATRIX_CACHE:
        if rot == "srft":
            _MATRIX_CACHE[key] = srft_matrix(d)
        elif rot == "srht":
            _MATRIX_CACHE[key] = srht_matrix(d)
        elif rot == "none":
            _MATRIX_CACHE[key] = np.eye(d)
        else:
            raise ValueError(f"unknown rotation {rot!r}")
    return _MATRIX_CACHE[key]


# ---------------------------------------------------------------------------
# Symmetric absmax int4 quantizer
# ---------------------------------------------------------------------------


def fp16_scale_from_absmax(a: np.ndarray) -> np.ndarray:
    """s = fp16(absmax / 8), round-to-nearest-even, saturated at 65504.

    Divisor 8: the int4 worked examples of [P3, "What Quantization Is,
    Mathematically"] (range -8..8 over 16 cells gives scale 1) and [P3, "How
    Many Numbers Should One Scale Cover"] (a group whose largest value is 20
    gets scale 20/8 = 2.5).  fp16 storage: same section of P3.
    """
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        s = (a / 8.0).astype(np.float16)
    return np.where(np.isinf(s), np.float16(FP16_MAX), s).astype(np.float16)


def quantize_with_scale(z: np.ndarray, s: np.ndarray) -> np.ndarray:
    """q = clamp(round_half_even(z / s), -8, 7); q = 0 where s == 0.

    The rounding-and-clamp step of the symmetric quantizer ([P3, "What
    Quantization Is, Mathematically"]; clamp to [-qmax-1, qmax] as in the
    quantizer code of [P5, "Python: Quantize, Simulate ..."]; its round is
    half-to-even).  ``s`` is the stored fp16 scale, widened exactly.
    """
    z = np.asarray(z, dtype=np.float64)
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    r = np.where(s64 > 0, z / safe, 0.0)
    return np.clip(np.rint(r), INT4_MIN, INT4_MAX).astype(np.int8)


def quantize_groups(z: np.ndarray, group: int):
    """Per-row, per-group absmax int4 quantization of the last axis.

    Groups are consecutive runs of ``group`` values ([P1, "Fusing four steps
    into two kernels is not enough": one absmax per 32 values]; group == d
    is the per-token recipe).  Returns (q int8 [..., d], s float16
    [..., d/group], a float64 [..., d/group]) where a is the exact absmax.
    """
    z = np.asarray(z, dtype=np.float64)
    d = z.shape[-1]
    if d % group:
        raise ValueError("group must divide d")
    zg = z.reshape(z.shape[:-1] + (d // group, group))
    a = np.max(np.abs(zg), axis=-1)
    s = fp16_scale_from_absmax(a)
    q = quantize_with_scale(zg, s[..., None])
    return q.reshape(z.shape), s, a


def dequantize_groups(q: np.ndarray, s: np.ndarray, group: int) -> np.ndarray:
    """x_hat = s * q (zero point 0), per group, in fp64."""
    q = np.asarray(q, dtype=np.float64)
    d = q.shape[-1]
    qg = q.reshape(q.shape[:-1] + (d // group, group))
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)
    return (qg * s64[..., None]).reshape(q.shape)


# ---------------------------------------------------------------------------
# Nibble packing ([P5, "Kernels: Marlin, CUTLASS, and Why INT4 Packing ..."])
# ---------------------------------------------------------------------------


def pack_nibbles(q: np.ndarray) -> np.ndarray:
    """byte m = (q[2m] & 0xF) | ((q[2m+1] & 0xF) << 4): w0 low, w1 high."""
    q = np.asarray(q, dtype=np.int64)
    lo = q[..., 0::2] & 0xF
    hi = q[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    """w0 = byte & 0x0F, w1 = (byte >> 4) & 0x0F, each sign-extended."""
    b = np.asarray(b, dtype=np.int64)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


# ---------------------------------------------------------------------------
# The two fused operations, as plain steps
# ---------------------------------------------------------------------------


def rotate_fwd(x_f16: np.ndarray, seed: int, rows_per_seed: int = 0,
               seed_period: int = 0, rot: str = "srft", row0: int = 0, rows=None) -> np.ndarray:
    """z = R (D (.) x) per row, fp64.  Sign first, then the transform.  Row i
    is cache row row0 + i, or rows[i] when ``rows`` is given."""
    x = np.asarray(x_f16, dtype=np.float16).astype(np.float64)
    n, d = x.shape
    D = sign_matrix(n, d, seed, rows_per_seed, seed_period, row0, rows)
    u = D * x
    return u @ rotation_matrix(rot, d).T


def rotate_inv(z: np.ndarray, seed: int, rows_per_seed: int = 0,
               seed_period: int = 0, rot: str = "srft", row0: int = 0, rows=None) -> np.ndarray:
    """u = D (.) (R^T z) per row, fp64 (before the fp16 rounding of y)."""
    z = np.asarray(z, dtype=np.float64)
    n, d = z.shape
    D = sign_matrix(n, d, seed, rows_per_seed, seed_period, row0, rows)
    return D * (z @ rotation_matrix(rot, d))


def quant_fwd(x_f16: np.ndarray, group: int, seed: int, rows_per_seed: int = 0,
              seed_period: int = 0, rot: str = "srft", row0: int = 0, rows=None):
    """Forward: sign, rotate, per-group absmax int4, pack.

    Returns (codes uint8 [n, d/2], scales float16 [n, d/group]).
    """
    z = rotate_fwd(x_f16, seed, rows_per_seed, seed_period, rot, row0, rows)
    q, s, _ = quantize_groups(z, group)
    return pack_nibbles(q), s


def dequant_inv(codes: np.ndarray, scales: np.ndarray, d: int, group: int,
                seed: int, rows_per_seed: int = 0, seed_period: int = 0,
                rot: str = "srft", row0: int = 0, return_fp64: bool = False, rows=None):
    """Inverse: unpack, dequantize, inverse-rotate, sign, round to fp16."""
    q = unpack_nibbles(codes)
    if q.shape[-1] != d:
        raise ValueError("codes do not match d")
    zhat = dequantize_groups(q, scales, group)
    u = rotate_inv(zhat, seed, rows_per_seed, seed_period, rot, row0, rows)
    with np.errstate(over="ignore"):
        y = u.astype(np.float16)
    return (y, u) if return_fp64 else y


def forward_detail(x_f16: np.ndarray, group: int, seed: int, rows_per_seed: int = 0,
                   seed_period: int = 0, rot: str = "srft", row0: int = 0, rows=None) -> dict:
    """All intermediate values of the forward step, for tolerance checks."""
    z = rotate_fwd(x_f16, seed, rows_per_seed, seed_period, rot, row0, rows)
    q, s, a = quantize_groups(z, group)
    return {"z": z, "q": q, "s": s, "a": a, "codes": pack_nibbles(q)}


# ---------------------------------------------------------------------------
# Other code widths and a per-channel lambda ([P1, "First, the 17%": the
# fused recipe adds one scale per channel to the per-group absmax, and the
# quality study runs 3-, 4-, 6- and 8-bit codes)
#
# Readings (the page gives neither formula): b-bit codes use the int4 rule
# with 2^(b-1) in place of 8: s = fp16(absmax / 2^(b-1)), q = clamp(rne(z/s),
# -2^(b-1), 2^(b-1)-1).  A row's codes form one little-endian bit stream:
# code i fills stream bits [i*b, (i+1)*b), stream bit k is bit (k mod 8) of
# byte k div 8, each field two's complement (b = 4 is the nibble layout
# above).  lambda is a caller-given fp16 vector, one value per channel,
# multiplied into x before the sign flip and divided out after the inverse
# rotation.
# ---------------------------------------------------------------------------

CODE_BITS = (3, 4, 6, 8)


def fp16_scale_bits(a: np.ndarray, bits: int) -> np.ndarray:
    """s = fp16(absmax / 2^(bits-1)), round-to-nearest-even, saturated at 65504."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(over="ignore"):
        s = (a / float(1 << (bits - 1))).astype(np.float16)
    return np.where(np.isinf(s), np.float16(FP16_MAX), s).astype(np.float16)


def quantize_groups_bits(z: np.ndarray, group: int, bits: int):
    """Per-group absmax b-bit quantization of the last axis: (q, s, a)."""
    z = np.asarray(z, dtype=np.float64)
    d = z.shape[-1]
    zg = z.reshape(z.shape[:-1] + (d // group, group))
    a = np.max(np.abs(zg), axis=-1)
    s = fp16_scale_bits(a, bits)
    s64 = s.astype(np.float64)[..., None]
    r = np.where(s64 > 0, zg / np.where(s64 > 0, s64, 1.0), 0.0)
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    q = np.clip(np.rint(r), lo, hi).astype(np.int16)
    return q.reshape(z.shape), s, a


def pack_bits(q: np.ndarray, bits: int) -> np.ndarray:
    """Rows of b-bit two's-complement codes -> bytes [..., d*bits/8], one
    little-endian bit stream per row."""
    q = np.asarray(q, dtype=np.int64)
    d = q.shape[-1]
    flat = q.reshape(-1, d) & ((1 << bits) - 1)
    out = np.zeros((flat.shape[0], d * bits // 8), dtype=np.uint8)
    for i in range(d):
        for k in range(bits):
            bit = (flat[:, i] >> k) & 1
            pos = i * bits + k
            out[:, pos // 8] |= (bit << (pos % 8)).astype(np.uint8)
    return out.reshape(q.shape[:-1] + (d * bits // 8,))


def unpack_bits(b: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Inverse of pack_bits: bytes -> sign-extended b-bit codes [..., d]."""
    b = np.asarray(b, dtype=np.int64)
    flat = b.reshape(-1, b.shape[-1])
    q = np.zeros((flat.shape[0], d), dtype=np.int64)
    for i in range(d):
        for k in range(bits):
            pos = i * bits + k
            q[:, i] |= ((flat[:, pos // 8] >> (pos % 8)) & 1) << k
    q = np.where(q >= (1 << (bits - 1)), q - (1 << bits), q)
    return q.astype(np.int16).reshape(b.shape[:-1] + (d,))


def forward_detail_ext(x_f16: np.ndarray, group: int, bits: int, lam_f16, seed: int, rows_per_seed: int = 0,
                       seed_period: int = 0, rot: str = "srft", row0: int = 0, rows=None) -> dict:
    """Forward with b-bit codes and an optional per-channel lambda: u = D (.)
    (lambda (.) x), z = R u, per-group absmax b-bit quantization, packing."""
    x = np.asarray(x_f16, dtype=np.float16).astype(np.float64)
    n, d = x.shape
    if lam_f16 is not None:
        x = x * np.asarray(lam_f16, dtype=np.float16).astype(np.float64)[None, :]
    D = sign_matrix(n, d, seed, rows_per_seed, seed_period, row0, rows)
    z = (D * x) @ rotation_matrix(rot, d).T
    q, s, a = quantize_groups_bits(z, group, bits)
    return {"z": z, "q": q, "s": s, "a": a, "codes": pack_bits(q, bits)}


def quant_fwd_ext(x_f16: np.ndarray, group: int, bits: int, lam_f16, seed: int, rows_per_seed: int = 0,
                  seed_period: int = 0, rot: str = "srft", row0: int = 0, rows=None):
    """(codes uint8 [n, d*bits/8], scales float16 [n, d/group])."""
    det = forward_detail_ext(x_f16, group, bits, lam_f16, seed, rows_per_seed, seed_period, rot, row0, rows)
    return det["codes"], det["s"]


def dequant_inv_ext(codes: np.ndarray, scales: np.ndarray, d: int, group: int, bits: int, lam_f16, seed: int,
                    rows_per_seed: int = 0, seed_period: int = 0, rot: str = "srft", row0: int = 0,
                    return_fp64: bool = False, rows=None):
    """Unpack b-bit codes, dequantize, inverse-rotate, flip signs, divide by
    lambda, round to fp16."""
    q = unpack_bits(codes, bits, d)
    zhat = dequantize_groups(q, scales, group)
    u = rotate_inv(zhat, seed, rows_per_seed, seed_period, rot, row0, rows)
    if lam_f16 is not None:
        u = u / np.asarray(lam_f16, dtype=np.float16).astype(np.float64)[None, :]
    with np.errstate(over="ignore"):
        y = u.astype(np.float16)
    return (y, u) if return_fp64 else y


# ---------------------------------------------------------------------------
# Generic granularity helper for the MSE-ordering check of [P4]
# ---------------------------------------------------------------------------


def int4_roundtrip_blocks(w: np.ndarray, block_rows: int, block_cols: int) -> np.ndarray:
    """Quantize-dequantize ``w`` with one absmax scale per (block_rows x block_cols) tile.

    (rows, cols) = whole matrix -> per-tensor; (1, cols) -> per-row (channel);
    (1, g) -> per-group.  Same scale and rounding rules as the method.
    """
    w = np.asarray(w, dtype=np.float64)
    r, c = w.shape
    if r % block_rows or c % block_cols:
        raise ValueError("blocks must tile the matrix")
    t = w.reshape(r // block_rows, block_rows, c // block_cols, block_cols)
    a = np.max(np.abs(t), axis=(1, 3))
    s = fp16_scale_from_absmax(a)
    sb = s[:, None, :, None]
    q = quantize_with_scale(t, sb)
    return (q.astype(np.float64) * sb.astype(np.float64)).reshape(r, c)


# ---------------------------------------------------------------------------
# Attention over the compressed cache (the consumer that dequantizes when it
# reads the cache: [P1, "First, the 17%"]; "Dequantize in the attention
# consumer" is the plain composition of dequant_inv and softmax attention).
# ---------------------------------------------------------------------------


def window_schedule(prefill_tokens: int, appended: int, window: int) -> tuple[int, int]:
    """(tokens in the int4 cache, tokens in the fp16 window) after a prefill
    of ``prefill_tokens`` (all quantized) and ``appended`` single-token
    appends, when the newest tokens stay in an fp16 window of ``window``
    tokens that is quantized as a whole, and the dequantized prefix refreshed,
    when it fills ([P1] "First, the 17%")."""
    quantized, held = prefill_tokens, 0
    for _ in range(appended):
        held += 1
        if held == window:
            quantized, held = quantized + window, 0
    return quantized, held


def cache_rows(layer: int, kv: int, stream: int, tokens: int, strides) -> np.ndarray:
    """Row indices of tokens 0 .. tokens-1 of one (layer, K/V, stream) in a
    cache whose row of (layer, kv, stream, t) is
    layer*strides[0] + kv*strides[1] + stream*strides[2] + t*strides[3]
    (kv = 0 for keys, 1 for values)."""
    sl, skv, ss, st = (int(v) for v in strides)
    return layer * sl + kv * skv + stream * ss + st * np.arange(tokens, dtype=np.int64)


def dequant_rows(codes: np.ndarray, scales: np.ndarray, rows: np.ndarray, d: int, group: int, seed: int,
                 rows_per_seed: int = 0, seed_period: int = 0, rot: str = "srft") -> np.ndarray:
    """u = D(seed'(r)) (R^T z_hat) of each listed row r, in fp64: the steps of
    dequant_inv (unpack, dequantize, inverse rotation, sign flip) before its
    fp16 rounding, for rows that need not be consecutive."""
    rows = np.asarray(rows, dtype=np.int64)
    zhat = dequantize_groups(unpack_nibbles(codes[rows]), scales[rows], group)
    u = zhat @ rotation_matrix(rot, d)
    row_seeds = [row_seed(seed, int(r), rows_per_seed, seed_period) for r in rows]
    for s in set(row_seeds):
        idx = [i for i, v in enumerate(row_seeds) if v == s]
        u[idx] *= sign_vector(s, d)
    return u


def attn_decode(q_f16: np.ndarray, codes: np.ndarray, scales: np.ndarray, strides, layers: int, streams: int,
                tokens: int, q_per_kv: int, d: int, group: int, seed: int, rows_per_seed: int = 0,
                seed_period: int = 0, rot: str = "srft", softmax_scale: float | None = None,
                pairs=None, window: np.ndarray | None = None, window_tokens: int = 0) -> np.ndarray:
    """One decode step of attention for every (layer, stream): query g of
    q[layer, stream] attends over the first `tokens` cached keys and values of
    its stream (rows from cache_rows), each dequantized and rotated back
    exactly (fp64, no fp16 rounding), followed by the first `window_tokens`
    tokens of the fp16 window (window[layer, kv, stream, j], kept unquantized
    in the original domain, as the method page's decode cache keeps its newest
    tokens: "Quantization Speed Is Often a Kernel Problem", "First, the 17%");
    one softmax runs over all of them; softmax_scale defaults to 1/sqrt(d).
    Returns o [layers, streams, q_per_kv, d] in fp64 (entries of (layer,
    stream) pairs outside `pairs`, when a list is given, stay zero)."""
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    q = np.asarray(q_f16, dtype=np.float16).astype(np.float64).reshape(layers, streams, q_per_kv, d)
    o = np.zeros_like(q)
    todo = [(l, s) for l in range(layers) for s in range(streams)] if pairs is None else list(pairs)
    for layer, st in todo:
        u = []
        for kv in (0, 1):
            rows = cache_rows(layer, kv, st, tokens, strides)
            part = dequant_rows(codes, scales, rows, d, group, seed, rows_per_seed, seed_period, rot)
            if window_tokens:
                win = np.asarray(window[layer, kv, st, :window_tokens], dtype=np.float16).astype(np.float64)
                part = np.concatenate([part, win])
            u.append(part)
        keys, values = u
        for g in range(q_per_kv):
            sc = keys @ q[layer, st, g] * softmax_scale
            w = np.exp(sc - sc.max())
            o[layer, st, g] = (w / w.sum()) @ values
    return o
