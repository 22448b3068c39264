"""Eager four-dispatch baseline: the same rotate-then-quantize computation as
the fused kernels, written as separate PyTorch operations (rotate, quantize,
dequantize, inverse rotate), for timing beside the fused kernels only.

This is the unfused form the method page measures against ("Quantization
Speed Is Often a Kernel Problem", section "First, the 17%": each of the four
steps launched as its own eager operation; section "Fusing four steps into two
kernels is not enough": the fused pair).  It follows the same contract as the C ABI (packed orthonormal
rfft, absmax/8 fp16 scales, round-half-even, clamp to [-8, 7], two's
complement nibbles, SplitMix64 signs and the per-row seed rule), using
torch.fft on the GPU (hipFFT underneath) and elementwise torch ops.  Nothing
in the library calls it, and it lives outside the package beside bench.py.
"""
from __future__ import annotations

import math

import numpy as np
import torch

_GAMMA = 0x9E3779B97F4A7C15
_MASK = (1 << 64) - 1


def _splitmix_sign_bits(seeds: np.ndarray, d: int) -> np.ndarray:
    """[len(seeds), d] array of sign bits: bit 63 of the (i+1)-th SplitMix64
    output started at each seed (Steele, Lea & Flood 2014), vectorized."""
    s = seeds.astype(np.uint64)[:, None]
    i = np.arange(1, d + 1, dtype=np.uint64)[None, :]
    with np.errstate(over="ignore"):
        z = s + i * np.uint64(_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return (z >> np.uint64(63)).astype(np.int64)


def sign_matrix(n: int, d: int, seed: int, rows_per_seed: int = 0, seed_period: int = 0,
                device="cuda", row0: int = 0) -> torch.Tensor:
    """[n, d] float32 +-1 signs of rows row0 .. row0+n-1 under the per-row seed rule."""
    rows = np.arange(row0, row0 + n, dtype=np.int64)
    if rows_per_seed:
        block = rows // rows_per_seed
        if seed_period:
            block %= seed_period
    else:
        block = np.zeros(n, dtype=np.int64)
    offsets, inverse = np.unique(block, return_inverse=True)
    seeds = (np.uint64(seed & _MASK) + offsets.astype(np.uint64))
    bits = _splitmix_sign_bits(seeds, d)                      # [distinct, d]
    signs = torch.from_numpy(1.0 - 2.0 * bits.astype(np.float32)).to(device)
    return signs[torch.from_numpy(inverse).to(device)]


def _hadamard(d: int, device) -> torch.Tensor:
    h = torch.ones((1, 1), dtype=torch.float32)
    while h.shape[0] < d:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    return (h / math.sqrt(d)).to(device)


def rotate(x16: torch.Tensor, signs: torch.Tensor, rot: str = "srft") -> torch.Tensor:
    """Dispatch 1: z = R (D x), fp32, packed to d reals."""
    u = x16.float() * signs
    d = u.shape[1]
    if rot == "srht":
        return u @ _hadamard(d, u.device)
    X = torch.view_as_real(torch.fft.rfft(u, dim=1, norm="ortho"))  # [n, d/2+1, 2]
    z = torch.empty_like(u)
    z[:, 0] = X[:, 0, 0]
    z[:, 1:d - 1] = math.sqrt(2.0) * X[:, 1:d // 2].reshape(-1, d - 2)
    z[:, d - 1] = X[:, d // 2, 0]
    return z


def quantize(z: torch.Tensor, group: int):
    """Dispatch 2: fp16 absmax/8 scales, round-half-even codes in [-8, 7],
    two per byte (even element in the low nibble)."""
    n, d = z.shape
    zg = z.view(n, d // group, group)
    s = (zg.abs().amax(dim=2) / 8.0).to(torch.float16)
    s = torch.where(torch.isinf(s), torch.full_like(s, 65504.0), s)
    sf = s.float().unsqueeze(2)
    q = torch.where(sf > 0, torch.round(zg / torch.where(sf > 0, sf, torch.ones_like(sf))), torch.zeros_like(zg))
    q = q.clamp(-8, 7).to(torch.int32).view(n, d) & 0xF
    codes = (q[:, 0::2] | (q[:, 1::2] << 4)).to(torch.uint8)
    return codes, s


def dequantize(codes: torch.Tensor, scales: torch.Tensor, d: int, group: int) -> torch.Tensor:
    """Dispatch 3: z_hat = s * q, fp32."""
    c = codes.to(torch.int32)
    q = torch.stack([c & 0xF, c >> 4], dim=2).view(c.shape[0], d)
    q = torch.where(q >= 8, q - 16, q).float()
    return (q.view(-1, d // group, group) * scales.float().unsqueeze(2)).view(-1, d)


def inverse_rotate(z: torch.Tensor, signs: torch.Tensor, rot: str = "srft") -> torch.Tensor:
    """Dispatch 4: y = fp16(D R^T z)."""
    n, d = z.shape
    if rot == "srht":
        u = z @ _hadamard(d, z.device)
    else:
        X = torch.zeros((n, d // 2 + 1, 2), dtype=torch.float32, device=z.device)
        X[:, 0, 0] = z[:, 0]
        X[:, 1:d // 2] = z[:, 1:d - 1].reshape(n, d // 2 - 1, 2) / math.sqrt(2.0)
        X[:, d // 2, 0] = z[:, d - 1]
        u = torch.fft.irfft(torch.view_as_complex(X), n=d, dim=1, norm="ortho")
    return (u * signs).to(torch.float16)


def quant_fwd(x16, group, seed, rows_per_seed=0, seed_period=0, rot="srft", signs=None):
    signs = sign_matrix(x16.shape[0], x16.shape[1], seed, rows_per_seed, seed_period, x16.device) \
        if signs is None else signs
    return quantize(rotate(x16, signs, rot), group)


def dequant_inv(codes, scales, d, group, seed, rows_per_seed=0, seed_period=0, rot="srft", signs=None):
    signs = sign_matrix(codes.shape[0], d, seed, rows_per_seed, seed_period, codes.device) \
        if signs is None else signs
    return inverse_rotate(dequantize(codes, scales, d, group), signs, rot)
