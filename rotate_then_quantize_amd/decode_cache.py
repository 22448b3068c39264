"""A decode-time K/V cache: int4 rotated codes for the quantized prefix, a
dequantized fp16 copy of that prefix kept between steps, and an fp16 window
of the newest tokens.

This is the cache policy the method page describes for decoding
("Quantization Speed Is Often a Kernel Problem", "First, the 17%"): the
dequantized prefix is cached between steps instead of being recomputed; the
newest 16 tokens stay in fp16; when that window fills, its tokens are
quantized into the int4 cache and the dequantized prefix is refreshed.  Rows
are independent, so refreshing the prefix only needs the rows that were just
quantized (``*_dequant_rows``); the result equals dequantizing the whole
prefix again.

Host orchestration only: every quantization and dequantization runs in the
HIP kernels (``*_quant_append`` and ``*_dequant_rows``), and ``attention``
reads the int4 prefix and the fp16 window in one kernel
(``*_attn_decode_window``); PyTorch allocates the buffers and copies each new
token into the window.

With ``keep_prefix=False`` no dequantized copy is kept: a consumer that
reads the int4 prefix directly (``attention``) needs none, which saves its
memory (3.5x the int4 cache at d = 128, g = 32) and the refresh on every
flush.

Layout: rows ``[layer][K, V][stream][token]`` with ``capacity`` token slots
per stream (strides ``(2*streams*capacity, streams*capacity, capacity, 1)``),
one sign seed per layer (``rows_per_seed = 2*streams*capacity``,
``seed_period = layers``).
"""
from __future__ import annotations

import rotate_then_quantize_amd as rtq


class DecodeCache:
    def __init__(self, layers: int, streams: int, capacity: int, d: int, group: int, seed: int,
                 rot: str = "srft", window: int = 16, device="cuda", keep_prefix: bool = True):
        import torch
        if min(layers, streams, capacity, window) < 1:
            raise ValueError("layers, streams, capacity and window must be positive")
        if window > rtq.ATTN_MAX_WINDOW:
            raise ValueError(f"window must be at most {rtq.ATTN_MAX_WINDOW} tokens (the attention kernel's limit)")
        if (d, group) not in rtq.CACHE_SUPPORTED:
            raise ValueError(f"(d, group) = ({d}, {group}) is not supported for the decode cache")
        self.layers, self.streams, self.capacity, self.d, self.group = layers, streams, capacity, d, group
        self.seed, self.rot, self.window = seed, rot, window
        n = layers * 2 * streams * capacity
        self.strides = (2 * streams * capacity, streams * capacity, capacity, 1)
        self.rows_per_seed, self.seed_period = (2 * streams * capacity, layers) if layers > 1 else (0, 0)
        self.codes = torch.zeros((n, d // 2), dtype=torch.uint8, device=device)
        self.scales = torch.zeros((n, d // group), dtype=torch.float16, device=device)
        # dequantized copy (None without keep_prefix)
        self.prefix = torch.zeros((n, d), dtype=torch.float16, device=device) if keep_prefix else None
        self.window_kv = torch.zeros((layers, 2, streams, window, d), dtype=torch.float16, device=device)
        self.quantized = 0  # tokens in the int4 cache (and in the dequantized copy)
        self.held = 0       # tokens in the fp16 window

    @property
    def tokens(self) -> int:
        return self.quantized + self.held

    def _quantize(self, block, t0: int) -> None:
        """block [layers, 2, streams, n, d] fp16 -> cache tokens t0 .. t0+n-1, then refresh their rows of the
        dequantized copy (if one is kept)."""
        n = block.shape[3]
        rtq.quant_append(self.rot, block, self.codes, self.scales, self.strides, t0, self.group, self.seed,
                         self.rows_per_seed, self.seed_period)
        if self.prefix is not None:
            rtq.dequant_rows(self.rot, self.codes, self.scales, self.prefix, self.layers, self.streams, t0, n,
                             self.strides, self.group, self.seed, self.rows_per_seed, self.seed_period)

    def prefill(self, kv) -> None:
        """Quantize a prompt's K/V, kv [layers, 2, streams, tokens, d] fp16, into an empty cache."""
        if self.tokens:
            raise RuntimeError("prefill needs an empty cache")
        if tuple(kv.shape[:3]) != (self.layers, 2, self.streams) or kv.shape[4] != self.d:
            raise ValueError(f"kv must be [{self.layers}, 2, {self.streams}, tokens, {self.d}]")
        if kv.shape[3] > self.capacity:
            raise ValueError("the prompt does not fit the cache")
        self._quantize(kv.contiguous(), 0)
        self.quantized = kv.shape[3]

    def append(self, kv) -> None:
        """Add one token's K/V, kv [layers, 2, streams, d] fp16.  It stays in the fp16 window; when the window
        is full, the whole window is quantized into the cache and the dequantized copy (if kept) refreshed."""
        if tuple(kv.shape) != (self.layers, 2, self.streams, self.d):
            raise ValueError(f"kv must be [{self.layers}, 2, {self.streams}, {self.d}]")
        if self.tokens + 1 > self.capacity:
            raise RuntimeError("the cache is full")
        self.window_kv[:, :, :, self.held].copy_(kv)
        self.held += 1
        if self.held == self.window:
            self._quantize(self.window_kv, self.quantized)
            self.quantized += self.window
            self.held = 0

    def attention(self, q, softmax_scale=None, out=None):
        """One decode step of attention over everything the cache holds: q [layers, streams, q_per_kv, d]
        fp16 attends over the int4 prefix and the fp16 window in one launch (*_attn_decode_window)."""
        return rtq.attn_decode(self.rot, q, self.codes, self.scales, self.strides, self.quantized, self.group,
                               self.seed, self.rows_per_seed, self.seed_period, softmax_scale, out=out,
                               window=self.window_kv, window_tokens=self.held)

    def row(self, layer: int, kv: int, stream: int, token: int) -> int:
        """Cache row of (layer, kv, stream, token)."""
        s = self.strides
        return layer * s[0] + kv * s[1] + stream * s[2] + token * s[3]
