"""Seeded synthetic K/V workloads (shapes and value distributions only).

This module holds none of the method's arithmetic: it builds fp16 input
tensors and the per-row seed parameters, and is the one piece shared by the
tests, the bench and the oracle-side checks.  No model weights or datasets are
used; these tensors stand in for the K/V caches of the models named below.

Row layout.  Layer-major workloads store rows as [layer][kv][batch*head][token]
so one sign seed per layer is seed + (row // rows_per_seed) with
rows_per_seed = kv * batch * heads * tokens and seed_period = layers.  The
decode workload is time-major, [token][layer][kv][batch*head], so
rows_per_seed = kv * batch * heads and seed_period = layers again.

Value recipes (seeded with torch generators, data seed = 1000 * workload id +
10 * layer + kv):
  * normal: i.i.d. N(0, 1), then outlier channels multiplied by a factor;
  * student_t3: i.i.d. Student-t with 3 degrees of freedom, Z / sqrt(V / 3)
    with V a sum of three squared normals (heavy tails).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    d: int
    group: int
    rots: tuple
    layers: int
    kv: int
    streams: int          # batch * kv_heads
    tokens: int
    layout: str           # "layer_major" | "time_major"
    dist: str             # "normal" | "student_t3"
    outlier: str          # "none" | "fixed" | "per_stream" | "per_layer" | "bernoulli"
    outlier_count: int = 0
    outlier_prob: float = 0.0
    outlier_scale: float = 1.0
    fixed_channels: tuple = ()
    new_tokens: int = 0   # decode: rows quantized per step = new_tokens * layers * kv * streams
    q_per_kv: int = 1     # query heads per K/V head of the model (grouped-query attention)

    @property
    def n_rows(self) -> int:
        return self.layers * self.kv * self.streams * self.tokens

    @property
    def rows_per_seed(self) -> int:
        if self.layers <= 1:
            return 0
        if self.layout == "layer_major":
            return self.kv * self.streams * self.tokens
        return self.kv * self.streams

    @property
    def seed_period(self) -> int:
        return self.layers if self.layers > 1 else 0

    @property
    def cache_strides(self) -> tuple:
        """Row of (layer, kv, stream, token) = layer*s0 + kv*s1 + stream*s2 +
        token*s3 in this workload's layout."""
        if self.layout == "layer_major":
            return (self.kv * self.streams * self.tokens, self.streams * self.tokens, self.tokens, 1)
        return (self.kv * self.streams, self.streams, 1, self.layers * self.kv * self.streams)

    @property
    def sign_seed(self) -> int:
        return 0x5EED * self.wid

    @property
    def new_rows(self) -> int:
        return self.new_tokens * self.layers * self.kv * self.streams

    def bytes_per_vector(self) -> int:
        """Algorithmic HBM bytes of one vector in one direction: fp16 in/out,
        int4 codes, fp16 scales."""
        return 2 * self.d + self.d // 2 + 2 * (self.d // self.group)

    def scaled(self, tokens: int) -> "Workload":
        """Same recipe with fewer tokens per stream (parity-test sizes)."""
        return replace(self, tokens=tokens)


WORKLOADS = {
    1: Workload(1, "per_token_outlier_4096x64", d=64, group=64, rots=("srft",), layers=1, kv=1, streams=1,
                tokens=4096, layout="layer_major", dist="normal", outlier="fixed", outlier_scale=20.0,
                fixed_channels=(3, 17)),
    2: Workload(2, "smollm2_360m_prefill_kv", d=64, group=32, rots=("srft",), layers=32, kv=2, streams=5,
                tokens=4096, layout="layer_major", dist="normal", outlier="per_stream", outlier_count=2,
                outlier_scale=15.0, q_per_kv=3),
    3: Workload(3, "qwen2.5_1.5b_decode_kv", d=128, group=32, rots=("srft",), layers=28, kv=2, streams=64 * 2,
                tokens=2049, layout="time_major", dist="student_t3", outlier="none", new_tokens=1, q_per_kv=6),
    4: Workload(4, "smollm2_1.7b_kv", d=64, group=64, rots=("srft", "srht"), layers=24, kv=2, streams=32,
                tokens=2048, layout="layer_major", dist="normal", outlier="bernoulli", outlier_prob=0.01,
                outlier_scale=20.0),
    5: Workload(5, "gemma3_1b_long_kv", d=256, group=32, rots=("srft",), layers=26, kv=2, streams=16,
                tokens=32768, layout="layer_major", dist="normal", outlier="per_layer", outlier_count=4,
                outlier_scale=25.0, q_per_kv=4),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _values(w: Workload, shape, g, device):
    if w.dist == "normal":
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if w.dist == "student_t3":
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        v = torch.randn((3,) + tuple(shape), generator=g, device=device, dtype=torch.float32).square_().sum(0)
        return z / torch.sqrt(v / 3.0)
    raise ValueError(w.dist)


def generate(w: Workload, device="cuda", out: torch.Tensor | None = None) -> torch.Tensor:
    """The whole [n_rows, d] fp16 input of workload ``w`` on ``device``."""
    device = torch.device(device)
    if out is None:
        out = torch.empty((w.n_rows, w.d), dtype=torch.float16, device=device)
    if w.layout == "time_major":
        # i.i.d. values: fill in slabs of tokens, one generator per slab
        per_tok = w.layers * w.kv * w.streams
        slab = max(1, (1 << 24) // (per_tok * w.d))
        for i, t0 in enumerate(range(0, w.tokens, slab)):
            t1 = min(w.tokens, t0 + slab)
            g = _gen(device, 1000 * w.wid + i)
            out[t0 * per_tok:t1 * per_tok] = _values(w, ((t1 - t0) * per_tok, w.d), g, device).to(torch.float16)
        return out
    chunk = w.streams * w.tokens
    for layer in range(w.layers):
        for kv in range(w.kv):
            g = _gen(device, 1000 * w.wid + 10 * layer + kv)
            vals = _values(w, (w.streams, w.tokens, w.d), g, device)
            if w.outlier == "fixed":
                vals[..., list(w.fixed_channels)] *= w.outlier_scale
            elif w.outlier == "per_stream":
                # outlier_count distinct channels per (layer, kv, head)
                ch = torch.rand((w.streams, w.d), generator=g, device=device).argsort(dim=1)[:, :w.outlier_count]
                mult = torch.ones((w.streams, w.d), device=device)
                mult.scatter_(1, ch, w.outlier_scale)
                vals *= mult[:, None, :]
            elif w.outlier == "per_layer":
                ch = torch.rand((w.d,), generator=g, device=device).argsort()[:w.outlier_count]
                vals[..., ch] *= w.outlier_scale
            elif w.outlier == "bernoulli":
                hit = torch.rand((w.streams, w.d), generator=g, device=device) < w.outlier_prob
                vals *= torch.where(hit, w.outlier_scale, 1.0)[:, None, :]
            base = (layer * w.kv + kv) * chunk
            out[base:base + chunk] = vals.reshape(chunk, w.d).to(torch.float16)
    return out


def decode_step_rows(w: Workload) -> tuple[int, int]:
    """(rows quantized, rows dequantized) of one decode step of ``w``."""
    return w.new_rows, w.n_rows
