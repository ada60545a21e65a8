"""Seeded synthetic Q/K/V generators shared by the tests, the bench and the oracle checks.

This module only draws random numbers; it holds none of Sol-Attn's arithmetic.
Every tensor is produced on the CPU with ``torch.Generator`` (portable and
reproducible), in float32, then rounded once to bfloat16 (RNE) in the
[batch, tokens, heads, head_dim] (BTHD) layout that the Sol-Attn README's
"Core API" fixes.  The shapes mimic the workloads the Sol-Attn pages measure
(video DiT self-attention on latent grids in raster order); see the recipe
descriptions below.

Recipes
-------
block_offset
    x = eps + o_blk: eps ~ N(0,1) per element, plus one offset vector
    o ~ N(0, offset_std^2 I) per (tensor, head, 64-token block), so block
    means differ and routing is non-trivial.
smooth_field
    per (tensor, head, channel): white noise on a (T, H, W) latent grid,
    Gaussian-filtered with sigma = corr cells on every axis (reflect
    boundaries), standardised to unit variance, plus noise_std * N(0,1);
    tokens laid out in raster (t, h, w) order.
text_prefix
    `prefix` i.i.d. N(0,1) tokens followed by a block_offset body (joint
    text + video attention with the text kept as an exact sink).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

BLOCK = 64


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def block_offset_tensor(batch: int, tokens: int, heads: int, dim: int, seed: int,
                        offset_std: float = 1.0, block: int = BLOCK) -> torch.Tensor:
    """One BTHD bf16 tensor: N(0,1) noise plus a per-(head, block) offset vector."""
    g = _gen(seed)
    nb = (tokens + block - 1) // block
    out = torch.empty(batch, tokens, heads, dim, dtype=torch.bfloat16)
    # Offsets are drawn first so that the body noise can be streamed in chunks.
    offs = torch.randn(batch, nb, heads, dim, generator=g, dtype=torch.float32) * offset_std
    chunk_blocks = max(1, (1 << 24) // (block * heads * dim))
    for b in range(batch):
        for j0 in range(0, nb, chunk_blocks):
            j1 = min(nb, j0 + chunk_blocks)
            t0, t1 = j0 * block, min(tokens, j1 * block)
            eps = torch.randn(t1 - t0, heads, dim, generator=g, dtype=torch.float32)
            blk_idx = torch.arange(t0, t1) // block - j0
            eps += offs[b, j0:j1][blk_idx]
            out[b, t0:t1] = eps.to(torch.bfloat16)
    return out


def smooth_field_tensor(batch: int, grid: tuple, heads: int, dim: int, seed: int,
                        corr: float = 4.0, noise_std: float = 0.3) -> torch.Tensor:
    """One BTHD bf16 tensor: standardised Gaussian random field on `grid` plus white noise."""
    from scipy.ndimage import gaussian_filter

    rng = np.random.Generator(np.random.PCG64(int(seed)))
    T, Hh, W = grid
    tokens = T * Hh * W
    out = torch.empty(batch, tokens, heads, dim, dtype=torch.bfloat16)
    for b in range(batch):
        white = rng.standard_normal((heads * dim, T, Hh, W), dtype=np.float32)
        field = gaussian_filter(white, sigma=(0, corr, corr, corr), mode="reflect")
        field = field.reshape(heads * dim, tokens)
        field -= field.mean(axis=1, keepdims=True)
        field /= field.std(axis=1, keepdims=True) + 1e-12
        field += noise_std * rng.standard_normal(field.shape, dtype=np.float32)
        # [H*D, tokens] -> [tokens, H, D]
        out[b] = torch.from_numpy(np.ascontiguousarray(field.T)).reshape(tokens, heads, dim).to(torch.bfloat16)
    return out


def text_prefix_tensor(batch: int, prefix: int, body_tokens: int, heads: int, dim: int,
                       seed: int, offset_std: float = 1.0) -> torch.Tensor:
    """`prefix` i.i.d. N(0,1) text tokens, then a block_offset body."""
    g = _gen(seed + 7919)
    text = torch.randn(batch, prefix, heads, dim, generator=g, dtype=torch.float32).to(torch.bfloat16)
    body = block_offset_tensor(batch, body_tokens, heads, dim, seed, offset_std)
    return torch.cat([text, body], dim=1).contiguous()


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    tokens: int
    heads: int
    dim: int
    kind: str                      # "block_offset" | "smooth_field" | "text_prefix"
    seed_base: int
    grid: Optional[tuple] = None   # (T, H, W) for smooth_field
    prefix: int = 0                # text tokens for text_prefix
    sink_start: int = -1
    sink_tokens: int = 0
    offset_std: float = 1.0

    def make(self, which: int) -> torch.Tensor:
        """which = 0, 1, 2 for q, k, v; seeds are seed_base + which."""
        seed = self.seed_base + which
        if self.kind == "block_offset":
            return block_offset_tensor(self.batch, self.tokens, self.heads, self.dim, seed, self.offset_std)
        if self.kind == "smooth_field":
            return smooth_field_tensor(self.batch, self.grid, self.heads, self.dim, seed)
        if self.kind == "text_prefix":
            return text_prefix_tensor(self.batch, self.prefix, self.tokens - self.prefix,
                                      self.heads, self.dim, seed, self.offset_std)
        raise ValueError(self.kind)

    def qkv(self):
        return self.make(0), self.make(1), self.make(2)


def tiny(tokens: int = 1024, heads: int = 2, batch: int = 1, seed_base: int = 1000) -> Workload:
    """Tiny Sol-Attn forward: B=1, H=2, N=1024 (16 blocks), d=128, block-offset data."""
    return Workload("tiny", batch, tokens, heads, 128, "block_offset", seed_base)


def wan_dit(batch: int = 1, seed_base: int = 2000) -> Workload:
    """Wan-2.1-1.3B-shaped DiT self-attention: H=12, N=14040 = 9x30x52 raster grid."""
    return Workload("wan21_1.3b_dit", batch, 9 * 30 * 52, 12, 128, "smooth_field", seed_base, grid=(9, 30, 52))


def operator_bench(tokens: int = 32768, batch: int = 1, seed_base: int = 3000) -> Workload:
    """Operator benchmark shape: H=32, d=128, N=32768 (8x64x64 grid), block-offset data."""
    return Workload("op_bench", batch, tokens, 32, 128, "block_offset", seed_base)


def long_sink(video_tokens: int = 65536, batch: int = 1, seed_base: int = 4000) -> Workload:
    """Long sequence with an exact text sink: 512 text tokens then `video_tokens` body tokens."""
    return Workload("long_sink", batch, 512 + video_tokens, 32, 128, "text_prefix", seed_base,
                    prefix=512, sink_start=0, sink_tokens=512)


def sol2_bench(tokens: int = 32768, batch: int = 1, seed_base: int = 3000) -> Workload:
    """Sol-Attn2 benchmark: the operator benchmark data (FP8 Q/K are derived by the method)."""
    return Workload("sol2_bench", batch, tokens, 32, 128, "block_offset", seed_base)
