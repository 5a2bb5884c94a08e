"""Seeded synthetic K/V/Q inputs shaped like the workloads on the pages.

This module only draws random numbers and rounds them to bf16 (torch does both); it holds
none of the quantization arithmetic, and neither the HIP package nor the oracle is
imported here.  Both sides of every parity test take their inputs from here.

Shapes follow causal video-diffusion caches: a K or V chunk is [tokens, heads, head_dim],
flattened to rows = tokens * heads (row = one (token, head) vector).  Latent frames have
1560 tokens (Wan 14B-class) or 880 tokens (5B-class); chunks are 3 latent frames.

Value recipes (all drawn in float32, rounded to bf16 by torch's round-to-nearest-even):
  gauss_outliers   N(0,1), each element multiplied by 20 with probability 0.01
  channel_lognormal N(0,1) times a per-(head, channel) factor exp(N(0,1)) that is fixed for
                   a tensor (K-style channel outliers), fresh N(0,1) per chunk
  student_t_mix    N(0,1), each element replaced with probability 0.001 by a Student-t(3)
                   draw z / sqrt(chi2_3 / 3)
  query            N(0,1) * scale
Seeds are derived from (config seed, layer, kv, chunk) by `sub_seed`, so any group can be
regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

GENERATOR_VERSION = 1


def sub_seed(seed: int, *parts: int) -> int:
    s = seed & 0xFFFFFFFF
    for p in parts:
        s = (s * 1_000_003 + int(p) + 0x9E37) & 0x7FFFFFFFFFFF
    return s


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gauss_outliers(shape, seed: int, p: float = 0.01, mul: float = 20.0, device="cpu"):
    g = _gen(seed, device)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    hit = torch.rand(shape, generator=g, device=device, dtype=torch.float32) < p
    z = torch.where(hit, z * mul, z)
    return z.to(torch.bfloat16)


def channel_factors(heads: int, head_dim: int, seed: int, device="cpu"):
    g = _gen(seed, device)
    return torch.exp(torch.randn((heads, head_dim), generator=g, device=device,
                                 dtype=torch.float32))


def channel_lognormal(tokens: int, heads: int, head_dim: int, seed: int, factors,
                      device="cpu"):
    g = _gen(seed, device)
    z = torch.randn((tokens, heads, head_dim), generator=g, device=device, dtype=torch.float32)
    return (z * factors.to(device)).to(torch.bfloat16)


def student_t_mix(shape, seed: int, p: float = 0.001, dof: int = 3, device="cpu"):
    g = _gen(seed, device)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    hit = torch.rand(shape, generator=g, device=device, dtype=torch.float32) < p
    n = int(hit.sum().item())
    if n:
        zt = torch.randn((n,), generator=g, device=device, dtype=torch.float32)
        chi2 = (torch.randn((n, dof), generator=g, device=device, dtype=torch.float32) ** 2).sum(-1)
        z[hit] = zt / torch.sqrt(chi2 / dof)
    return z.to(torch.bfloat16)


def query(shape, seed: int, scale: float, device="cpu"):
    g = _gen(seed, device)
    return (torch.randn(shape, generator=g, device=device, dtype=torch.float32) * scale).to(
        torch.bfloat16)


# ---- the five workloads ------------------------------------------------------------------

@dataclass(frozen=True)
class CacheConfig:
    name: str
    layers: int
    heads: int
    head_dim: int
    chunk_tokens: int
    chunks: int
    seed: int

    @property
    def rows_per_group(self) -> int:          # one chunk of one tensor
        return self.chunk_tokens * self.heads

    @property
    def groups_per_chunk(self) -> int:        # every layer's K and V
        return self.layers * 2

    @property
    def cache_tokens(self) -> int:
        return self.chunk_tokens * self.chunks


# Tiny round trip: K and V [1, 256, 4, 64], N(0,1) with 1% x20 outliers, seed 0.
C1 = CacheConfig("tiny_roundtrip_256x4x64", layers=1, heads=4, head_dim=64, chunk_tokens=256,
                 chunks=1, seed=0)
# One layer's chunk append: K and V [1, 4680 (3 x 1560), 12, 128], channel log-normal.
C2 = CacheConfig("chunk_append_4680x12x128", layers=1, heads=12, head_dim=128,
                 chunk_tokens=4680, chunks=1, seed=2)
# Full-cache read: 30 layers x K,V [1, 32760 (21 x 1560), 12, 128] in 7 chunks of 4680.
C3 = CacheConfig("full_cache_30Lx32760x12x128", layers=30, heads=12, head_dim=128,
                 chunk_tokens=4680, chunks=7, seed=3)
# 5B-shaped rollout step: 30 layers, 24 heads, cache 36960 tokens (42 x 880) = 14 chunks of
# 2640 tokens (3 x 880), Gaussian with 0.1% Student-t(3) entries.
C4 = CacheConfig("rollout_5b_30Lx36960x24x128", layers=30, heads=24, head_dim=128,
                 chunk_tokens=2640, chunks=14, seed=4)
# Fused attention: Q [4680, 12, 128] N(0,1)/sqrt(128) against K/V [32760, 12, 128] N(0,1)
# quantized static_6 in 7 groups of 4680 tokens.
C5 = CacheConfig("attend_q4680_kv32760x12x128", layers=1, heads=12, head_dim=128,
                 chunk_tokens=4680, chunks=7, seed=5)
C5_Q_TOKENS = 4680

CONFIGS = {"C1": C1, "C2": C2, "C3": C3, "C4": C4, "C5": C5}

# Paged cache: the pages' dequantize_kv_cache example uses 16-token blocks; here a
# full-cache-sized paged cache of 30 layers x K,V x 2048 pages of 16 tokens (32768 tokens)
# x 12 heads x 128, values as the full-cache workload (channel log-normal).
P1 = CacheConfig("paged_30Lx2048px16x12x128", layers=30, heads=12, head_dim=128,
                 chunk_tokens=16, chunks=2048, seed=6)


def paged_tensor(cfg: CacheConfig, layer: int, kv: int, device="cpu"):
    """bf16 [chunks * chunk_tokens, heads, head_dim] of one layer's K or V (all its pages)."""
    f = channel_factors(cfg.heads, cfg.head_dim, sub_seed(cfg.seed, layer, kv, 1 << 20),
                        device=device)
    return channel_lognormal(cfg.chunks * cfg.chunk_tokens, cfg.heads, cfg.head_dim,
                             sub_seed(cfg.seed, layer, kv, 0), f, device=device)


def chunk_group(cfg: CacheConfig, layer: int, kv: int, chunk: int, device="cpu"):
    """bf16 [chunk_tokens, heads, head_dim] for one (layer, K/V, chunk) scale group."""
    shape = (cfg.chunk_tokens, cfg.heads, cfg.head_dim)
    s = sub_seed(cfg.seed, layer, kv, chunk)
    if cfg is C1:
        return gauss_outliers(shape, s, device=device)
    if cfg is C2 or cfg is C3:
        f = channel_factors(cfg.heads, cfg.head_dim, sub_seed(cfg.seed, layer, kv, 1 << 20),
                            device=device)
        return channel_lognormal(*shape, seed=s, factors=f, device=device)
    if cfg is C4:
        return student_t_mix(shape, s, device=device)
    if cfg is C5:
        g = _gen(s, device)
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    raise ValueError(cfg)


def chunk_all_layers(cfg: CacheConfig, chunk: int, device="cpu"):
    """bf16 [layers * 2 * chunk_tokens * heads, head_dim]: every layer's K then V for one
    chunk, in (layer, kv) order -- one contiguous append slab."""
    parts = [chunk_group(cfg, l, kv, chunk, device=device).reshape(-1, cfg.head_dim)
             for l in range(cfg.layers) for kv in (0, 1)]
    return torch.cat(parts, 0)


def c5_query(device="cpu"):
    return query((C5_Q_TOKENS, C5.heads, C5.head_dim), sub_seed(C5.seed, 99), 128 ** -0.5,
                 device=device)
