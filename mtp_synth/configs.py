"""Workload shapes for the MTP head.

Each configuration fixes the head's dimensions, the batch, the cache context,
the number of speculative steps K and the planted agreement rate of the
synthetic target. ``cid`` seeds every random stream of that configuration.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Config:
    name: str
    cid: int
    hidden: int
    n_q: int
    n_kv: int
    head_dim: int
    ffn: int
    vocab: int
    batch: int
    K: int
    ctx_lo: int              # cache length of every sequence (or the low end of U{lo..hi})
    ctx_hi: int | None       # None: all sequences have ctx_lo cached positions
    agree_lo: float          # planted agreement rate (or the low end of U[lo, hi])
    agree_hi: float | None
    dtype: str               # "f32" or "bf16": storage of weights, inputs and cache
    rope_theta: float = 1.0e6
    rms_eps: float = 1.0e-6

    def with_(self, **kw) -> "Config":
        return replace(self, **kw)


CONFIGS = {
    # Tiny fp32 head: H=256, 4/2 heads of 64, FFN 768, V=4096, B=1, 128 cached slots, K=3.
    "tiny": Config("tiny", 0, 256, 4, 2, 64, 768, 4096, 1, 3, 128, None, 0.8, None, "f32"),
    # Qwen3-8B-shaped head, bf16: H=4096, 32/8 heads of 128, FFN 12288, V=151936, B=1, L=4096, K=5.
    "q8b": Config("q8b", 1, 4096, 32, 8, 128, 12288, 151936, 1, 5, 4096, None, 0.9, None, "bf16"),
    # Same shape, B=32 with ragged cache lengths U{512..8192}, K=3, agreement 0.6.
    "q8b-b32": Config("q8b-b32", 2, 4096, 32, 8, 128, 12288, 151936, 32, 3, 512, 8192, 0.6, None,
                      "bf16"),
    # Qwen3-32B-shaped head, bf16: H=5120, 64/8 heads of 128, FFN 25600, B=8, L=32768, K=5,
    # agreement drawn per sequence from U[0.5, 0.95].
    "q32b": Config("q32b", 3, 5120, 64, 8, 128, 25600, 151936, 8, 5, 32768, None, 0.5, 0.95,
                   "bf16"),
    # Wide dense head, bf16: H=7168, 56/8 heads of 128, FFN 18432, V=129280, B=64, L=4096, K=1.
    "wide": Config("wide", 4, 7168, 56, 8, 128, 18432, 129280, 64, 1, 4096, None, 0.85, None,
                   "bf16"),
}


def get_config(name: str, **overrides) -> Config:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


__all__ = ["Config", "CONFIGS", "get_config", "replace"]
