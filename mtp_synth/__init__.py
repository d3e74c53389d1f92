"""Seeded synthetic inputs for the MTP draft / verify / rollback path.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic. Both the oracle (``oracle/``) and the GPU path take
their inputs from here, so the two sides see bit-identical data.

Seed streams: every array comes from ``numpy.random.SeedSequence([cid, stream,
sub])`` split into fixed-size chunks (``CHUNK`` elements, one spawned child per
chunk), so the values depend neither on the thread count nor on the machine.

    stream 0  projection weights and lm_head, N(0, 0.02)
    stream 1  norm gains, N(1, 0.02)
    stream 2  shared token embedding, N(0, 1)
    stream 3  verifier hidden states, N(0, 1) (sub = iteration)
    stream 4  last_tokens, uniform over the vocabulary
    stream 5  initial MTP K/V cache, N(0, 1)
    stream 6  ragged cache lengths
    stream 7  target-logit noise, N(0, 1) (sub = iteration)
    stream 8  planting Bernoullis (sub = iteration)
    stream 9  per-sequence agreement rate
    stream 10 small synthetic target decoder: projections, N(0, 0.02)
    stream 11 small synthetic target decoder: norm gains, N(1, 0.02)
    stream 12 prompts for the synthetic target
    stream 13 target hidden states for verification from hidden states, N(0, 1)
              (sub = iteration)
    stream 14 the target's final-norm gain, N(1, 0.02)
    stream 15 logits for sampling verification (sub 2*it: target rows, N(0, scale^2);
              sub 2*it+1: draft-row perturbation, N(0, noise^2))
    stream 16 per-sequence random-stream seeds, uniform 63-bit integers
    stream 17 target hidden states over a prompt (prefill), N(0, 1) (sub = call)
    stream 18 the token after each prompt position (prefill), uniform over the vocabulary

bf16 configurations draw in fp32 and round to bf16 (round to nearest even);
bf16 arrays are carried as their uint16 bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

from .configs import CONFIGS, Config, get_config  # noqa: F401

CHUNK = 1 << 21

# Sub-stream ids inside stream 0 (projection weights) and stream 1 (gains).
PROJ_SUB = {"w_eh": 0, "w_q": 1, "w_k": 2, "w_v": 3, "w_o": 4,
            "w_gate": 5, "w_up": 6, "w_down": 7, "lm_head": 8}
GAIN_SUB = {"g_h": 0, "g_e": 1, "g_attn": 2, "g_mlp": 3, "g_final": 4}

WEIGHT_NAMES = ("g_h", "g_e", "w_eh", "g_attn", "w_q", "w_k", "w_v", "w_o",
                "g_mlp", "w_gate", "w_up", "w_down", "g_final", "embed", "lm_head")


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


_POOL: ThreadPoolExecutor | None = None


def _pool() -> ThreadPoolExecutor:
    global _POOL
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=_workers())
    return _POOL


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(cid: int, stream: int, sub: int, n: int, mean: float = 0.0, std: float = 1.0,
           out_dtype: str = "f32") -> np.ndarray:
    """n draws of N(mean, std^2) as float32, or as bf16 bits when out_dtype == 'bf16'."""
    ss = np.random.SeedSequence([cid, stream, sub])
    nchunks = max(1, math.ceil(n / CHUNK))
    kids = ss.spawn(nchunks)
    out = np.empty(n, np.uint16 if out_dtype == "bf16" else np.float32)

    def fill(i: int) -> None:
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        if hi <= lo:
            return
        g = np.random.Generator(np.random.PCG64(kids[i]))
        t = g.standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            t *= np.float32(std)
        if mean != 0.0:
            t += np.float32(mean)
        if out_dtype == "bf16":
            out[lo:hi] = f32_to_bf16_bits(t)
        else:
            out[lo:hi] = t

    if nchunks == 1:
        fill(0)
    else:
        list(_pool().map(fill, range(nchunks)))
    return out


def _rng(cid: int, stream: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cid, stream, sub])))


def weight_shapes(cfg: Config) -> dict:
    H, F, V = cfg.hidden, cfg.ffn, cfg.vocab
    qd, kvd = cfg.n_q * cfg.head_dim, cfg.n_kv * cfg.head_dim
    return {
        "g_h": (H,), "g_e": (H,), "w_eh": (H, 2 * H), "g_attn": (H,),
        "w_q": (qd, H), "w_k": (kvd, H), "w_v": (kvd, H), "w_o": (H, qd),
        "g_mlp": (H,), "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F),
        "g_final": (H,), "embed": (V, H), "lm_head": (V, H),
    }


def make_weights(cfg: Config) -> dict:
    """All MTP-head weights plus the shared embedding / lm_head, in storage dtype."""
    dt = cfg.dtype
    out = {}
    for name, shape in weight_shapes(cfg).items():
        n = int(np.prod(shape))
        if name in GAIN_SUB:
            a = normal(cfg.cid, 1, GAIN_SUB[name], n, 1.0, 0.02, dt)
        elif name == "embed":
            a = normal(cfg.cid, 2, 0, n, 0.0, 1.0, dt)
        else:
            a = normal(cfg.cid, 0, PROJ_SUB[name], n, 0.0, 0.02, dt)
        out[name] = a.reshape(shape)
    return out


def cache_lengths(cfg: Config) -> np.ndarray:
    if cfg.ctx_hi is None:
        return np.full(cfg.batch, cfg.ctx_lo, np.int32)
    g = _rng(cfg.cid, 6)
    return g.integers(cfg.ctx_lo, cfg.ctx_hi + 1, size=cfg.batch).astype(np.int32)


def agreement(cfg: Config) -> np.ndarray:
    if cfg.agree_hi is None:
        return np.full(cfg.batch, cfg.agree_lo, np.float64)
    g = _rng(cfg.cid, 9)
    return g.uniform(cfg.agree_lo, cfg.agree_hi, size=cfg.batch)


def hidden_states(cfg: Config, it: int = 0) -> np.ndarray:
    """Verifier hidden state handed to the draft at iteration `it`, [B, H] storage dtype."""
    return normal(cfg.cid, 3, it, cfg.batch * cfg.hidden, 0.0, 1.0, cfg.dtype).reshape(
        cfg.batch, cfg.hidden)


def target_hidden(cfg: Config, K: int, it: int = 0) -> np.ndarray:
    """The target's pre-norm hidden states at the K+1 verified inputs, [B, K+1, H]."""
    return normal(cfg.cid, 13, it, cfg.batch * (K + 1) * cfg.hidden, 0.0, 1.0,
                  cfg.dtype).reshape(cfg.batch, K + 1, cfg.hidden)


def target_norm(cfg: Config) -> np.ndarray:
    """The target's final-norm gain, [H]."""
    return normal(cfg.cid, 14, 0, cfg.hidden, 1.0, 0.02, cfg.dtype)


def prefill_hidden(cfg: Config, n: int, sub: int = 0) -> np.ndarray:
    """The target's pre-norm hidden states at n prompt positions, [B, n, H], N(0, 1)."""
    return normal(cfg.cid, 17, sub, cfg.batch * n * cfg.hidden, 0.0, 1.0,
                  cfg.dtype).reshape(cfg.batch, n, cfg.hidden)


def prefill_tokens(cfg: Config, n: int, sub: int = 0) -> np.ndarray:
    """The token after each of n prompt positions, [B, n] int32, uniform over the vocabulary."""
    return _rng(cfg.cid, 18, sub).integers(0, cfg.vocab, size=(cfg.batch, n)).astype(np.int32)


def last_tokens(cfg: Config) -> np.ndarray:
    return _rng(cfg.cid, 4).integers(0, cfg.vocab, size=cfg.batch).astype(np.int32)


def default_capacity(cfg: Config, iters: int = 64) -> int:
    return int(cache_lengths(cfg).max()) + iters * max(cfg.K, 1)


def kv_cache(cfg: Config, capacity: int) -> tuple[np.ndarray, np.ndarray]:
    """Initial MTP cache, [B, n_kv, S, d] storage dtype, every slot N(0, 1)."""
    shape = (cfg.batch, cfg.n_kv, capacity, cfg.head_dim)
    n = int(np.prod(shape))
    k = normal(cfg.cid, 5, 0, n, 0.0, 1.0, cfg.dtype).reshape(shape)
    v = normal(cfg.cid, 5, 1, n, 0.0, 1.0, cfg.dtype).reshape(shape)
    return k, v


def plant_target_logits(cfg: Config, draft_tokens: np.ndarray, it: int = 0,
                        bump: float = 8.0) -> np.ndarray:
    """Synthetic target logits [B, K+1, V] float32.

    Every row is N(0, 1) noise. Row j < K scores the token after verified input j
    (inputs are [last_token, d_1 .. d_K]); with probability p_b it also gets +bump
    at the draft token d_{j+1}, so that the target agrees with that draft.
    Row K gets noise only.
    """
    d = np.asarray(draft_tokens, dtype=np.int64).reshape(cfg.batch, -1)
    K = d.shape[1]
    B, V = cfg.batch, cfg.vocab
    t = normal(cfg.cid, 7, it, B * (K + 1) * V, 0.0, 1.0, "f32").reshape(B, K + 1, V)
    if K:
        u = _rng(cfg.cid, 8, it).random((B, K))
        hit = u < agreement(cfg)[:, None]
        bb, jj = np.nonzero(hit)
        t[bb, jj, d[bb, jj]] += np.float32(bump)
    return t


def sampling_logits(cfg: Config, K: int, it: int = 0, scale: float = 3.0,
                    noise: float = 1.0) -> tuple[np.ndarray, np.ndarray]:
    """Target logits [B, K+1, V] ~ N(0, scale^2) and draft logits [B, K, V] equal to the
    first K target rows plus N(0, noise^2), float32. With the defaults about 60% of
    sampled drafts are accepted at temperature 1 over a large vocabulary."""
    B, V = cfg.batch, cfg.vocab
    t = normal(cfg.cid, 15, 2 * it, B * (K + 1) * V, 0.0, scale, "f32").reshape(B, K + 1, V)
    e = normal(cfg.cid, 15, 2 * it + 1, B * K * V, 0.0, noise, "f32").reshape(B, K, V)
    return t, (t[:, :K] + e).astype(np.float32)


def sample_seeds(cfg: Config, sub: int = 0) -> np.ndarray:
    """One random-stream seed per sequence, [B] uint64."""
    return _rng(cfg.cid, 16, sub).integers(0, 2 ** 63, size=cfg.batch, dtype=np.uint64)


TARGET_PROJ = ("w_q", "w_k", "w_v", "w_o", "w_gate", "w_up", "w_down")
TARGET_GAIN = ("g_attn", "g_mlp")


def target_weights(cfg: Config, n_layers: int = 2) -> dict:
    """Weights of a small random decoder stack of the head's shape, used as a synthetic
    verifier in end-to-end checks. It shares the embedding and lm_head of the head.
    Returns {"layers": [dict per layer], "g_final": gain} in storage dtype."""
    shapes = weight_shapes(cfg)
    layers = []
    for li in range(n_layers):
        lw = {}
        for j, name in enumerate(TARGET_PROJ):
            n = int(np.prod(shapes[name]))
            lw[name] = normal(cfg.cid, 10, li * 16 + j, n, 0.0, 0.02, cfg.dtype).reshape(
                shapes[name])
        for j, name in enumerate(TARGET_GAIN):
            lw[name] = normal(cfg.cid, 11, li * 16 + j, cfg.hidden, 1.0, 0.02, cfg.dtype)
        layers.append(lw)
    g_final = normal(cfg.cid, 11, 1000, cfg.hidden, 1.0, 0.02, cfg.dtype)
    return {"layers": layers, "g_final": g_final}


def prompt_tokens(cfg: Config, n: int, sub: int = 0) -> np.ndarray:
    return _rng(cfg.cid, 12, sub).integers(0, cfg.vocab, size=n).astype(np.int32)


@dataclass
class SynthInputs:
    cfg: Config
    capacity: int
    weights: dict
    hidden: np.ndarray
    last_tokens: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    lens: np.ndarray
    pos: np.ndarray
    agree: np.ndarray = field(default=None)


def make_inputs(cfg: Config, capacity: int | None = None) -> SynthInputs:
    cap = default_capacity(cfg) if capacity is None else int(capacity)
    lens = cache_lengths(cfg)
    if int(lens.max()) + cfg.K > cap:
        raise ValueError("capacity too small for the configured cache lengths")
    k, v = kv_cache(cfg, cap)
    return SynthInputs(cfg=cfg, capacity=cap, weights=make_weights(cfg),
                       hidden=hidden_states(cfg, 0), last_tokens=last_tokens(cfg),
                       k_cache=k, v_cache=v, lens=lens.copy(), pos=lens.copy(),
                       agree=agreement(cfg))


__all__ = ["CONFIGS", "Config", "get_config", "replace", "make_inputs", "make_weights",
           "hidden_states", "last_tokens", "kv_cache", "cache_lengths", "agreement",
           "plant_target_logits", "f32_to_bf16_bits", "bf16_bits_to_f32", "normal",
           "weight_shapes", "default_capacity", "SynthInputs", "WEIGHT_NAMES",
           "target_weights", "prompt_tokens"]
