"""Shared set-up for the GPU tests: moves seeded synthetic inputs to the device and
builds the library's head / cache objects. Not collected by pytest."""
from __future__ import annotations

import numpy as np

import mtp_synth as S

TOL = {"f32": 1e-4, "bf16": 2e-2}
MARGIN = 1e-2


def torch_mod():
    import torch
    return torch


def to_dev(a: np.ndarray, storage: str, device="cuda"):
    torch = torch_mod()
    if storage == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.float32:
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device)


def cache_to_np(t, storage: str) -> np.ndarray:
    torch = torch_mod()
    if storage == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def make_head(cfg, inp, max_batch=None, max_k=None, packed_copy=True):
    torch = torch_mod()
    from mtp_self_speculative_amd import MtpCache, MtpHead
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    w = {k: to_dev(v, cfg.dtype) for k, v in inp.weights.items()}
    head = MtpHead(hidden=cfg.hidden, n_q_heads=cfg.n_q, n_kv_heads=cfg.n_kv,
                   head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=cfg.vocab, weights=w,
                   max_batch=max_batch or cfg.batch, max_k=max_k or max(cfg.K, 1),
                   max_capacity=inp.capacity, rope_theta=cfg.rope_theta, rms_eps=cfg.rms_eps,
                   dtype=dt, packed_copy=packed_copy)
    cache = MtpCache(to_dev(inp.k_cache, cfg.dtype), to_dev(inp.v_cache, cfg.dtype),
                     torch.from_numpy(inp.lens.astype(np.int32)).cuda(),
                     torch.from_numpy(inp.pos.astype(np.int32)).cuda())
    return head, cache


def compare_draft(cfg, orc: dict, gpu_tokens, gpu_hidden, gpu_top2, gpu_logits=None):
    """Teacher-forced comparison: orc was run with force_tokens = gpu_tokens.
    gpu_top2 [K, B, 2] holds the GPU's largest logit and the largest other one per step.
    Tokens must agree wherever either side's own top-2 margin clears the near-tie margin.
    Returns the number of (b, k) tokens checked."""
    tol = TOL[cfg.dtype]
    K = gpu_tokens.shape[1]
    gpu_margin = gpu_top2[..., 0] - gpu_top2[..., 1]
    assert np.all(gpu_margin >= 0), "second-best logit above the drafted token's"
    checked = 0
    for k in range(K):
        for b in range(gpu_tokens.shape[0]):
            if orc["margin"][k, b] > MARGIN or gpu_margin[k, b] > MARGIN + 2 * tol:
                assert int(orc["draft_tokens"][b, k]) == int(gpu_tokens[b, k]), (k, b)
                checked += 1
    dh = np.max(np.abs(gpu_hidden - orc["hidden_steps"]))
    assert dh < tol, f"hidden max-abs {dh}"
    dm = np.max(np.abs(gpu_top2[..., 0] - orc["top1"]))
    assert dm < tol, f"max-logit max-abs {dm}"
    d2 = np.max(np.abs(gpu_top2[..., 1] - (orc["top1"] - orc["margin"])))
    assert d2 < tol, f"second-logit max-abs {d2}"
    if gpu_logits is not None:
        dl = np.max(np.abs(gpu_logits - orc["logits"]))
        assert dl < tol, f"logits max-abs {dl}"
    return checked


def small(name="small", **kw) -> S.Config:
    base = dict(name=name, cid=100, hidden=384, n_q=6, n_kv=2, head_dim=128, ffn=1000,
                vocab=5003, batch=3, K=4, ctx_lo=1, ctx_hi=300, agree_lo=0.7, agree_hi=None,
                dtype="bf16")
    base.update(kw)
    return S.Config(**base)
