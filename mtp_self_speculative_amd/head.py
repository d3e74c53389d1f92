"""PyTorch-facing wrapper of the C ABI: device memory and streams only.

``MtpHead`` owns the weight tensors' lifetime and the library workspace (a torch
allocation); ``MtpCache`` holds the MTP layer's single-layer KV cache and its
per-sequence len/pos. Every method marshals pointers into the library; no
arithmetic of the method happens here.
"""
from __future__ import annotations

import torch

from . import _lib as L

_DT = {torch.float32: L.MTP_F32, torch.bfloat16: L.MTP_BF16}


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class MtpCache:
    """k, v: [batch, n_kv, capacity, head_dim] (head dtype); len, pos: [batch] int32."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, lens: torch.Tensor, pos: torch.Tensor):
        assert k.shape == v.shape and k.dim() == 4 and k.is_contiguous() and v.is_contiguous()
        assert lens.dtype == torch.int32 and pos.dtype == torch.int32
        self.k, self.v, self.len, self.pos = k, v, lens, pos
        self.kv = L.mtp_kv(k.data_ptr(), v.data_ptr(), lens.data_ptr(), pos.data_ptr(),
                           k.shape[0], k.shape[2])

    @property
    def batch(self) -> int:
        return self.k.shape[0]

    @property
    def capacity(self) -> int:
        return self.k.shape[2]


class MtpHead:
    def __init__(self, *, hidden: int, n_q_heads: int, n_kv_heads: int, head_dim: int, ffn: int,
                 vocab: int, weights: dict, max_batch: int, max_k: int, max_capacity: int,
                 rope_theta: float = 1.0e6, rms_eps: float = 1.0e-6,
                 dtype: torch.dtype = torch.bfloat16):
        self.dtype = dtype
        self.cfg = L.make_config(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, rope_theta,
                                 rms_eps, _DT[dtype])
        self.weights = {}
        for name in L.WEIGHT_FIELDS:
            t = weights[name]
            if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
                raise ValueError(f"weight {name} must be a contiguous {dtype} device tensor")
            self.weights[name] = t
        self.w = L.mtp_weights(*[self.weights[n].data_ptr() for n in L.WEIGHT_FIELDS])
        self.max_batch, self.max_k, self.max_capacity = max_batch, max_k, max_capacity
        nbytes = L.mtp_workspace_size(self.cfg, max_batch, max_k, max_capacity)
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8,
                                     device=self.weights["lm_head"].device)
        base = self.workspace.data_ptr()
        off = (-base) % 256
        self.handle = L.mtp_create(self.cfg, self.w, max_batch, max_k, max_capacity, base + off,
                                   nbytes)

    def close(self) -> None:
        if getattr(self, "handle", None):
            L.mtp_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()

    @property
    def vocab(self) -> int:
        return self.cfg.vocab

    def draft(self, hidden: torch.Tensor, last_tokens: torch.Tensor, cache: MtpCache, K: int,
              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        B = hidden.shape[0]
        if out is None:
            out = torch.empty((B, K), dtype=torch.int32, device=hidden.device)
        L.mtp_draft(self.handle, hidden.data_ptr(), last_tokens.data_ptr(), cache.kv, B, K,
                    out.data_ptr(), _stream(stream))
        return out

    def draft_debug(self, hidden, last_tokens, cache: MtpCache, K: int, want_logits=False,
                    stream=None):
        B, H = hidden.shape
        dev = hidden.device
        out = torch.empty((B, K), dtype=torch.int32, device=dev)
        hid = torch.empty((K, B, H), dtype=torch.float32, device=dev)
        mx = torch.empty((K, B), dtype=torch.float32, device=dev)
        lg = torch.empty((K, B, self.vocab), dtype=torch.float32, device=dev) if want_logits else None
        L.mtp_draft_debug(self.handle, hidden.data_ptr(), last_tokens.data_ptr(), cache.kv, B, K,
                          out.data_ptr(), hid.data_ptr(), mx.data_ptr(), _ptr(lg), _stream(stream))
        return out, hid, mx, lg

    def draft_sample(self, hidden: torch.Tensor, last_tokens: torch.Tensor, cache: MtpCache,
                     K: int, temperature: float, seeds: torch.Tensor, offset: int,
                     out: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                     stream=None):
        """K draft steps sampling at `temperature`; seeds [B] int64 on the device.
        Returns (draft tokens [B, K] int32, draft logits [B, K, V] fp32)."""
        B = hidden.shape[0]
        dev = hidden.device
        if out is None:
            out = torch.empty((B, K), dtype=torch.int32, device=dev)
        lg = logits
        if lg is None:
            lg = torch.empty((B, K, self.vocab), dtype=torch.float32, device=dev)
        L.mtp_draft_sample(self.handle, hidden.data_ptr(), last_tokens.data_ptr(), cache.kv, B, K,
                           float(temperature), seeds.data_ptr(), int(offset), out.data_ptr(),
                           lg.data_ptr(), _stream(stream))
        return out, lg

    def verify_sample(self, target_logits: torch.Tensor, draft_logits: torch.Tensor | None,
                      draft_tokens: torch.Tensor | None, temperature: float, seeds: torch.Tensor,
                      offset: int, accepted: torch.Tensor | None = None,
                      next_token: torch.Tensor | None = None, stream=None):
        """Speculative-sampling verification against target logits [B, K+1, V]."""
        B, K1, V = target_logits.shape
        dev = target_logits.device
        if accepted is None:
            accepted = torch.empty(B, dtype=torch.int32, device=dev)
        if next_token is None:
            next_token = torch.empty(B, dtype=torch.int32, device=dev)
        L.mtp_verify_sample(self.handle, target_logits.data_ptr(), _ptr(draft_logits),
                            _ptr(draft_tokens), B, K1 - 1, float(temperature), seeds.data_ptr(),
                            int(offset), accepted.data_ptr(), next_token.data_ptr(),
                            _stream(stream))
        return accepted, next_token

    def verify(self, target_logits: torch.Tensor, draft_tokens: torch.Tensor | None,
               accepted: torch.Tensor | None = None, next_token: torch.Tensor | None = None,
               stream=None):
        B, K1, V = target_logits.shape
        dev = target_logits.device
        if accepted is None:
            accepted = torch.empty(B, dtype=torch.int32, device=dev)
        if next_token is None:
            next_token = torch.empty(B, dtype=torch.int32, device=dev)
        L.mtp_verify(self.handle, target_logits.data_ptr(), _ptr(draft_tokens), B, K1 - 1,
                     accepted.data_ptr(), next_token.data_ptr(), _stream(stream))
        return accepted, next_token

    def verify_hidden(self, target_hidden: torch.Tensor, target_norm: torch.Tensor,
                      draft_tokens: torch.Tensor | None, accepted: torch.Tensor | None = None,
                      next_token: torch.Tensor | None = None, stream=None):
        """Greedy verification from the target's pre-norm hidden states [B, K+1, H]
        through its final-norm gain [H] and the shared lm_head."""
        B, K1, _ = target_hidden.shape
        dev = target_hidden.device
        if accepted is None:
            accepted = torch.empty(B, dtype=torch.int32, device=dev)
        if next_token is None:
            next_token = torch.empty(B, dtype=torch.int32, device=dev)
        th = target_hidden.contiguous()
        L.mtp_verify_hidden(self.handle, th.data_ptr(), target_norm.data_ptr(),
                            _ptr(draft_tokens), B, K1 - 1, accepted.data_ptr(),
                            next_token.data_ptr(), _stream(stream))
        return accepted, next_token

    def catchup(self, cache: MtpCache, target_hidden: torch.Tensor, draft_tokens: torch.Tensor,
                accepted: torch.Tensor, stream=None) -> None:
        """Exact cache commit after verification (instead of rollback): rewrites the
        committed slots from the target's hidden states [B, K+1, H]."""
        B, K1, _ = target_hidden.shape
        th = target_hidden.contiguous()
        L.mtp_kv_catchup(self.handle, cache.kv, th.data_ptr(), draft_tokens.data_ptr(),
                         accepted.data_ptr(), B, K1 - 1, _stream(stream))

    def rollback(self, cache: MtpCache, accepted: torch.Tensor, K: int, stream=None) -> None:
        L.mtp_kv_rollback(self.handle, cache.kv, accepted.data_ptr(), accepted.shape[0], K,
                          _stream(stream))

    def set_profiling(self, mask: int) -> None:
        L.mtp_set_profiling(self.handle, mask)

    def get_profile(self) -> dict:
        return L.mtp_get_profile(self.handle)

    def get_error(self, stream=None) -> int:
        return L.mtp_get_error(self.handle, _stream(stream))
