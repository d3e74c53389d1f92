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


def _need(name: str, t, dtype: torch.dtype, shape: tuple, device_type: str) -> None:
    """Raise ValueError unless t is a contiguous `dtype` tensor of exactly `shape` on a
    `device_type` device: the library reads these buffers by the shapes it is given, so a
    mismatch would read or write past them on the device."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.device.type != device_type:
        raise ValueError(f"{name} must be on a {device_type} device, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream) -> int | None:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


class MtpCache:
    """k, v: [batch, n_kv, capacity, head_dim] (head dtype); len, pos: [batch] int32."""

    def __init__(self, k: torch.Tensor, v: torch.Tensor, lens: torch.Tensor, pos: torch.Tensor):
        if not (isinstance(k, torch.Tensor) and isinstance(v, torch.Tensor)) or k.dim() != 4:
            raise ValueError("k and v must be [batch, n_kv, capacity, head_dim] tensors")
        _need("v", v, k.dtype, tuple(k.shape), k.device.type)
        _need("k", k, k.dtype, tuple(k.shape), k.device.type)
        _need("len", lens, torch.int32, (k.shape[0],), k.device.type)
        _need("pos", pos, torch.int32, (k.shape[0],), k.device.type)
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
    # Every tensor handed to the library must live here (tests of the host-side checks
    # point it at the CPU; the library itself then rejects the null handle).
    _device_type = "cuda"

    def __init__(self, *, hidden: int, n_q_heads: int, n_kv_heads: int, head_dim: int, ffn: int,
                 vocab: int, weights: dict, max_batch: int, max_k: int, max_capacity: int,
                 rope_theta: float = 1.0e6, rms_eps: float = 1.0e-6,
                 dtype: torch.dtype = torch.bfloat16, packed_copy: bool = True):
        """packed_copy=False: keep no re-laid-out copy of the weights in the workspace
        (MTP_CREATE_NO_PACKED_COPY); batches of 3+ sequences then read the weights in place."""
        self.dtype = dtype
        self.cfg = L.make_config(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, rope_theta,
                                 rms_eps, _DT[dtype])
        H, F, V = hidden, ffn, vocab
        qd, kvd = n_q_heads * head_dim, n_kv_heads * head_dim
        shapes = {"g_h": (H,), "g_e": (H,), "w_eh": (H, 2 * H), "g_attn": (H,), "w_q": (qd, H),
                  "w_k": (kvd, H), "w_v": (kvd, H), "w_o": (H, qd), "g_mlp": (H,),
                  "w_gate": (F, H), "w_up": (F, H), "w_down": (H, F), "g_final": (H,),
                  "embed": (V, H), "lm_head": (V, H)}
        self.weights = {}
        for name in L.WEIGHT_FIELDS:
            if name not in weights:
                raise ValueError(f"weight {name} is missing")
            _need(f"weight {name}", weights[name], dtype, shapes[name], self._device_type)
            self.weights[name] = weights[name]
        self.w = L.mtp_weights(*[self.weights[n].data_ptr() for n in L.WEIGHT_FIELDS])
        self.max_batch, self.max_k, self.max_capacity = max_batch, max_k, max_capacity
        self.flags = 0 if packed_copy else L.CREATE_NO_PACKED_COPY
        nbytes = L.mtp_workspace_size_ex(self.cfg, max_batch, max_k, max_capacity, self.flags)
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8,
                                     device=self.weights["lm_head"].device)
        base = self.workspace.data_ptr()
        off = (-base) % 256
        self.handle = L.mtp_create_ex(self.cfg, self.w, max_batch, max_k, max_capacity,
                                      self.flags, base + off, nbytes)

    def close(self) -> None:
        if getattr(self, "handle", None):
            L.mtp_destroy(self.handle)
            self.handle = None

    def __del__(self):
        self.close()

    @property
    def vocab(self) -> int:
        return self.cfg.vocab

    # ---- host-side checks of shapes, dtypes and devices (raise ValueError)

    def _t(self, name, t, dtype, shape):
        _need(name, t, dtype, shape, self._device_type)

    def _check_cache(self, cache: "MtpCache", B: int) -> None:
        c = self.cfg
        shape = (cache.k.shape[0], c.n_kv_heads, cache.k.shape[2], c.head_dim)
        self._t("cache.k", cache.k, self.dtype, shape)
        self._t("cache.v", cache.v, self.dtype, shape)
        self._t("cache.len", cache.len, torch.int32, (shape[0],))
        self._t("cache.pos", cache.pos, torch.int32, (shape[0],))
        if not 1 <= B <= shape[0]:
            raise ValueError(f"batch {B} outside 1..{shape[0]} (the cache's batch)")

    def _check_batch(self, B: int, K: int) -> None:
        if not 1 <= B <= self.max_batch:
            raise ValueError(f"batch {B} outside 1..{self.max_batch}")
        if not 0 <= K <= self.max_k:
            raise ValueError(f"K = {K} outside 0..{self.max_k}")

    def _check_draft_in(self, hidden, last_tokens, cache, K):
        if not isinstance(hidden, torch.Tensor) or hidden.dim() != 2:
            raise ValueError("hidden must be a [B, hidden] tensor")
        B = hidden.shape[0]
        self._check_batch(B, K)
        self._t("hidden", hidden, self.dtype, (B, self.cfg.hidden))
        self._t("last_tokens", last_tokens, torch.int32, (B,))
        self._check_cache(cache, B)
        return B

    def _check_outs(self, B, accepted, next_token):
        if accepted is not None:
            self._t("accepted", accepted, torch.int32, (B,))
        if next_token is not None:
            self._t("next_token", next_token, torch.int32, (B,))

    def _check_drafts(self, draft_tokens, B, K, required):
        if draft_tokens is None:
            if required and K > 0:
                raise ValueError("draft_tokens is required when K > 0")
            return
        self._t("draft_tokens", draft_tokens, torch.int32, (B, K))

    def _check_logits(self, target_logits):
        if not isinstance(target_logits, torch.Tensor) or target_logits.dim() != 3:
            raise ValueError("target_logits must be a [B, K+1, vocab] float32 tensor")
        B, K = target_logits.shape[0], target_logits.shape[1] - 1
        self._check_batch(B, K)
        self._t("target_logits", target_logits, torch.float32, (B, K + 1, self.vocab))
        return B, K

    def _check_target_hidden(self, target_hidden):
        if not isinstance(target_hidden, torch.Tensor) or target_hidden.dim() != 3:
            raise ValueError("target_hidden must be a [B, K+1, hidden] tensor")
        B, K = target_hidden.shape[0], target_hidden.shape[1] - 1
        self._check_batch(B, K)
        self._t("target_hidden", target_hidden, self.dtype, (B, K + 1, self.cfg.hidden))
        return B, K

    def draft(self, hidden: torch.Tensor, last_tokens: torch.Tensor, cache: MtpCache, K: int,
              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        B = self._check_draft_in(hidden, last_tokens, cache, K)
        if out is None:
            out = torch.empty((B, K), dtype=torch.int32, device=hidden.device)
        self._t("out", out, torch.int32, (B, K))
        L.mtp_draft(self.handle, hidden.data_ptr(), last_tokens.data_ptr(), cache.kv, B, K,
                    out.data_ptr(), _stream(stream))
        return out

    def draft_debug(self, hidden, last_tokens, cache: MtpCache, K: int, want_logits=False,
                    stream=None):
        """mtp_draft with diagnostics: (draft tokens [B, K], h^(k) [K, B, H], top-2 logits
        [K, B, 2] (the drafted token's and the best other one), logits [K, B, V] or None)."""
        B = self._check_draft_in(hidden, last_tokens, cache, K)
        H = hidden.shape[1]
        dev = hidden.device
        out = torch.empty((B, K), dtype=torch.int32, device=dev)
        hid = torch.empty((K, B, H), dtype=torch.float32, device=dev)
        top2 = torch.empty((K, B, 2), dtype=torch.float32, device=dev)
        lg = torch.empty((K, B, self.vocab), dtype=torch.float32, device=dev) if want_logits else None
        L.mtp_draft_debug(self.handle, hidden.data_ptr(), last_tokens.data_ptr(), cache.kv, B, K,
                          out.data_ptr(), hid.data_ptr(), top2.data_ptr(), _ptr(lg),
                          _stream(stream))
        return out, hid, top2, lg

    def draft_sample(self, hidden: torch.Tensor, last_tokens: torch.Tensor, cache: MtpCache,
                     K: int, temperature: float, seeds: torch.Tensor, offset: int,
                     out: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                     stream=None):
        """K draft steps sampling at `temperature`; seeds [B] int64 on the device.
        Returns (draft tokens [B, K] int32, draft logits [B, K, V] fp32)."""
        B = self._check_draft_in(hidden, last_tokens, cache, K)
        self._t("seeds", seeds, torch.int64, (B,))
        dev = hidden.device
        if out is None:
            out = torch.empty((B, K), dtype=torch.int32, device=dev)
        self._t("out", out, torch.int32, (B, K))
        lg = logits
        if lg is None:
            lg = torch.empty((B, K, self.vocab), dtype=torch.float32, device=dev)
        self._t("logits", lg, torch.float32, (B, K, self.vocab))
        L.mtp_draft_sample(self.handle, hidden.data_ptr(), last_tokens.data_ptr(), cache.kv, B, K,
                           float(temperature), seeds.data_ptr(), int(offset), out.data_ptr(),
                           lg.data_ptr(), _stream(stream))
        return out, lg

    def verify_sample(self, target_logits: torch.Tensor, draft_logits: torch.Tensor | None,
                      draft_tokens: torch.Tensor | None, temperature: float, seeds: torch.Tensor,
                      offset: int, accepted: torch.Tensor | None = None,
                      next_token: torch.Tensor | None = None, stream=None):
        """Speculative-sampling verification against target logits [B, K+1, V]."""
        B, K = self._check_logits(target_logits)
        if K > 0:
            self._t("draft_logits", draft_logits, torch.float32, (B, K, self.vocab))
        self._check_drafts(draft_tokens, B, K, required=True)
        self._t("seeds", seeds, torch.int64, (B,))
        self._check_outs(B, accepted, next_token)
        K1 = K + 1
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
        B, K = self._check_logits(target_logits)
        self._check_drafts(draft_tokens, B, K, required=True)
        self._check_outs(B, accepted, next_token)
        K1 = K + 1
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
        B, K = self._check_target_hidden(target_hidden)
        self._t("target_norm", target_norm, self.dtype, (self.cfg.hidden,))
        self._check_drafts(draft_tokens, B, K, required=True)
        self._check_outs(B, accepted, next_token)
        K1 = K + 1
        dev = target_hidden.device
        if accepted is None:
            accepted = torch.empty(B, dtype=torch.int32, device=dev)
        if next_token is None:
            next_token = torch.empty(B, dtype=torch.int32, device=dev)
        th = target_hidden
        L.mtp_verify_hidden(self.handle, th.data_ptr(), target_norm.data_ptr(),
                            _ptr(draft_tokens), B, K1 - 1, accepted.data_ptr(),
                            next_token.data_ptr(), _stream(stream))
        return accepted, next_token

    def catchup(self, cache: MtpCache, target_hidden: torch.Tensor, draft_tokens: torch.Tensor,
                accepted: torch.Tensor, stream=None) -> None:
        """Exact cache commit after verification (instead of rollback): rewrites the
        committed slots from the target's hidden states [B, K+1, H]."""
        B, K = self._check_target_hidden(target_hidden)
        if K < 1:
            raise ValueError("catch-up needs K >= 1 (target_hidden with at least 2 rows)")
        self._check_cache(cache, B)
        self._check_drafts(draft_tokens, B, K, required=True)
        self._t("accepted", accepted, torch.int32, (B,))
        K1 = K + 1
        th = target_hidden
        L.mtp_kv_catchup(self.handle, cache.kv, th.data_ptr(), draft_tokens.data_ptr(),
                         accepted.data_ptr(), B, K1 - 1, _stream(stream))

    def draft_seqk(self, hidden: torch.Tensor, last_tokens: torch.Tensor, cache: MtpCache,
                   k_seq: torch.Tensor, K_max: int, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
        """Draft with k_seq[b] (int32 [B] on the device, 0..K_max) steps for sequence b;
        returns [B, K_max] int32 (entries past k_seq[b] are unspecified)."""
        B = self._check_draft_in(hidden, last_tokens, cache, K_max)
        self._t("k_seq", k_seq, torch.int32, (B,))
        if out is None:
            out = torch.empty((B, K_max), dtype=torch.int32, device=hidden.device)
        self._t("out", out, torch.int32, (B, K_max))
        L.mtp_draft_seqk(self.handle, hidden.data_ptr(), last_tokens.data_ptr(), cache.kv,
                         k_seq.data_ptr(), B, K_max, out.data_ptr(), _stream(stream))
        return out

    def verify_seqk(self, target_logits: torch.Tensor, draft_tokens: torch.Tensor | None,
                    k_seq: torch.Tensor, accepted: torch.Tensor | None = None,
                    next_token: torch.Tensor | None = None, stream=None):
        """Greedy verification of k_seq[b] drafts per sequence against target_logits
        [B, K_max+1, V] (rows past k_seq[b] are not read)."""
        B, K = self._check_logits(target_logits)
        self._check_drafts(draft_tokens, B, K, required=True)
        self._t("k_seq", k_seq, torch.int32, (B,))
        self._check_outs(B, accepted, next_token)
        dev = target_logits.device
        if accepted is None:
            accepted = torch.empty(B, dtype=torch.int32, device=dev)
        if next_token is None:
            next_token = torch.empty(B, dtype=torch.int32, device=dev)
        L.mtp_verify_seqk(self.handle, target_logits.data_ptr(), _ptr(draft_tokens),
                          k_seq.data_ptr(), B, K, accepted.data_ptr(), next_token.data_ptr(),
                          _stream(stream))
        return accepted, next_token

    def rollback_seqk(self, cache: MtpCache, accepted: torch.Tensor, k_seq: torch.Tensor,
                      K_max: int, stream=None) -> None:
        if not isinstance(accepted, torch.Tensor) or accepted.dim() != 1:
            raise ValueError("accepted must be a [B] int32 tensor")
        B = accepted.shape[0]
        self._check_batch(B, K_max)
        self._t("accepted", accepted, torch.int32, (B,))
        self._t("k_seq", k_seq, torch.int32, (B,))
        self._check_cache(cache, B)
        L.mtp_kv_rollback_seqk(self.handle, cache.kv, accepted.data_ptr(), k_seq.data_ptr(), B,
                               K_max, _stream(stream))

    def prefill(self, cache: MtpCache, target_hidden: torch.Tensor, tokens: torch.Tensor,
                n_valid: torch.Tensor | None = None, stream=None) -> None:
        """Fill the cache over a prompt: row s of target_hidden [B, n, H] (the target's
        pre-norm hidden state at position pos+s) with tokens [B, n] int32 (the token after
        that position) goes to slot len+s; len / pos advance by n (or n_valid [B])."""
        if not isinstance(target_hidden, torch.Tensor) or target_hidden.dim() != 3:
            raise ValueError("target_hidden must be a [B, n, hidden] tensor")
        B, n = target_hidden.shape[0], target_hidden.shape[1]
        if not 1 <= B <= self.max_batch:
            raise ValueError(f"batch {B} outside 1..{self.max_batch}")
        self._t("target_hidden", target_hidden, self.dtype, (B, n, self.cfg.hidden))
        self._t("tokens", tokens, torch.int32, (B, n))
        if n_valid is not None:
            self._t("n_valid", n_valid, torch.int32, (B,))
        self._check_cache(cache, B)
        L.mtp_kv_prefill(self.handle, cache.kv, target_hidden.data_ptr(), tokens.data_ptr(),
                         _ptr(n_valid), B, n, _stream(stream))

    def rollback(self, cache: MtpCache, accepted: torch.Tensor, K: int, stream=None) -> None:
        if not isinstance(accepted, torch.Tensor) or accepted.dim() != 1:
            raise ValueError("accepted must be a [B] int32 tensor")
        B = accepted.shape[0]
        self._check_batch(B, K)
        self._t("accepted", accepted, torch.int32, (B,))
        self._check_cache(cache, B)
        L.mtp_kv_rollback(self.handle, cache.kv, accepted.data_ptr(), accepted.shape[0], K,
                          _stream(stream))

    def set_profiling(self, mask: int) -> None:
        L.mtp_set_profiling(self.handle, mask)

    def get_profile(self) -> dict:
        return L.mtp_get_profile(self.handle)

    def get_error(self, stream=None) -> int:
        return L.mtp_get_error(self.handle, _stream(stream))

    def refresh_weights(self, stream=None) -> None:
        """Rebuild the re-laid-out weight copy after the weight tensors changed in place
        (nothing to do for a handle created with packed_copy=False)."""
        L.mtp_refresh_weights(self.handle, _stream(stream))

    def info(self) -> dict:
        """Workspace and packed-copy bytes and the row grouping of this handle."""
        return L.mtp_get_info(self.handle)
