"""A small synthetic verifier for end-to-end checks of speculative decoding.

TEST INFRASTRUCTURE ONLY (same rules as ``mtp_oracle``).

The target is a random causal decoder stack of the MTP head's shape that shares
the head's token embedding and lm_head (devnotes, "How OpenVINO MTP Speculative
Decoding Works Internally", "Shared embeddings reduce duplication"). Every call
recomputes the whole prefix from scratch, so the logits for a given prefix are
bit-identical however the prefix was reached; plain greedy decoding and greedy
speculative decoding therefore must emit the same tokens (same page,
"Correctness before performance").

Its hidden state is the last decoder layer's output before the final norm, the
residual-stream tensor that the MTP head consumes (same page, "hidden_states").
"""
from __future__ import annotations

import numpy as np

from .mtp_oracle import (argmax_lowest, as_float, rmsnorm, rope, rope_tables, silu)


class TinyTarget:
    def __init__(self, cfg, tw: dict, embed: np.ndarray, lm_head: np.ndarray, dt=np.float32):
        self.cfg, self.dt = cfg, dt
        st = cfg.dtype
        self.layers = [{k: as_float(v, st, dt) for k, v in lw.items()} for lw in tw["layers"]]
        self.g_final = as_float(tw["g_final"], st, dt)
        self.embed = as_float(embed, st, dt)
        self.lm_head = as_float(lm_head, st, dt)

    def forward(self, tokens) -> tuple[np.ndarray, np.ndarray]:
        """tokens [n] -> (hidden [n, H] before the final norm, logits [n, V])."""
        cfg, dt = self.cfg, self.dt
        nq, nkv, d = cfg.n_q, cfg.n_kv, cfg.head_dim
        grp = nq // nkv
        t = np.asarray(tokens, np.int64)
        n = t.shape[0]
        x = self.embed[t]
        tabs = [rope_tables(p, d, cfg.rope_theta, dt) for p in range(n)]
        scale = dt(1.0 / np.sqrt(d))
        for lw in self.layers:
            a = rmsnorm(x, lw["g_attn"], cfg.rms_eps)
            q = (a @ lw["w_q"].T).reshape(n, nq, d)
            k = (a @ lw["w_k"].T).reshape(n, nkv, d)
            v = (a @ lw["w_v"].T).reshape(n, nkv, d)
            for p in range(n):
                q[p] = rope(q[p], *tabs[p])
                k[p] = rope(k[p], *tabs[p])
            o = np.empty((n, nq, d), dt)
            for h in range(nq):
                kk, vv = k[:, h // grp, :], v[:, h // grp, :]
                for p in range(n):
                    s = (kk[:p + 1] @ q[p, h]) * scale
                    s = s - s.max()
                    w = np.exp(s)
                    o[p, h] = (w / w.sum()) @ vv[:p + 1]
            x = x + o.reshape(n, nq * d) @ lw["w_o"].T
            m = rmsnorm(x, lw["g_mlp"], cfg.rms_eps)
            x = x + (silu(m @ lw["w_gate"].T) * (m @ lw["w_up"].T)) @ lw["w_down"].T
        logits = rmsnorm(x, self.g_final, cfg.rms_eps) @ self.lm_head.T
        return x, logits

    def next_token(self, tokens) -> int:
        return int(argmax_lowest(self.forward(tokens)[1][-1]))

    def greedy(self, prompt, n_new: int) -> list[int]:
        """Plain greedy decoding: one full forward per emitted token."""
        seq = [int(x) for x in prompt]
        for _ in range(n_new):
            seq.append(self.next_token(seq))
        return seq[len(prompt):]


def speculative_greedy(target: TinyTarget, prompt, n_new: int, draft_fn, verify_fn,
                       rollback_fn, K: int, from_hidden: bool = False, next_k=None):
    """Greedy speculative decoding driven by a draft head.

    draft_fn(hidden [H], last_token, K, committed) -> K draft tokens (the head keeps
    its cache and advances it by K; committed is the sequence so far);
    verify_fn(target_rows [K+1, X], drafts) -> (a, next); rollback_fn(a) cuts the
    head's cache back.  Target rows are taken at the last position of full forwards
    over the committed prefix extended by j drafts: its logits (X = V), or with
    from_hidden its hidden states before the final norm (X = H), which verify_fn turns
    into tokens through the target's final norm and the shared lm_head.
    With next_k, the speculative length of the next iteration is next_k(a, K) (K is
    the first iteration's length).
    Returns (emitted tokens, list of accepted lengths).
    """
    seq = [int(x) for x in prompt]
    hid, lg = target.forward(seq)
    seq.append(int(argmax_lowest(lg[-1])))
    h = hid[-1]
    accepted = []
    while len(seq) - len(prompt) < n_new:
        d = [int(x) for x in draft_fn(h, seq[-1], K, list(seq))]
        rows, hids = [], []
        for j in range(K + 1):
            hj, lj = target.forward(seq + d[:j])
            rows.append(lj[-1])
            hids.append(hj[-1])
        a, nxt = verify_fn(np.stack(hids if from_hidden else rows), d)
        a, nxt = int(a), int(nxt)
        rollback_fn(a)
        accepted.append(a)
        seq += d[:a] + [nxt]
        h = hids[a]
        if next_k is not None:
            K = int(next_k(a, K))
    return seq[len(prompt):len(prompt) + n_new], accepted


def lockstep_seqk(target: TinyTarget, prompts, n_new: int, k0: int, window: int, k_min: int,
                  k_max: int, draft_fn, verify_fn, rollback_fn, adapt_fn):
    """Greedy speculative decoding of several sequences in lock step, each with its own
    speculative length (OpenVINO GenAI "Speculative Decoding", Backend Differences).

    draft_fn(hidden [B, H], last [B], k [B], k_max) -> drafts [B, k_max] (entries past k[b]
    unused); verify_fn(target rows [B, k_max+1, V], drafts, k) -> (accepted [B], next [B]);
    rollback_fn(accepted, k). adapt_fn(accepted history [W, B], length history [W, B],
    k_min, k_max) -> next lengths [B], over the last `window` iterations. Target rows of
    sequence b are full forwards over its committed prefix extended by j drafts (rows past
    k[b] are zero). Returns the first n_new emitted tokens per sequence and the length
    history [iterations, B].
    """
    B = len(prompts)
    seqs = [[int(x) for x in p] for p in prompts]
    hid = []
    for b in range(B):
        h, lg = target.forward(seqs[b])
        seqs[b].append(int(argmax_lowest(lg[-1])))
        hid.append(h[-1])
    k = np.full(B, k0, np.int64)
    a_hist, k_hist = [], []
    while min(len(s) - len(p) for s, p in zip(seqs, prompts)) < n_new:
        d = np.asarray(draft_fn(np.stack(hid), np.array([s[-1] for s in seqs]), k, k_max))
        rows = np.zeros((B, k_max + 1, target.cfg.vocab), np.float32)
        hrows = []
        for b in range(B):
            hb = []
            for j in range(int(k[b]) + 1):
                hj, lj = target.forward(seqs[b] + [int(x) for x in d[b, :j]])
                rows[b, j] = lj[-1]
                hb.append(hj[-1])
            hrows.append(hb)
        a, nxt = verify_fn(rows, d, k)
        a, nxt = np.asarray(a, np.int64), np.asarray(nxt, np.int64)
        rollback_fn(a, k)
        for b in range(B):
            seqs[b] += [int(x) for x in d[b, :a[b]]] + [int(nxt[b])]
            hid[b] = hrows[b][int(a[b])]
        a_hist.append(a)
        k_hist.append(k.copy())
        k = np.asarray(adapt_fn(np.array(a_hist[-window:]), np.array(k_hist[-window:]), k_min,
                                k_max), np.int64)
    return [s[len(p):len(p) + n_new] for s, p in zip(seqs, prompts)], np.array(k_hist)


def softmax_rows(logits: np.ndarray, T: float) -> np.ndarray:
    x = np.asarray(logits, np.float64) / T
    x = np.exp(x - x.max(axis=-1, keepdims=True))
    return x / x.sum(axis=-1, keepdims=True)


def speculative_sample_batch(target: TinyTarget, prompt, n_new: int, first_tokens, draft_fn,
                             verify_fn, commit_fn, K: int):
    """B independent sampled generations from one prompt, advanced in lock step.

    first_tokens [B]: the token after the prompt, sampled by the caller from the target.
    Each iteration i: draft_fn(hidden [B, H], last [B], K, i) -> (drafts [B, K],
    draft_logits [B, K, V]); verify_fn(target_logits [B, K+1, V], drafts, draft_logits, i)
    -> (accepted_len [B], next_token [B]); commit_fn(accepted_len) cuts the head's cache.
    Target rows come from full forwards over each committed prefix extended by j drafts
    (memoised by prefix). Returns the first n_new emitted tokens per sequence [B, n_new]
    and the accepted lengths [iterations, B].
    """
    memo = {}

    def fwd(seq):
        key = tuple(seq)
        if key not in memo:
            h, lg = target.forward(list(seq))
            memo[key] = (h[-1], lg[-1])
        return memo[key]

    B = len(first_tokens)
    seqs = [[int(x) for x in prompt] + [int(first_tokens[b])] for b in range(B)]
    accepted = []
    it = 0
    while min(len(s) for s in seqs) - len(prompt) < n_new:
        last = np.array([s[-1] for s in seqs])
        # the head consumes the hidden state that produced the last committed token
        hid = np.stack([fwd(s[:-1])[0] for s in seqs])
        d, dl = draft_fn(hid, last, K, it)
        d = np.asarray(d, np.int64)
        rows = np.stack([[fwd(seqs[b] + [int(x) for x in d[b, :j]])[1] for j in range(K + 1)]
                         for b in range(B)])
        a, nxt = verify_fn(rows, d, dl, it)
        a, nxt = np.asarray(a, np.int64), np.asarray(nxt, np.int64)
        commit_fn(a)
        accepted.append(a)
        for b in range(B):
            seqs[b] += [int(x) for x in d[b, :a[b]]] + [int(nxt[b])]
        it += 1
    out = np.array([s[len(prompt):len(prompt) + n_new] for s in seqs])
    return out, np.array(accepted)
