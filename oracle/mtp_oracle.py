"""Oracle for the MTP draft step, greedy verification and MTP-cache rollback.

TEST INFRASTRUCTURE ONLY. This is a plain, slow CPU implementation written from
the pages. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it; the product library never does, and it
shares no code with the HIP path (inputs come from ``mtp_synth`` only).

Arithmetic is NumPy in float64 by default (``dt=np.float32`` re-runs the same
steps in single precision). Where a floating-point value decides an integer (the
argmax that picks a draft or target token), the decision is taken on the logits
rounded to float32, the precision the kernels decide in; ties go to the lowest index
on both sides. Matrices are row-major ``[out, in]``, ``y = W @ x``.

Sources (page title, then section):
  [SPEC]  speculators user guide, "MTP (Multi-Token Prediction)",
          How It Works > Architecture; Step Weight Formula.
  [OVMTP] devnotes, "How OpenVINO MTP Speculative Decoding Works Internally",
          sections "The MTP inputs", "KV cache", "Stateful execution",
          "Shared embeddings reduce duplication", "Correctness before performance".
  [OVSD]  OpenVINO GenAI docs, "Speculative Decoding", Overview and
          "Measuring Effectiveness".
  [FI]    forceinjection, "MTP 深度解析", sections 4.2 (self-speculation) and
          4.4 (chaining on the predicted token).

Readings where the pages are silent (each is the plainest one the rest supports):
  concat order: [RMSNorm(h); RMSNorm(e)], hidden first, as [SPEC] lists them.
  recursion: the hidden state fed to step k+1 is the decoder-layer output before
    the final norm; the final norm only feeds the lm_head.
  token input: step 1 takes last_tokens, step k>1 the token drafted at step k-1.
  positions: step k uses RoPE position pos+k-1 and writes cache slot len+k-1.
  decoder layer: pre-norm residual blocks, no biases, no QK-norm, scale 1/sqrt(d),
    causal over all cached slots including the new one, SwiGLU with silu(x)=x*sigmoid(x).
  RMSNorm: x * (mean(x^2) + eps)^(-1/2) * g, eps from the config.
  RoPE: rotate-half pairs (i, i+d/2), inv_freq_i = theta^(-2i/d); cos/sin are
    evaluated in float64 from the integer position and rounded to float32.
  argmax ties: the lowest vocabulary index wins.
  new K/V entries are rounded to the cache dtype when they are written, and
    attention reads them back from the cache.
  verify: row j of the target logits scores the token after input j of
    [last_token, d_1 .. d_K]; accepted_len counts accepted drafts (0..K);
    next_token is the target's argmax at the first mismatch (row K if all match).
  rollback: slot k (from the pair (h^(k-1), tok_{k-1})) is kept iff tok_{k-1}
    was committed, so len advances by min(a+1, K) and pos by a+1.
  prefill: the slot of prompt position s holds the pair (verifier hidden state at s,
    token s+1), the same pair a one-step draft at s would process; after a prompt of
    P tokens the cache holds P-1 slots and the first draft takes (h_{P-1}, x_P).
"""
from __future__ import annotations

import numpy as np

from .sampling import sample_tokens


# ----------------------------------------------------------------------------- dtypes

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact): the 16 bits become the high half.

    Large tables are converted in slices on a few threads (the result is the same)."""
    b = np.ascontiguousarray(bits, np.uint16)
    out = np.empty(b.shape, np.uint32)
    fb, fo = b.reshape(-1), out.reshape(-1)
    step = 1 << 22

    def part(i):
        np.left_shift(fb[i:i + step], 16, out=fo[i:i + step], dtype=np.uint32)

    if fb.size <= step:
        part(0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(16) as ex:
            list(ex.map(part, range(0, fb.size, step)))
    return out.view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even) and return it widened to float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def as_float(a: np.ndarray, storage: str, dt=np.float32) -> np.ndarray:
    """Storage array (float32, or bf16 bits when storage == 'bf16') -> dt."""
    if storage == "bf16":
        return widen_bf16(a).astype(dt, copy=False)
    return np.asarray(a, dtype=np.float32).astype(dt, copy=False)


# ----------------------------------------------------------------------------- building blocks

def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x * (mean(x^2) + eps)^(-1/2) * g.  [SPEC] Architecture:
    the hidden state and the token embedding are each normalized separately."""
    dt = x.dtype
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + dt.type(eps))) * g


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x)."""
    one = x.dtype.type(1)
    return x / (one + np.exp(-x))


def rope_tables(position: int, head_dim: int, theta: float, dt=np.float32):
    """cos/sin of position * theta^(-2i/d), i < d/2, in float64, rounded to dt."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    ang = float(position) * inv_freq
    return np.cos(ang).astype(dt), np.sin(ang).astype(dt)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE on the last axis: (x1, x2) -> (x1*c - x2*s, x2*c + x1*s)."""
    h = x.shape[-1] // 2
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


def gqa_attention(q: np.ndarray, kc: np.ndarray, vc: np.ndarray) -> np.ndarray:
    """One query per head over T cached slots.

    q [n_q, d]; kc, vc [n_kv, T, d]; query head h reads kv head h // (n_q / n_kv).
    softmax(q.K^T / sqrt(d)) V per head.  -> [n_q, d]
    """
    n_q, d = q.shape
    n_kv = kc.shape[0]
    grp = n_q // n_kv
    dt = q.dtype
    out = np.empty_like(q)
    scale = dt.type(1.0 / np.sqrt(d))
    for h in range(n_q):
        kk = kc[h // grp]
        vv = vc[h // grp]
        s = (kk @ q[h]) * scale
        s = s - s.max()
        p = np.exp(s)
        p = p / p.sum()
        out[h] = p @ vv
    return out


def argmax_lowest(x: np.ndarray) -> np.ndarray:
    """argmax over the last axis; the lowest index wins ties (numpy's rule)."""
    return np.argmax(x, axis=-1)


# ----------------------------------------------------------------------------- weights

class OracleWeights:
    """The MTP head's weights widened to the oracle's arithmetic dtype once.

    The embedding table stays in storage dtype; only gathered rows are widened.
    """

    def __init__(self, cfg, weights: dict, dt=np.float64):
        self.cfg, self.dt = cfg, dt
        self.storage = cfg.dtype
        self.embed_store = weights["embed"]
        self.w = {k: as_float(v, cfg.dtype, dt) for k, v in weights.items() if k != "embed"}

    def embed_rows(self, tokens: np.ndarray) -> np.ndarray:
        return as_float(self.embed_store[np.asarray(tokens, np.int64)], self.storage, self.dt)


# ----------------------------------------------------------------------------- the draft step

def draft(cfg, W: OracleWeights, hidden: np.ndarray, last_tokens: np.ndarray,
          k_cache: np.ndarray, v_cache: np.ndarray, lens: np.ndarray, pos: np.ndarray,
          K: int, force_tokens: np.ndarray | None = None, sample: dict | None = None) -> dict:
    """K recursive MTP draft steps for every sequence.  [SPEC] Architecture; [FI] 4.4.

    hidden [B, H] (storage dtype); last_tokens [B]; k_cache/v_cache [B, n_kv, S, d]
    (storage dtype, updated in place with slots len..len+K-1); lens/pos [B] (returned
    advanced by K). force_tokens [B, K]: step k+1 consumes force_tokens[:, k] instead
    of the oracle's own draft (teacher forcing). sample = {"T", "seeds", "offset"}: each
    token is sampled from softmax(logits / T) by ``sampling.sample_tokens`` (row k for
    step k+1) instead of taken by argmax ([OVSD] Overview, temperature > 0).

    Returns draft_tokens [B, K], hidden_steps [K, B, H] (h^(k)), logits [K, B, V],
    top1 / margin [K, B] (largest logit, and its gap to the second largest; when
    sampling, the gap between the two largest perturbed keys), lens, pos.
    """
    dt = W.dt
    w = W.w
    B, H, V = hidden.shape[0], cfg.hidden, cfg.vocab
    nq, nkv, d = cfg.n_q, cfg.n_kv, cfg.head_dim
    eps = cfg.rms_eps
    bf16_cache = cfg.dtype == "bf16"
    lens = np.asarray(lens, np.int64).copy()
    pos = np.asarray(pos, np.int64).copy()
    h = as_float(hidden, cfg.dtype, dt)
    tok = np.asarray(last_tokens, np.int64).copy()
    drafts = np.zeros((B, K), np.int64)
    hsteps = np.zeros((K, B, H), dt)
    logits_all = np.zeros((K, B, V), dt)
    top1 = np.zeros((K, B), dt)
    margin = np.zeros((K, B), dt)
    for k in range(K):
        # Shared-embedding gather, separate RMSNorms, concat, 2H -> H projection.
        e = W.embed_rows(tok)
        hn = rmsnorm(h, w["g_h"], eps)
        en = rmsnorm(e, w["g_e"], eps)
        x = np.concatenate([hn, en], axis=1) @ w["w_eh"].T
        # Standard pre-norm decoder layer: attention block.
        a = rmsnorm(x, w["g_attn"], eps)
        q = (a @ w["w_q"].T).reshape(B, nq, d)
        kn = (a @ w["w_k"].T).reshape(B, nkv, d)
        vn = (a @ w["w_v"].T).reshape(B, nkv, d)
        o = np.zeros((B, nq, d), dt)
        for b in range(B):
            p = int(pos[b]) + k
            slot = int(lens[b]) + k
            cos, sin = rope_tables(p, d, cfg.rope_theta, dt)
            qb = rope(q[b], cos, sin)
            kb = rope(kn[b], cos, sin)
            vb = vn[b]
            if bf16_cache:
                k_cache[b, :, slot, :] = _store_bf16(kb)
                v_cache[b, :, slot, :] = _store_bf16(vb)
            else:
                k_cache[b, :, slot, :] = kb.astype(np.float32)
                v_cache[b, :, slot, :] = vb.astype(np.float32)
            kc = as_float(k_cache[b, :, :slot + 1, :], cfg.dtype, dt)
            vc = as_float(v_cache[b, :, :slot + 1, :], cfg.dtype, dt)
            o[b] = gqa_attention(qb, kc, vc)
        x1 = x + o.reshape(B, nq * d) @ w["w_o"].T
        # MLP block (SwiGLU).
        m = rmsnorm(x1, w["g_mlp"], eps)
        act = silu(m @ w["w_gate"].T) * (m @ w["w_up"].T)
        x2 = x1 + act @ w["w_down"].T
        # Final norm + shared lm_head + argmax.
        lg = rmsnorm(x2, w["g_final"], eps) @ w["lm_head"].T
        lg32 = lg.astype(np.float32)  # the token is decided in the kernels' precision
        dk = argmax_lowest(lg32)
        srt = np.partition(lg32, V - 2, axis=1)[:, V - 2:]
        top1[k] = srt[:, 1]
        margin[k] = srt[:, 1] - srt[:, 0]
        if sample is not None:
            dk, margin[k] = sample_tokens(lg, sample["T"], sample["seeds"], sample["offset"], k)
        drafts[:, k] = dk
        hsteps[k] = x2
        logits_all[k] = lg
        # Recursion: the next step consumes this step's hidden state and token.
        h = x2
        tok = dk if force_tokens is None else np.asarray(force_tokens, np.int64)[:, k]
    return {"draft_tokens": drafts, "hidden_steps": hsteps, "logits": logits_all,
            "top1": top1, "margin": margin, "lens": lens + K, "pos": pos + K}


def _store_bf16(x: np.ndarray) -> np.ndarray:
    """float -> bfloat16 bit patterns (round to nearest even)."""
    r = round_to_bf16(np.asarray(x, np.float32))
    return (r.view(np.uint32) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------- verify / rollback

def verify(target_logits: np.ndarray, draft_tokens: np.ndarray):
    """Greedy verification.  [OVSD] Overview; [FI] 4.2.

    target_logits [B, K+1, V]: row j scores the token after input j of
    [last_token, d_1 .. d_K].  The target's token at row j is its argmax (lowest
    index on ties).  Drafts are accepted while they equal the target's token;
    the first divergent position (or row K when all K match) supplies the bonus
    token.  Returns accepted_len [B] in 0..K and next_token [B].
    """
    t = np.asarray(target_logits)
    d = np.asarray(draft_tokens, np.int64).reshape(t.shape[0], -1)
    B, K = d.shape
    g = argmax_lowest(t)
    acc = np.zeros(B, np.int64)
    nxt = np.zeros(B, np.int64)
    for b in range(B):
        a = 0
        while a < K and d[b, a] == g[b, a]:
            a += 1
        acc[b] = a
        nxt[b] = g[b, a]
    return acc, nxt


def verify_from_hidden(cfg, target_hidden: np.ndarray, target_norm: np.ndarray,
                       lm_head: np.ndarray, draft_tokens: np.ndarray, dt=np.float64):
    """Greedy verification from the target's hidden states.  [OVSD] Overview;
    [SPEC] Architecture (the LM head is shared with the verifier).

    target_hidden [B, K+1, H] (storage dtype): the target's last-layer outputs before
    its final norm at the K+1 verified inputs [last_token, d_1 .. d_K]; target_norm [H]
    is the target's final-norm gain; lm_head [V, H] is the shared head. The target's
    logits are lm_head . RMSNorm(h; target_norm), and verification then proceeds as in
    ``verify``. Returns accepted_len [B], next_token [B], and the top-1 minus top-2
    margin [B, K+1] of each row (for near-tie aware comparisons).
    """
    st = cfg.dtype
    th = as_float(target_hidden, st, dt)
    g = as_float(target_norm, st, dt)
    w = as_float(lm_head, st, dt)
    # tokens are decided on the logits rounded to float32, the kernels' precision
    logits = (rmsnorm(th, g, cfg.rms_eps) @ w.T).astype(np.float32)
    V = logits.shape[-1]
    srt = np.partition(logits, V - 2, axis=-1)[..., V - 2:]
    acc, nxt = verify(logits, draft_tokens)
    return acc, nxt, srt[..., 1] - srt[..., 0]


def kv_rollback(lens: np.ndarray, pos: np.ndarray, accepted_len: np.ndarray, K: int):
    """Cut the MTP cache back to the committed prefix.  [OVMTP] Stateful execution;
    [OVSD] Overview (drafting resumes after the first divergent token).

    On entry lens/pos are the values after a K-step draft (advanced by K).
    Slot k = 1..K came from the pair (h^(k-1), tok_{k-1}); it stays iff tok_{k-1}
    was committed, i.e. k <= a + 1.  pos moves to the position of the last
    verified input, a + 1 past the draft's starting position.
    """
    a = np.asarray(accepted_len, np.int64)
    lens = np.asarray(lens, np.int64) - K + np.minimum(a + 1, K)
    pos = np.asarray(pos, np.int64) - K + a + 1
    return lens, pos


def kv_catchup(cfg, W: OracleWeights, target_hidden: np.ndarray, draft_tokens: np.ndarray,
               accepted_len: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
               lens: np.ndarray, pos: np.ndarray, K: int):
    """Commit the MTP cache exactly after verification.  [OVMTP] Stateful execution
    (the MTP cache holds the MTP layer's K/V of the committed positions, built from the
    verifier's hidden states); [SPEC] Architecture (the layer's input at a position is
    the projection of the normalised hidden state and next-token embedding).

    On entry lens/pos are the values after a K-step draft. Draft step k wrote slot
    lens-K+k-1 from (h^(k-1), tok_{k-1}); for k >= 2 that hidden state was the head's own,
    and with a = K the pair (h_{t+K}, d_K) was never processed. Here every committed
    pair j = 1..a, (target_hidden[b, j-1], d_j) at position pos-K+j, is run through the
    layer's input side (eh_proj, attention norm, K/V projections, RoPE) and written to
    slot lens-K+j in the cache dtype. target_hidden [B, K+1, H] (storage dtype) are the
    target's pre-norm hidden states at the verified inputs [last_token, d_1 .. d_K].
    Returns lens, pos advanced to the committed prefix: lens-K+a+1, pos-K+a+1.
    """
    dt = W.dt
    w = W.w
    nkv, d = cfg.n_kv, cfg.head_dim
    eps = cfg.rms_eps
    th = as_float(target_hidden, cfg.dtype, dt)
    dtok = np.asarray(draft_tokens, np.int64).reshape(th.shape[0], -1)
    acc = np.asarray(accepted_len, np.int64)
    lens = np.asarray(lens, np.int64)
    pos = np.asarray(pos, np.int64)
    for b in range(th.shape[0]):
        for j in range(1, int(acc[b]) + 1):
            h = th[b, j - 1][None]
            e = W.embed_rows(dtok[b, j - 1:j])
            x = np.concatenate([rmsnorm(h, w["g_h"], eps), rmsnorm(e, w["g_e"], eps)],
                               axis=1) @ w["w_eh"].T
            a = rmsnorm(x, w["g_attn"], eps)
            kn = (a @ w["w_k"].T).reshape(nkv, d)
            vn = (a @ w["w_v"].T).reshape(nkv, d)
            p = int(pos[b]) - K + j
            slot = int(lens[b]) - K + j
            cos, sin = rope_tables(p, d, cfg.rope_theta, dt)
            kb = rope(kn, cos, sin)
            if cfg.dtype == "bf16":
                k_cache[b, :, slot, :] = _store_bf16(kb)
                v_cache[b, :, slot, :] = _store_bf16(vn)
            else:
                k_cache[b, :, slot, :] = kb.astype(np.float32)
                v_cache[b, :, slot, :] = vn.astype(np.float32)
    return lens - K + acc + 1, pos - K + acc + 1


def kv_prefill(cfg, W: OracleWeights, target_hidden: np.ndarray, tokens: np.ndarray,
               k_cache: np.ndarray, v_cache: np.ndarray, lens: np.ndarray, pos: np.ndarray,
               n_valid: np.ndarray | None = None):
    """Fill the MTP cache over a prompt from the verifier's hidden states.  [OVMTP] KV cache
    and Stateful execution (the MTP layer keeps its own one-layer cache, filled for every
    position it has seen); [SPEC] Architecture (the layer's input at position s is the
    projection of the normalised verifier hidden state at s and the normalised embedding of
    the token that follows it).

    target_hidden [B, n, H] (storage dtype): the target's last-layer outputs before its
    final norm at n consecutive positions pos[b] .. pos[b]+n-1; tokens [B, n]: the token
    after each of those positions (row s pairs h_s with x_{s+1}). For every sequence b and
    s < n_valid[b] (default n), the pair runs through the layer's input side (embedding
    gather, separate RMSNorms, concat, eh_proj, attention norm, K/V projections, RoPE at
    position pos[b]+s) and is written to slot lens[b]+s in the cache dtype.
    Returns lens + n_valid, pos + n_valid.
    """
    dt = W.dt
    w = W.w
    nkv, d = cfg.n_kv, cfg.head_dim
    eps = cfg.rms_eps
    th = as_float(target_hidden, cfg.dtype, dt)
    B, n = th.shape[0], th.shape[1]
    tok = np.asarray(tokens, np.int64).reshape(B, n)
    nv = np.full(B, n, np.int64) if n_valid is None else np.asarray(n_valid, np.int64)
    lens = np.asarray(lens, np.int64)
    pos = np.asarray(pos, np.int64)
    for b in range(B):
        m = int(nv[b])
        if m == 0:
            continue
        # every row of the sequence at once: row s of each product is that row's projection
        e = W.embed_rows(tok[b, :m])
        x = np.concatenate([rmsnorm(th[b, :m], w["g_h"], eps), rmsnorm(e, w["g_e"], eps)],
                           axis=1) @ w["w_eh"].T
        a = rmsnorm(x, w["g_attn"], eps)
        kn = (a @ w["w_k"].T).reshape(m, nkv, d)
        vn = (a @ w["w_v"].T).reshape(m, nkv, d)
        for s in range(m):
            cos, sin = rope_tables(int(pos[b]) + s, d, cfg.rope_theta, dt)
            kb = rope(kn[s], cos, sin)
            slot = int(lens[b]) + s
            if cfg.dtype == "bf16":
                k_cache[b, :, slot, :] = _store_bf16(kb)
                v_cache[b, :, slot, :] = _store_bf16(vn[s])
            else:
                k_cache[b, :, slot, :] = kb.astype(np.float32)
                v_cache[b, :, slot, :] = vn[s].astype(np.float32)
    return lens + nv, pos + nv


def adapt_k(accepted_len, K: int, k_min: int, k_max: int) -> int:
    """Speculative length for the next iteration.  [OVSD] Backend Differences (the
    stateful backend adapts num_assistant_tokens per step from recent acceptance and
    backs off when it is low); [FI] 7.3 (depth adapted to the live acceptance rate).

    Reading: a sequence that accepted all K drafts asks for K + 1, one that accepted a < K
    asks for a + 1; the batch takes the largest request, clipped to [k_min, k_max].
    """
    a = np.asarray(accepted_len, np.int64).reshape(-1)
    want = np.where(a >= K, K + 1, a + 1)
    return int(min(max(int(want.max()), k_min), k_max))


def adapt_k_seq(accepted_hist, k_hist, k_min: int, k_max: int) -> np.ndarray:
    """Per-sequence speculative lengths for the next iteration from a window of recent
    iterations.  [OVSD] Backend Differences (the length follows recent acceptance and backs
    off when it is low); [FI] 7.3 (depth adapted to the live acceptance rate, per request).

    accepted_hist, k_hist [W, B]: the accepted length a and the length k each sequence used
    in each of its last W iterations (any order). Reading: iteration i of sequence b asks
    for k+1 when it accepted all k drafts and for a+1 otherwise (the batch-wide rule, per
    sequence); the sequence takes the mean of its W requests rounded up, clipped to
    [k_min, k_max]. With W = 1 this is the per-iteration rule applied to each sequence.
    Returns k_next [B].
    """
    a = np.asarray(accepted_hist, np.int64)
    k = np.asarray(k_hist, np.int64)
    a = a.reshape(-1, a.shape[-1]) if a.ndim > 1 else a.reshape(1, -1)
    k = k.reshape(a.shape)
    want = np.where(a >= k, k + 1, a + 1)
    W = want.shape[0]
    mean_up = -(-want.sum(axis=0) // W)
    return np.clip(mean_up, k_min, k_max)


def draft_seqk(cfg, W: OracleWeights, hidden, last_tokens, k_cache, v_cache, lens, pos,
               k_seq, K_max: int) -> dict:
    """Draft with a speculative length per sequence: sequence b runs k_seq[b] (0..K_max)
    recursive steps, exactly as ``draft`` with K = k_seq[b] on that sequence alone
    ([SPEC] Architecture; [OVSD] Backend Differences). Returns draft_tokens [B, K_max]
    (entries past k_seq[b] are -1, not drafted), lens / pos advanced by k_seq."""
    B = hidden.shape[0]
    ks = np.asarray(k_seq, np.int64)
    drafts = np.full((B, K_max), -1, np.int64)
    lens = np.asarray(lens, np.int64).copy()
    pos = np.asarray(pos, np.int64).copy()
    margin = np.full((K_max, B), np.inf)
    for b in range(B):
        kb = int(ks[b])
        if kb == 0:
            continue
        r = draft(cfg, W, hidden[b:b + 1], np.asarray(last_tokens)[b:b + 1], k_cache[b:b + 1],
                  v_cache[b:b + 1], lens[b:b + 1], pos[b:b + 1], kb)
        drafts[b, :kb] = r["draft_tokens"][0]
        margin[:kb, b] = r["margin"][:, 0]
        lens[b], pos[b] = r["lens"][0], r["pos"][0]
    return {"draft_tokens": drafts, "lens": lens, "pos": pos, "margin": margin}


def verify_seqk(target_logits, draft_tokens, k_seq):
    """Greedy verification with a length per sequence: sequence b checks its first
    k_seq[b] drafts against target rows 0..k_seq[b] ([OVSD] Overview), rows past that are
    not read. Returns accepted_len [B] (0..k_seq[b]) and next_token [B]."""
    t = np.asarray(target_logits)
    d = np.asarray(draft_tokens, np.int64)
    ks = np.asarray(k_seq, np.int64)
    B = t.shape[0]
    acc = np.zeros(B, np.int64)
    nxt = np.zeros(B, np.int64)
    for b in range(B):
        kb = int(ks[b])
        a, n = verify(t[b:b + 1, :kb + 1], d[b:b + 1, :kb])
        acc[b], nxt[b] = a[0], n[0]
    return acc, nxt


def kv_rollback_seqk(lens, pos, accepted_len, k_seq):
    """Rollback after a draft with a length per sequence: ``kv_rollback`` with K = k_seq[b]
    for each sequence ([OVMTP] Stateful execution)."""
    ks = np.asarray(k_seq, np.int64)
    a = np.asarray(accepted_len, np.int64)
    lens = np.asarray(lens, np.int64) - ks + np.minimum(a + 1, ks)
    pos = np.asarray(pos, np.int64) - ks + a + 1
    return lens, pos


def step_weights(beta: float, K: int) -> np.ndarray:
    """Normalised exponential-decay step weights alpha_k = beta^(k-1) / sum_j beta^(j-1).
    [SPEC] Step Weight Formula."""
    num = np.array([beta ** (k - 1) for k in range(1, K + 1)], np.float64)
    return num / num.sum()


def tokens_per_iteration(accepted_len: np.ndarray) -> np.ndarray:
    """Tokens emitted per target iteration: the accepted drafts plus the bonus token.
    [OVSD] Measuring Effectiveness."""
    return np.asarray(accepted_len, np.int64) + 1
