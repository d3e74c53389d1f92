"""Oracle for temperature (sampling) speculative decoding with the MTP head.

TEST INFRASTRUCTURE ONLY. Same rules as ``mtp_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may use it;
it shares no code with the HIP path. Arithmetic is float64 (NumPy).

What the pages fix:
  [OVSD] OpenVINO GenAI docs, "Speculative Decoding", Overview: the target validates the
    drafts with the standard scheme, which leaves the output statistically the same as
    sampling from the target alone; at the first divergent position the target's own
    sample replaces the draft.
  [FI] forceinjection, "MTP 深度解析", section 4.3: acceptance is lower at temperature
    1.0 (50-70%) than under greedy decoding.

Readings where the pages are silent (the plainest ones the rest supports):
  * The standard scheme is speculative sampling (Leviathan, Kalman and Matias, ICML 2023;
    Chen et al. 2023). With p_j = softmax(t_j / T) the target's distribution at verified
    input j and q_j = softmax(z_j / T) the draft distribution that produced d_{j+1},
    draft d_{j+1} is accepted with probability min(1, p_j(d_{j+1}) / q_j(d_{j+1})). At the
    first rejection (row j) the next token is drawn from max(0, p_j - q_j) renormalised;
    after K acceptances the bonus token is drawn from p_K.
  * The draft samples d_{j+1} from q_j; draft and target use the same temperature T > 0;
    no top-k / top-p truncation.
  * A categorical distribution w is sampled by the Gumbel-max rule:
    argmax_v (log w_v + G_v) with G_v = -log(-log U_v), U_v uniform on (0, 1); equal keys
    go to the lowest index. Normalising constants drop out of the argmax.
  * The acceptance test is log U < log p_j(d) - log q_j(d) (U < p/q, strictly).
  * If rounding leaves no v with p_j(v) > q_j(v) after a rejection, the token is drawn
    from p_j with the same noise.

Random numbers are counter based, so every element is drawn independently of the
launch shape: Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
As Easy as 1, 2, 3", SC'11), key (seed_b, 0), counter (c0, row, purpose, offset); the
vocabulary entry v uses word v & 3 of block c0 = v >> 2. A 64-bit word w becomes
U = ((w >> 40) | 1) / 2^24, an odd multiple of 2^-24 (exact in float32).
Purposes: 0 = the draft's noise at step j (row j), 1 = the acceptance uniform of
d_{j+1} (c0 = 0, row j, word 0), 2 = the noise of the resampled or bonus token
(row = the accepted length a).
"""
from __future__ import annotations

import numpy as np

_MASK = (1 << 64) - 1
# Philox4x64 multipliers and Weyl key increments (the paper's Philox-4x64 constants).
_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

PURPOSE_DRAFT, PURPOSE_ACCEPT, PURPOSE_RESAMPLE = 0, 1, 2


def _mulhilo(a: np.ndarray, m: np.uint64):
    """High and low 64-bit halves of the 128-bit product a * m (a uint64 array)."""
    a0, a1 = a & _LO, a >> _S32
    m0, m1 = m & _LO, m >> _S32
    p00, p01, p10, p11 = a0 * m0, a0 * m1, a1 * m0, a1 * m1
    mid = (p00 >> _S32) + (p01 & _LO) + (p10 & _LO)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    return hi, a * m


def philox4x64_10(c0, c1, c2, c3, k0, k1=0):
    """One Philox4x64 block per element (10 rounds). Arguments broadcast; returns four
    uint64 arrays (the output words 0..3)."""
    arrs = np.broadcast_arrays(*[np.atleast_1d(np.asarray(v, dtype=np.uint64))
                                 for v in (c0, c1, c2, c3, k0, k1)])
    x0, x1, x2, x3, ka, kb = (a.copy() for a in arrs)
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                ka = ka + _W0
                kb = kb + _W1
            hi0, lo0 = _mulhilo(x0, _M0)
            hi1, lo1 = _mulhilo(x2, _M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ ka, lo1, hi0 ^ x3 ^ kb, lo0
    return x0, x1, x2, x3


def to_uniform(w: np.ndarray) -> np.ndarray:
    """64-bit word -> odd multiple of 2^-24 in (0, 1)."""
    return ((np.asarray(w, np.uint64) >> np.uint64(40)) | np.uint64(1)).astype(np.float64) \
        * 2.0 ** -24


def gumbel(u: np.ndarray) -> np.ndarray:
    return -np.log(-np.log(u))


def vocab_uniforms(seeds, offset: int, purpose: int, rows, V: int) -> np.ndarray:
    """U [B, V] for every vocabulary entry; rows is a scalar or [B]."""
    seeds = np.asarray(seeds, np.uint64).reshape(-1, 1)
    rows = np.broadcast_to(np.asarray(rows, np.uint64).reshape(-1, 1), seeds.shape)
    nblk = (V + 3) // 4
    blk = np.arange(nblk, dtype=np.uint64).reshape(1, -1)
    words = philox4x64_10(blk, rows, purpose, offset, seeds, 0)
    w = np.stack(words, axis=-1).reshape(seeds.shape[0], 4 * nblk)[:, :V]
    return to_uniform(w)


def accept_uniforms(seeds, offset: int, K: int) -> np.ndarray:
    """U [B, K]: the acceptance uniform of draft d_{j+1} in column j."""
    seeds = np.asarray(seeds, np.uint64).reshape(-1, 1)
    j = np.arange(K, dtype=np.uint64).reshape(1, -1)
    w0 = philox4x64_10(0, j, PURPOSE_ACCEPT, offset, seeds, 0)[0]
    return to_uniform(w0)


def _argmax_gap(keys: np.ndarray):
    """Row-wise argmax (lowest index on ties) and the gap between the two largest keys."""
    idx = np.argmax(keys, axis=-1)
    if keys.shape[-1] < 2:
        return idx, np.full(idx.shape, np.inf)
    top2 = np.partition(keys, keys.shape[-1] - 2, axis=-1)[..., -2:]
    return idx, top2[..., 1] - top2[..., 0]


def sample_tokens(logits: np.ndarray, T: float, seeds, offset: int, step: int):
    """The draft's token at step `step` for every sequence: Gumbel-max over z / T.

    logits [B, V] -> (tokens [B], gap [B] between the two largest perturbed keys)."""
    z = np.asarray(logits, np.float64)
    g = gumbel(vocab_uniforms(seeds, offset, PURPOSE_DRAFT, step, z.shape[-1]))
    return _argmax_gap(z / T + g)


def logsumexp(x: np.ndarray) -> np.ndarray:
    m = x.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True)))[..., 0]


def verify_sample(target_logits: np.ndarray, draft_logits: np.ndarray,
                  draft_tokens: np.ndarray, T: float, seeds, offset: int) -> dict:
    """Speculative-sampling verification of K drafts per sequence.

    target_logits [B, K+1, V]; draft_logits [B, K, V] (row j produced d_{j+1});
    draft_tokens [B, K]. Returns accepted_len [B] (0..K), next_token [B], and for
    near-tie aware comparisons: margin [B, K] = log p - log q - log U of each acceptance
    test (accept iff > 0), gap [B] between the two largest keys of the final draw, and
    residual [B] (True when the final draw used max(0, p - q))."""
    t = np.asarray(target_logits, np.float64) / T
    B, K1, V = t.shape
    K = K1 - 1
    d = np.asarray(draft_tokens, np.int64).reshape(B, K)
    bi = np.arange(B)
    lse_t = logsumexp(t)                                     # [B, K+1]
    if K:
        z = np.asarray(draft_logits, np.float64).reshape(B, K, V) / T
        lse_z = logsumexp(z)                                 # [B, K]
        jj = np.arange(K)
        log_p = t[bi[:, None], jj[None, :], d] - lse_t[:, :K]
        log_q = z[bi[:, None], jj[None, :], d] - lse_z
        margin = log_p - log_q - np.log(accept_uniforms(seeds, offset, K))
        rejected = margin <= 0
        acc = np.where(rejected.any(axis=1), rejected.argmax(axis=1), K)
    else:
        margin = np.zeros((B, 0))
        acc = np.zeros(B, np.int64)
    g = gumbel(vocab_uniforms(seeds, offset, PURPOSE_RESAMPLE, acc, V))
    keys = np.empty((B, V))
    residual = np.zeros(B, bool)
    for b in range(B):
        a = int(acc[b])
        if a < K:
            r = np.exp(t[b, a] - lse_t[b, a]) - np.exp(z[b, a] - lse_z[b, a])
            if np.any(r > 0):
                with np.errstate(divide="ignore"):
                    keys[b] = np.where(r > 0, np.log(np.where(r > 0, r, 1.0)) + g[b], -np.inf)
                residual[b] = True
                continue
        keys[b] = t[b, a] + g[b]
    nxt, gap = _argmax_gap(keys)
    return {"accepted_len": acc.astype(np.int64), "next_token": nxt.astype(np.int64),
            "margin": margin, "gap": gap, "residual": residual}
