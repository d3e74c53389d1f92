"""Temperature sampling on the GPU: the draft's sampled tokens (Gumbel-max in the lm_head
kernels) and speculative-sampling verification, each against the oracle on the same
inputs; and the whole GPU loop's output distribution against a tiny target's exact
sequence probabilities."""
import numpy as np
import pytest
from scipy import stats

import mtp_synth as S
from gpu_util import MARGIN, TOL, make_head, small, to_dev
from oracle import mtp_oracle as O
from oracle import sampling as SP

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

# Below this margin fp32 (GPU) and fp64 (oracle) rounding may decide a sampling test.
GATE = 1e-3


def seeds_dev(seeds: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(seeds).view(np.int64)).cuda()


def verify_head(cfg):
    """A small head with the vocabulary and batch of cfg: verification reads no weights."""
    h = small(name="vsh", cid=cfg.cid, hidden=128, n_q=2, n_kv=1, head_dim=64, ffn=128,
              vocab=cfg.vocab, batch=cfg.batch, K=cfg.K, ctx_lo=0, ctx_hi=None)
    inp = S.make_inputs(h, capacity=8)
    head, _ = make_head(h, inp, max_k=max(cfg.K, 1))
    return head


VCASES = {
    # (config, temperature)
    "ragged-k3": (small(name="vs1", cid=170, batch=3, K=3, vocab=5003), 1.0),
    "k5-b1": (small(name="vs2", cid=171, batch=1, K=5, vocab=4099), 0.7),
    "k0": (small(name="vs3", cid=172, batch=4, K=0, vocab=3001), 1.0),
    "k1-b9": (small(name="vs4", cid=173, batch=9, K=1, vocab=8192), 1.3),
    "k8-b16": (small(name="vs5", cid=174, batch=16, K=8, vocab=2048), 1.0),
    # full vocabulary of the Qwen3-8B-shaped head: B=1 K=5, B=32 K=3, B=64 K=1
    "q8b": (S.get_config("q8b"), 1.0),
    "q8b-b32": (S.get_config("q8b-b32"), 1.0),
    "wide": (S.get_config("wide"), 1.0),
}


def _drafts(zl, T, seeds, offset):
    B, K = zl.shape[0], zl.shape[1]
    if K == 0:
        return np.zeros((B, 0), np.int64)
    return np.stack([SP.sample_tokens(zl[:, j], T, seeds, offset, j)[0] for j in range(K)], 1)


@pytest.mark.parametrize("case", list(VCASES))
def test_verify_sample_parity(case):
    cfg, T = VCASES[case]
    K, B = cfg.K, cfg.batch
    tl, zl = S.sampling_logits(cfg, K)
    seeds = S.sample_seeds(cfg)
    offset = 5
    d = _drafts(zl, T, seeds, offset)
    r = SP.verify_sample(tl, zl, d, T, seeds, offset)
    head = verify_head(cfg)
    tl_d = torch.from_numpy(tl).cuda()
    zl_d = torch.from_numpy(zl).cuda() if K else None
    d_d = torch.from_numpy(d.astype(np.int32)).cuda() if K else None
    for rep in range(2):  # the second call checks that partials, keys and counters were reset
        acc, nxt = head.verify_sample(tl_d, zl_d, d_d, T, seeds_dev(seeds), offset)
        assert head.get_error() == 0
        acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
        checked = 0
        for b in range(B):
            a = int(r["accepted_len"][b])
            consulted = r["margin"][b, :min(a + 1, K)]
            if np.all(np.abs(consulted) > GATE) and r["gap"][b] > GATE:
                assert acc[b] == a and nxt[b] == r["next_token"][b], (rep, b)
                checked += 1
        assert checked >= max(1, (3 * B) // 4), checked
    head.close()


def test_verify_sample_identical_distributions_accept_all():
    cfg = small(name="vs6", cid=175, batch=6, K=4, vocab=6000)
    tl, _ = S.sampling_logits(cfg, cfg.K)
    zl = np.ascontiguousarray(tl[:, :cfg.K])
    seeds = S.sample_seeds(cfg)
    d = _drafts(zl, 1.0, seeds, 0)
    r = SP.verify_sample(tl, zl, d, 1.0, seeds, 0)
    head = verify_head(cfg)
    acc, nxt = head.verify_sample(torch.from_numpy(tl).cuda(), torch.from_numpy(zl).cuda(),
                                  torch.from_numpy(d.astype(np.int32)).cuda(), 1.0,
                                  seeds_dev(seeds), 0)
    assert np.all(acc.cpu().numpy() == cfg.K) and np.all(r["accepted_len"] == cfg.K)
    ok = r["gap"] > GATE
    assert np.array_equal(nxt.cpu().numpy()[ok], r["next_token"][ok]) and ok.sum() >= 4
    head.close()


def test_verify_sample_errors():
    from mtp_self_speculative_amd import MtpError
    cfg = small(name="vs7", cid=176, batch=3, K=3, vocab=1000)
    tl, zl = S.sampling_logits(cfg, cfg.K)
    seeds = S.sample_seeds(cfg)
    d = _drafts(zl, 1.0, seeds, 1).astype(np.int32)
    d[1, 0] = cfg.vocab  # out of range: rejected at position 0, error bit set
    head = verify_head(cfg)
    args = (torch.from_numpy(tl).cuda(), torch.from_numpy(zl).cuda(),
            torch.from_numpy(d).cuda())
    acc, _ = head.verify_sample(*args, 1.0, seeds_dev(seeds), 1)
    assert head.get_error() == 1
    assert int(acc[1].item()) == 0
    for bad_t in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(MtpError):
            head.verify_sample(*args, bad_t, seeds_dev(seeds), 1)
    head.close()


DCASES = {
    # (config, temperature): bf16 batch 1-2 take the pipelined GEMV, 3-64 the matrix-core
    # contraction, fp32 the column-blocked GEMV
    "bf16-b1": (small(name="ds1", cid=180, batch=1, K=4), 1.0),
    "bf16-b2": (small(name="ds2", cid=181, batch=2, K=3), 1.0),
    "bf16-mm-b5": (small(name="ds3", cid=182, batch=5, K=3), 1.0),
    "bf16-mm-b33": (small(name="ds4", cid=183, batch=33, K=2, hidden=256, n_q=4, n_kv=2,
                          head_dim=64, ffn=512, vocab=4099, ctx_hi=64), 1.0),
    "f32-b3": (small(name="ds5", cid=184, batch=3, K=3, hidden=256, vocab=3001, dtype="f32"), 0.7),
    # 64 sequences over a 50021-row vocabulary: the sampling lm_head on 256-row items in
    # 128-column stages (the last item ends inside its first 128-row block)
    "bf16-mm-b64-wide-items": (small(name="ds6", cid=185, batch=64, K=2, hidden=256, n_q=4,
                                     n_kv=2, head_dim=64, ffn=512, vocab=50021, ctx_hi=64), 1.0),
    # full q8b head: each wave of the lm_head kernel draws noise for 64 rows at a time and
    # owns more than 64 vocabulary rows here, so the refill is exercised
    "q8b": (S.get_config("q8b"), 1.0),
}


@pytest.mark.parametrize("case", list(DCASES))
def test_draft_sample_parity(case):
    cfg, T = DCASES[case]
    K, B = cfg.K, cfg.batch
    inp = S.make_inputs(cfg, capacity=int(S.cache_lengths(cfg).max()) + K + 4)
    head, cache = make_head(cfg, inp)
    seeds = S.sample_seeds(cfg)
    offset = 3
    lt = torch.from_numpy(inp.last_tokens.astype(np.int32)).cuda()
    tok, lg = head.draft_sample(to_dev(inp.hidden, cfg.dtype), lt, cache, K, T, seeds_dev(seeds),
                                offset)
    assert head.get_error() == 0
    tok, lg = tok.cpu().numpy(), lg.cpu().numpy()
    g_len, g_pos = cache.len.cpu().numpy(), cache.pos.cpu().numpy()
    head.close()
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, K,
                force_tokens=tok, sample={"T": T, "seeds": seeds, "offset": offset})
    assert np.array_equal(g_len, inp.lens + K) and np.array_equal(g_pos, inp.pos + K)
    dl = np.max(np.abs(lg - np.transpose(r["logits"], (1, 0, 2))))
    assert dl < TOL[cfg.dtype], dl
    checked = 0
    for k in range(K):
        for b in range(B):
            if r["margin"][k, b] > MARGIN / T:
                assert int(r["draft_tokens"][b, k]) == int(tok[b, k]), (k, b)
                checked += 1
    assert checked >= max(1, (B * K) // 2), checked
    # a sample, not the argmax: over all steps some token differs from the greedy choice
    if B * K >= 8:
        assert np.any(tok != np.argmax(lg, axis=-1))


def test_gpu_speculative_sampling_reproduces_target_sequence_probabilities():
    """Many independent generations in one batch: the GPU head drafts by sampling, the GPU
    verifies by speculative sampling against a tiny random target sharing its embedding and
    lm_head, and rollback commits; the first three emitted tokens follow the target's exact
    sequence probabilities (chi-square)."""
    from oracle.tiny_target import TinyTarget, softmax_rows, speculative_sample_batch
    V, K, T, n = 4, 2, 1.0, 2000
    cfg = small(name="gsamp", cid=190, hidden=128, n_q=4, n_kv=2, head_dim=64, ffn=256, vocab=V,
                batch=n, K=K, ctx_lo=0, ctx_hi=None, dtype="f32")
    inp = S.make_inputs(cfg, capacity=32)
    head, cache = make_head(cfg, inp)
    tgt = TinyTarget(cfg, S.target_weights(cfg, 2), inp.weights["embed"], inp.weights["lm_head"])
    prompt = [int(x) for x in S.prompt_tokens(cfg, 5)]
    cache.len.zero_()
    cache.pos.fill_(len(prompt) - 1)
    seeds = S.sample_seeds(cfg)
    sd = seeds_dev(seeds)
    p1 = softmax_rows(tgt.forward(prompt)[1][-1:], T)[0]
    first = np.random.default_rng(13).choice(V, size=n, p=p1)
    st = {}

    def draft_fn(h, last, K_, it):
        tok, lg = head.draft_sample(torch.from_numpy(np.asarray(h, np.float32)).cuda(),
                                    torch.from_numpy(last.astype(np.int32)).cuda(), cache, K_, T,
                                    sd, it)
        st["d"], st["lg"] = tok, lg
        return tok.cpu().numpy(), lg.cpu().numpy()

    def verify_fn(rows, d, dl, it):
        a, nx = head.verify_sample(torch.from_numpy(rows.astype(np.float32)).cuda(), st["lg"],
                                   st["d"], T, sd, it)
        st["a"] = a
        return a.cpu().numpy(), nx.cpu().numpy()

    def commit_fn(a):
        head.rollback(cache, st["a"], K)

    out, acc = speculative_sample_batch(tgt, prompt, 3, first, draft_fn, verify_fn, commit_fn, K)
    assert head.get_error() == 0
    head.close()
    probs = np.zeros((V, V, V))
    for x1 in range(V):
        p2 = softmax_rows(tgt.forward(prompt + [x1])[1][-1:], T)[0]
        for x2 in range(V):
            p3 = softmax_rows(tgt.forward(prompt + [x1, x2])[1][-1:], T)[0]
            probs[x1, x2] = p1[x1] * p2[x2] * p3
    counts = np.bincount(out[:, 0] * V * V + out[:, 1] * V + out[:, 2], minlength=V ** 3)
    expect = probs.ravel() * n
    keep = expect >= 5
    obs, exp = counts[keep], expect[keep]
    if not keep.all():
        obs = np.append(obs, counts[~keep].sum())
        exp = np.append(exp, expect[~keep].sum())
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert stats.chi2.sf(chi2, len(obs) - 1) > 1e-5, chi2
    rate = np.concatenate(acc).mean() / K
    assert 0.05 < rate < 0.95
