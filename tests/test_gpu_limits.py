"""Parity at the limits of the supported shapes: the longest speculative length (K = 100),
batches past the matrix-core path (B = 80), rows too long for the batched row kernels
(hidden 8200), and a cache at the maximum capacity (262144 slots, 256 attention splits).
Each case runs the HIP path through the C ABI against the oracle on the same inputs."""
import numpy as np
import pytest

import mtp_synth as S
from gpu_util import MARGIN, TOL, cache_to_np, compare_draft, make_head, small, to_dev
from oracle import mtp_oracle as O
from oracle import sampling as SP

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

K100 = small(name="k100", cid=200, hidden=128, n_q=2, n_kv=1, head_dim=64, ffn=256, vocab=1000,
             batch=2, K=100, ctx_lo=3, ctx_hi=40, agree_lo=0.95)
DRAFT_CASES = {
    # the longest draft, bf16 at batch 2 (pipelined GEMV) and fp32
    "k100-bf16": K100,
    "k100-f32": K100.with_(name="k100f", cid=201, dtype="f32"),
    # 80 sequences: beyond the 64 of the matrix-core path, bf16 weights on the column GEMV
    "b80-bf16": small(name="b80", cid=202, hidden=256, n_q=4, n_kv=2, head_dim=64, ffn=512,
                      vocab=3001, batch=80, K=2, ctx_lo=0, ctx_hi=60),
    # hidden 8200: rows longer than the batched row kernels take, so 3 sequences use the GEMV
    "h8200-b3": small(name="h8200", cid=203, hidden=8200, n_q=2, n_kv=1, head_dim=64, ffn=256,
                      vocab=512, batch=3, K=2, ctx_lo=5, ctx_hi=30),
}


def _draft(cfg, inp, K):
    head, cache = make_head(cfg, inp)
    hid = to_dev(inp.hidden, cfg.dtype)
    lt = torch.from_numpy(inp.last_tokens.astype(np.int32)).cuda()
    tok, h, t2, lg = head.draft_debug(hid, lt, cache, K, want_logits=True)
    assert head.get_error() == 0
    out = {"tokens": tok.cpu().numpy(), "hidden": h.cpu().numpy(), "top2": t2.cpu().numpy(),
           "logits": lg.cpu().numpy(), "k": cache_to_np(cache.k, cfg.dtype),
           "len": cache.len.cpu().numpy(), "pos": cache.pos.cpu().numpy()}
    return head, cache, out


@pytest.mark.parametrize("case", list(DRAFT_CASES))
def test_draft_parity_at_limits(case):
    cfg = DRAFT_CASES[case]
    K = cfg.K
    inp = S.make_inputs(cfg, capacity=int(S.cache_lengths(cfg).max()) + K + 4)
    head, _, g = _draft(cfg, inp, K)
    head.close()
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, K,
                force_tokens=g["tokens"])
    n = compare_draft(cfg, r, g["tokens"], g["hidden"], g["top2"], g["logits"])
    assert n >= 0.5 * K * cfg.batch
    assert np.array_equal(g["len"], inp.lens + K) and np.array_equal(g["pos"], inp.pos + K)
    tol = TOL[cfg.dtype]
    for b in range(cfg.batch):
        L0 = int(inp.lens[b])
        assert np.array_equal(g["k"][b, :, :L0], inp.k_cache[b, :, :L0])
        x = O.as_float(g["k"][b, :, L0:L0 + K], cfg.dtype)
        y = O.as_float(kc[b, :, L0:L0 + K], cfg.dtype)
        assert np.allclose(x, y, rtol=1e-2 if cfg.dtype == "bf16" else 0, atol=tol)


def test_k100_verify_rollback_sampling_and_catchup():
    """K = 100 through every verification and commit entry point: greedy verification of
    planted logits (bit-exact), rollback, speculative-sampling verification (near-tie
    aware), verification from hidden states and the exact catch-up."""
    cfg = K100
    K, B, V = cfg.K, cfg.batch, cfg.vocab
    inp = S.make_inputs(cfg, capacity=int(S.cache_lengths(cfg).max()) + K + 4)
    head, cache, g = _draft(cfg, inp, K)
    d = torch.from_numpy(g["tokens"].astype(np.int32)).cuda()
    # greedy verification of planted logits
    tl = S.plant_target_logits(cfg, g["tokens"], 0)
    acc, nxt = head.verify(torch.from_numpy(tl).cuda(), d)
    a_o, n_o = O.verify(tl, g["tokens"])
    assert np.array_equal(acc.cpu().numpy(), a_o) and np.array_equal(nxt.cpu().numpy(), n_o)
    assert a_o.max() > 20  # the planted agreement reaches deep into the draft
    # rollback
    head.rollback(cache, acc, K)
    lens, pos = O.kv_rollback(inp.lens + K, inp.pos + K, a_o, K)
    assert np.array_equal(cache.len.cpu().numpy(), lens)
    assert np.array_equal(cache.pos.cpu().numpy(), pos)
    # sampling verification with 100 drafts: a perturbed draft distribution (early
    # rejections) and a nearly exact one (all 100 accepted, then the bonus draw)
    seeds = S.sample_seeds(cfg)
    sd = torch.from_numpy(seeds.view(np.int64)).cuda()
    for scale, full in ((0.1, False), (0.001, True)):
        st, sz = S.sampling_logits(cfg, K)
        sz[:, :, :] = st[:, :K] + scale * (sz - st[:, :K])
        ds = np.stack([SP.sample_tokens(sz[:, j], 1.0, seeds, 3, j)[0] for j in range(K)], 1)
        r = SP.verify_sample(st, sz, ds, 1.0, seeds, 3)
        acc_s, nxt_s = head.verify_sample(torch.from_numpy(st).cuda(),
                                          torch.from_numpy(sz).cuda(),
                                          torch.from_numpy(ds.astype(np.int32)).cuda(), 1.0, sd, 3)
        assert head.get_error() == 0
        acc_s, nxt_s = acc_s.cpu().numpy(), nxt_s.cpu().numpy()
        for b in range(B):
            a = int(r["accepted_len"][b])
            if np.all(np.abs(r["margin"][b, :min(a + 1, K)]) > 1e-3) and r["gap"][b] > 1e-3:
                assert acc_s[b] == a and nxt_s[b] == r["next_token"][b], (scale, b)
        assert (r["accepted_len"].min() == K) == full
    # verification from hidden states: 2 x 101 rows in four groups
    th, tn = S.target_hidden(cfg, K), S.target_norm(cfg)
    a_h, n_h, margin = O.verify_from_hidden(cfg, th, tn, inp.weights["lm_head"], g["tokens"])
    acc_h, nxt_h = head.verify_hidden(to_dev(th, cfg.dtype), to_dev(tn, cfg.dtype), d)
    acc_h, nxt_h = acc_h.cpu().numpy(), nxt_h.cpu().numpy()
    for b in range(B):
        if np.all(margin[b, :a_h[b] + 1] > MARGIN):
            assert acc_h[b] == a_h[b] and nxt_h[b] == n_h[b]
    head.close()
    # exact catch-up after the 100-step draft, full acceptance for sequence 0
    head, cache, g = _draft(cfg, inp, K)
    acc_c = np.array([K, 37], np.int32)
    head.catchup(cache, to_dev(th, cfg.dtype), torch.from_numpy(g["tokens"].astype(np.int32)).cuda(),
                 torch.from_numpy(acc_c).cuda())
    assert head.get_error() == 0
    gk = cache_to_np(cache.k, cfg.dtype)
    g_len = cache.len.cpu().numpy()
    head.close()
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    rd = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, K,
                 force_tokens=g["tokens"])
    lens_c, _ = O.kv_catchup(cfg, W, th, g["tokens"], acc_c, kc, vc, rd["lens"], rd["pos"], K)
    assert np.array_equal(g_len, lens_c)
    for b in range(B):
        L0, a = int(inp.lens[b]), int(acc_c[b])
        x = O.as_float(gk[b, :, L0:L0 + a + 1], cfg.dtype)
        y = O.as_float(kc[b, :, L0:L0 + a + 1], cfg.dtype)
        assert np.allclose(x, y, rtol=1e-2, atol=TOL[cfg.dtype])


def test_maximum_capacity_cache():
    """A cache of 262144 slots (the supported maximum: 256 attention splits of 1024) filled
    to its last slots: the draft's attention reads all of it."""
    cap = 256 * 1024
    cfg = small(name="cap", cid=204, hidden=128, n_q=2, n_kv=1, head_dim=64, ffn=256, vocab=777,
                batch=1, K=2, ctx_lo=cap - 2, ctx_hi=None)
    inp = S.make_inputs(cfg, capacity=cap)
    head, _, g = _draft(cfg, inp, cfg.K)
    head.close()
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, cfg.K,
                force_tokens=g["tokens"])
    compare_draft(cfg, r, g["tokens"], g["hidden"], g["top2"], g["logits"])
    assert np.array_equal(g["len"], [cap])
    x = O.as_float(g["k"][0, :, cap - 2:], cfg.dtype)
    y = O.as_float(kc[0, :, cap - 2:], cfg.dtype)
    assert np.allclose(x, y, rtol=1e-2, atol=TOL[cfg.dtype])
