"""Exact MTP-cache catch-up after verification: HIP path against the oracle."""
import numpy as np
import pytest

import mtp_synth as S
from gpu_util import TOL, cache_to_np, make_head, small, to_dev
from oracle import mtp_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

CASES = {
    # bf16, 3 x 4 candidate rows: matrix-core route
    "bf16-mm": small(name="cu1", cid=160, batch=3, K=4, ctx_lo=5, ctx_hi=200),
    # fp32, 2 x 3 rows: column-blocked GEMV route
    "f32": small(name="cu2", cid=161, batch=2, K=3, hidden=256, vocab=3001, dtype="f32",
                 ctx_lo=1, ctx_hi=100),
    # bf16, 1 x 2 rows: pipelined GEMV route
    "bf16-pipe": small(name="cu3", cid=162, batch=1, K=2, ctx_lo=30, ctx_hi=None),
    # bf16, 20 x 4 = 80 rows: one group on the tiled contraction (more than 64 rows)
    "bf16-tiled-80": small(name="cu4", cid=163, batch=20, K=4, hidden=512, n_q=8, n_kv=2,
                         ctx_lo=0, ctx_hi=120),
    # bf16, 4 x 3 rows on the matrix cores with n_q * d = 320, not a whole 128-row tile:
    # eh_proj from the packed copy, the K/V rows from the row-major weights
    "bf16-mm-kv-rowmajor": small(name="cu5", cid=164, batch=4, K=3, hidden=320, n_q=5, n_kv=1,
                                 head_dim=64, ffn=640, vocab=2053, ctx_lo=3, ctx_hi=90),
    # bf16, 12 x 4 = 48 rows (three 16-row tiles): eh_proj's 384 rows are three 128-row
    # blocks, and the K/V rows start at the packed copy's third (odd) 128-row block
    "bf16-mm-odd-kv-block": small(name="cu6", cid=165, batch=12, K=4, hidden=384, n_q=3, n_kv=1,
                                head_dim=128, ffn=768, vocab=3001, ctx_lo=2, ctx_hi=150),
    # bf16, 33 x 4 = 132 rows: one group on the tiled contraction, two 128-row input tiles
    # (the second ragged)
    "bf16-tiled-132": small(name="cu7", cid=166, batch=33, K=4, hidden=256, n_q=4, n_kv=2,
                            head_dim=64, ffn=512, vocab=3001, ctx_lo=2, ctx_hi=100),
    # bf16, 260 x 8 = 2080 rows: a 2048-row group on the tiled contraction, then 32 rows on
    # the weight-streaming one (the draft before it, 260 sequences, takes the GEMV)
    "bf16-tiled-then-streaming": small(name="cu8", cid=167, batch=260, K=8, hidden=256, n_q=4,
                                       n_kv=2, head_dim=64, ffn=512, vocab=3001, ctx_lo=2,
                                       ctx_hi=40),
    # the Qwen3-8B-shaped head at full size, B=1 K=5 and B=32 K=3
    "q8b": S.get_config("q8b"),
    "q8b-b32": S.get_config("q8b-b32"),
}


@pytest.mark.parametrize("case", list(CASES))
def test_catchup_parity(case):
    cfg = CASES[case]
    K, B = cfg.K, cfg.batch
    inp = S.make_inputs(cfg, capacity=int(S.cache_lengths(cfg).max()) + K + 8)
    head, cache = make_head(cfg, inp)
    hid = to_dev(inp.hidden, cfg.dtype)
    lt = torch.from_numpy(inp.last_tokens.astype(np.int32)).cuda()
    d = head.draft(hid, lt, cache, K)
    torch.cuda.synchronize()
    d_np = d.cpu().numpy()
    th = S.target_hidden(cfg, K)
    acc = np.random.default_rng(cfg.cid).integers(0, K + 1, size=B).astype(np.int32)
    acc[0] = K  # the full-acceptance gap is always covered
    head.catchup(cache, to_dev(th, cfg.dtype), d, torch.from_numpy(acc).cuda())
    assert head.get_error() == 0
    torch.cuda.synchronize()
    gk, gv = cache_to_np(cache.k, cfg.dtype), cache_to_np(cache.v, cfg.dtype)
    g_len, g_pos = cache.len.cpu().numpy(), cache.pos.cpu().numpy()
    head.close()

    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, K,
                force_tokens=d_np)
    lens, pos = O.kv_catchup(cfg, W, th, d_np, acc, kc, vc, r["lens"], r["pos"], K)
    assert np.array_equal(g_len, lens) and np.array_equal(g_pos, pos)
    assert np.array_equal(g_len, inp.lens + acc + 1)
    tol = TOL[cfg.dtype]
    for b in range(B):
        L0, a = int(inp.lens[b]), int(acc[b])
        assert np.array_equal(gk[b, :, :L0], inp.k_cache[b, :, :L0])
        assert np.array_equal(gv[b, :, :L0], inp.v_cache[b, :, :L0])
        for name, got, ref in (("k", gk, kc), ("v", gv, vc)):
            x = O.as_float(got[b, :, L0:L0 + a + 1], cfg.dtype)
            y = O.as_float(ref[b, :, L0:L0 + a + 1], cfg.dtype)
            assert np.allclose(x, y, rtol=1e-2 if cfg.dtype == "bf16" else 0, atol=tol), (name, b)


def test_speculative_decoding_with_catchup_on_gpu_equals_greedy():
    """GPU head drafts, GPU verifies from the target's hidden states, GPU catch-up commits
    the cache; the output equals plain greedy decoding and the committed cache matches
    the oracle's exact cache for the same committed tokens."""
    from oracle.tiny_target import TinyTarget, speculative_greedy
    cfg = small(name="e2ec", cid=143, hidden=128, n_q=4, n_kv=2, head_dim=64, ffn=256, vocab=8,
                batch=1, K=3, ctx_lo=0, ctx_hi=None, dtype="f32")
    inp = S.make_inputs(cfg, capacity=160)
    head, cache = make_head(cfg, inp)
    tw = S.target_weights(cfg, 2)
    tgt = TinyTarget(cfg, tw, inp.weights["embed"], inp.weights["lm_head"])
    gn = torch.from_numpy(np.ascontiguousarray(tw["g_final"])).cuda()
    prompt = S.prompt_tokens(cfg, 6)
    cache.len.zero_()
    cache.pos.fill_(len(prompt) - 1)
    st = {}

    def draft_fn(h, last, K, _seq):
        out = head.draft(torch.from_numpy(np.asarray(h, np.float32)[None]).cuda(),
                         torch.tensor([last], dtype=torch.int32, device="cuda"), cache, K)
        st["d"] = out
        return out[0].cpu().numpy()

    def verify_fn(hid_rows, d):
        st["th"] = torch.from_numpy(hid_rows[None].astype(np.float32)).cuda()
        a, n = head.verify_hidden(st["th"], gn, st["d"])
        st["a"] = a
        return int(a[0]), int(n[0])

    def commit_fn(a):
        head.catchup(cache, st["th"], st["d"], st["a"])

    out, acc = speculative_greedy(tgt, prompt, 40, draft_fn, verify_fn, commit_fn, 3,
                                  from_hidden=True)
    ref = tgt.greedy(prompt, 40)
    assert out == ref
    assert head.get_error() == 0
    n = int(cache.len.cpu().numpy()[0])
    gk = cache.k.cpu().numpy()
    head.close()
    # the oracle's exact cache: one-step drafts from the target's hidden states
    W = O.OracleWeights(cfg, inp.weights)
    seq = list(prompt) + ref
    hid, _ = tgt.forward(seq)
    kc, vc = np.zeros_like(inp.k_cache), np.zeros_like(inp.v_cache)
    for slot in range(n):
        p = len(prompt) - 1 + slot
        O.draft(cfg, W, hid[p][None], np.array([seq[p + 1]]), kc, vc, np.array([slot]),
                np.array([p]), 1)
    assert n > 20
    assert np.allclose(gk[:, :, :n], kc[:, :, :n], rtol=0, atol=TOL["f32"])
