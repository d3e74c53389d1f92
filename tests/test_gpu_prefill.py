"""Prompt prefill of the MTP cache (mtp_kv_prefill): HIP path against the oracle, then
speculative decoding that starts from a prefilled cache."""
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
    # fp32 (column-blocked GEMV route), ragged counts including 0
    "f32": (small(name="pf1", cid=200, batch=3, K=1, hidden=256, vocab=3001, dtype="f32",
                  ctx_lo=1, ctx_hi=40), 9, [9, 4, 0]),
    # bf16, 1 x 2 rows: pipelined GEMV route
    "bf16-pipe": (small(name="pf2", cid=201, batch=1, K=1, ctx_lo=30, ctx_hi=None), 2, None),
    # bf16, 3 x 30 = 90 rows in one group on the tiled contraction (more than 64 rows),
    # ragged counts
    "bf16-mm": (small(name="pf3", cid=202, batch=3, K=2, ctx_lo=0, ctx_hi=60), 30, [30, 17, 0]),
    # bf16, 5 x 13 = 65 rows: one group on the tiled contraction, its 128-row input tile
    # ragged
    "bf16-mm-tail": (small(name="pf4", cid=203, batch=5, K=2, hidden=256, n_q=4, n_kv=2,
                           head_dim=64, ffn=512, vocab=2053, ctx_lo=3, ctx_hi=90), 13, None),
    # bf16, n_q * d = 320 (the K/V rows are not a whole 128-row block of the packed copy)
    "bf16-mm-kv-rowmajor": (small(name="pf5", cid=204, batch=4, K=3, hidden=320, n_q=5, n_kv=1,
                                  head_dim=64, ffn=640, vocab=2053, ctx_lo=0, ctx_hi=50), 11,
                            None),
    # bf16, 2 x 1050 = 2100 rows: a 2048-row group on the tiled contraction, then 52 rows on
    # the weight-streaming one
    "bf16-tiled-then-streaming": (small(name="pf6", cid=206, batch=2, K=1, hidden=256, n_q=4,
                                        n_kv=2, head_dim=64, ffn=512, vocab=2053, ctx_lo=0,
                                        ctx_hi=20), 1050, [1050, 1050]),
}


def _run(cfg, n, nv, cap, pos_off=0):
    inp = S.make_inputs(cfg, capacity=cap)
    th = S.prefill_hidden(cfg, n)
    tok = S.prefill_tokens(cfg, n)
    head, cache = make_head(cfg, inp)
    cache.len.copy_(torch.from_numpy(inp.lens.astype(np.int32)))
    pos0 = inp.pos.astype(np.int64) + pos_off
    cache.pos.copy_(torch.from_numpy(pos0.astype(np.int32)))
    nvt = None if nv is None else torch.tensor(nv, dtype=torch.int32, device="cuda")
    print(f"prefill {cfg.name}: B={cfg.batch} n={n} H={cfg.hidden} {cfg.dtype}", flush=True)
    head.prefill(cache, to_dev(th, cfg.dtype), torch.from_numpy(tok).cuda(), nvt)
    assert head.get_error() == 0
    torch.cuda.synchronize()
    g = {"k": cache_to_np(cache.k, cfg.dtype), "v": cache_to_np(cache.v, cfg.dtype),
         "len": cache.len.cpu().numpy(), "pos": cache.pos.cpu().numpy()}
    head.close()
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    ln, ps = O.kv_prefill(cfg, W, th, tok, kc, vc, inp.lens, pos0, nv)
    return inp, g, kc, vc, ln, ps


def _check(cfg, inp, g, kc, vc, ln, ps):
    tol = TOL[cfg.dtype]
    assert np.array_equal(g["len"], ln) and np.array_equal(g["pos"], ps)
    for name, oc in (("k", kc), ("v", vc)):
        gc, ic = g[name], getattr(inp, name + "_cache")
        for b in range(cfg.batch):
            L0, L1 = int(inp.lens[b]), int(ln[b])
            assert np.array_equal(gc[b, :, :L0], ic[b, :, :L0])   # older slots untouched
            assert np.array_equal(gc[b, :, L1:], ic[b, :, L1:])   # past the count untouched
            new_g = O.as_float(gc[b, :, L0:L1], cfg.dtype)
            new_o = O.as_float(oc[b, :, L0:L1], cfg.dtype)
            rt = 1e-2 if cfg.dtype == "bf16" else 0
            assert np.allclose(new_g, new_o, rtol=rt, atol=tol), (name, b)


@pytest.mark.parametrize("case", list(CASES))
def test_prefill_parity(case):
    cfg, n, nv = CASES[case]
    cap = int(S.cache_lengths(cfg).max()) + n + 4
    _check(cfg, *_run(cfg, n, nv, cap, pos_off=5))


def test_prefill_q8b_4096_token_prompt():
    """The Qwen3-8B-shaped head at full size: a 4096-token prompt into an empty cache
    (two groups of 2048 rows on the tiled contraction), every slot against the oracle."""
    cfg = S.get_config("q8b").with_(ctx_lo=0, ctx_hi=None)
    n = 4096
    _check(cfg, *_run(cfg, n, None, n + 64))


def test_prefill_q8b_b32_ragged_prompts():
    """The batched workload's shape: 32 prompts of ragged lengths (1..300 rows) in one call
    (9600 candidate rows: four 2048-row groups and one of 1408 on the tiled contraction)."""
    cfg = S.get_config("q8b-b32").with_(ctx_lo=0, ctx_hi=None)
    n = 300
    nv = [int(x) for x in np.random.default_rng(5).integers(1, n + 1, size=cfg.batch)]
    nv[0] = n
    _check(cfg, *_run(cfg, n, nv, n + 16))


def test_prefill_errors_and_noop():
    from mtp_self_speculative_amd import _lib as L
    cfg, n, _ = CASES["bf16-mm"]
    inp = S.make_inputs(cfg, capacity=100)
    head, cache = make_head(cfg, inp)
    th = to_dev(S.prefill_hidden(cfg, n), cfg.dtype)
    tok = torch.from_numpy(S.prefill_tokens(cfg, n)).cuda()
    len0 = cache.len.clone()
    head.prefill(cache, th[:, :0].contiguous(), tok[:, :0].contiguous())   # n = 0: nothing
    assert torch.equal(cache.len, len0)
    bad = torch.tensor([n + 1, -1, 2], dtype=torch.int32, device="cuda")
    head.prefill(cache, th, tok, bad)   # counts clamped to [0, n], error bit set
    assert head.get_error() & L.DEVERR_COUNT
    assert np.array_equal(cache.len.cpu().numpy(), inp.lens + np.array([n, 0, 2]))
    cache.len.fill_(100 - 5)
    head.prefill(cache, th, tok)        # rows past the capacity are skipped, error bit set
    assert head.get_error() & L.DEVERR_CAPACITY
    tok_bad = tok.clone()
    tok_bad[1, 3] = cfg.vocab
    cache.len.copy_(len0)
    head.prefill(cache, th, tok_bad)
    assert head.get_error() & L.DEVERR_TOKEN
    assert head.get_error() == 0
    head.close()


def test_decoding_from_a_prefilled_cache_equals_greedy_and_tracks_the_oracle():
    """End to end on a tiny target: prefill the prompt from an empty cache, then greedy
    speculative decoding with the GPU head, verification and exact catch-up; the output is
    plain greedy decoding and the cache equals the oracle's prefill of the committed
    sequence."""
    from oracle.tiny_target import TinyTarget, speculative_greedy
    cfg = small(name="pfe", cid=205, hidden=128, n_q=4, n_kv=2, head_dim=64, ffn=256, vocab=16,
                batch=1, K=3, ctx_lo=0, ctx_hi=None, dtype="f32")
    inp = S.make_inputs(cfg, capacity=160)
    head, cache = make_head(cfg, inp)
    tw = S.target_weights(cfg, 2)
    tgt = TinyTarget(cfg, tw, inp.weights["embed"], inp.weights["lm_head"])
    prompt = [int(x) for x in S.prompt_tokens(cfg, 12)]
    P = len(prompt)
    hid, _ = tgt.forward(prompt)
    cache.len.zero_()
    cache.pos.zero_()
    head.prefill(cache, torch.from_numpy(np.ascontiguousarray(hid[None, :P - 1], np.float32)).cuda(),
                 torch.tensor([prompt[1:]], dtype=torch.int32, device="cuda"))
    tn = torch.from_numpy(np.asarray(tw["g_final"], np.float32)).cuda()
    st = {}

    def draft_fn(h, last, K, _seq):
        out = head.draft(torch.from_numpy(np.asarray(h, np.float32)[None]).cuda(),
                         torch.tensor([last], dtype=torch.int32, device="cuda"), cache, K)
        st["d"], st["K"] = out, K
        return out[0].cpu().numpy()

    def verify_fn(rows, d):
        th = torch.from_numpy(np.ascontiguousarray(rows[None], np.float32)).cuda()
        a, n = head.verify_hidden(th, tn, st["d"])
        st["a"], st["th"] = a, th
        return int(a[0]), int(n[0])

    def commit_fn(a):
        head.catchup(cache, st["th"], st["d"], st["a"])

    n_new = 30
    out, acc = speculative_greedy(tgt, prompt, n_new, draft_fn, verify_fn, commit_fn, 3,
                                  from_hidden=True)
    assert out == tgt.greedy(prompt, n_new)
    assert head.get_error() == 0
    n = int(cache.len[0])
    # the first generated token comes from the target alone; every later one went through an
    # iteration whose committed pairs were written: P - 1 + (emitted - 1) slots
    assert n == int(cache.pos[0]) and n >= P - 2 + n_new
    seq = prompt + tgt.greedy(prompt, n_new + 4)
    hid_all, _ = tgt.forward(seq)
    W = O.OracleWeights(cfg, inp.weights)
    rk, rv = np.zeros_like(inp.k_cache), np.zeros_like(inp.v_cache)
    O.kv_prefill(cfg, W, hid_all[None, :n], np.array([seq[1:n + 1]]), rk, rv, np.array([0]),
                 np.array([0]))
    gk, gv = cache.k.cpu().numpy(), cache.v.cpu().numpy()
    assert np.allclose(gk[:, :, :n], rk[:, :, :n], rtol=0, atol=1e-4)
    assert np.allclose(gv[:, :, :n], rv[:, :, :n], rtol=0, atol=1e-4)
    head.close()
