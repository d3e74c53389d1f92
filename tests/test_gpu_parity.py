"""Parity of the HIP path (through the C ABI) with the oracle, element by element on the
same seeded inputs. Needs an MI355X and the built libmtp.so."""
import numpy as np
import pytest

import mtp_synth as S
from gpu_util import MARGIN, TOL, cache_to_np, compare_draft, make_head, small, to_dev
from oracle import mtp_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def run_draft(cfg, inp, K, want_logits=True, B=None):
    head, cache = make_head(cfg, inp)
    B = B or cfg.batch
    hid = to_dev(inp.hidden[:B], cfg.dtype)
    lt = torch.from_numpy(inp.last_tokens[:B].astype(np.int32)).cuda()
    tok, h, t2, lg = head.draft_debug(hid, lt, cache, K, want_logits=want_logits)
    assert head.get_error() == 0
    torch.cuda.synchronize()
    out = {"tokens": tok.cpu().numpy(), "hidden": h.cpu().numpy(), "top2": t2.cpu().numpy(),
           "logits": None if lg is None else lg.cpu().numpy(),
           "k": cache_to_np(cache.k, cfg.dtype), "v": cache_to_np(cache.v, cfg.dtype),
           "len": cache.len.cpu().numpy(), "pos": cache.pos.cpu().numpy()}
    head.close()
    return out


def oracle_forced(cfg, inp, K, tokens, B=None):
    B = B or cfg.batch
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache[:B].copy(), inp.v_cache[:B].copy()
    r = O.draft(cfg, W, inp.hidden[:B], inp.last_tokens[:B], kc, vc, inp.lens[:B], inp.pos[:B], K,
                force_tokens=tokens)
    r["k"], r["v"] = kc, vc
    return r


def check_cache(cfg, inp, g, r, K, B):
    tol = TOL[cfg.dtype]
    assert np.array_equal(g["len"][:B], inp.lens[:B] + K)
    assert np.array_equal(g["pos"][:B], inp.pos[:B] + K)
    for name in ("k", "v"):
        gc, oc, ic = g[name], r[name], getattr(inp, name + "_cache")
        for b in range(B):
            L0 = int(inp.lens[b])
            # untouched slots stay bit-identical
            assert np.array_equal(gc[b, :, :L0], ic[b, :, :L0])
            assert np.array_equal(gc[b, :, L0 + K:], ic[b, :, L0 + K:])
            new_g = O.as_float(gc[b, :, L0:L0 + K], cfg.dtype)
            new_o = O.as_float(oc[b, :, L0:L0 + K], cfg.dtype)
            assert np.allclose(new_g, new_o, rtol=1e-2 if cfg.dtype == "bf16" else 0, atol=tol)


CASES = {
    "tiny": S.get_config("tiny"),
    # bf16, ragged H (384), F (1000), V (5003), ragged cache lengths, G = 3, B = 3
    "small-bf16": small(),
    # fp32, head_dim 64, G = 8, B = 5 (partially filled batch tile), K = 2
    "small-f32-g8": small(name="f32g8", cid=101, hidden=256, n_q=16, n_kv=2, head_dim=64, ffn=520,
                          vocab=3000, batch=5, K=2, ctx_lo=60, ctx_hi=200, dtype="f32"),
    # bf16, B = 9 (two batch tiles), G = 4, empty caches (len 0), K = 5
    "small-bf16-b9-empty": small(name="b9", cid=102, hidden=512, n_q=8, n_kv=2, head_dim=128,
                                 ffn=1536, vocab=7777, batch=9, K=5, ctx_lo=0, ctx_hi=None),
    # bf16 batched path (MFMA contraction): B = 16, 17, 33, 64 cover one to four 16-sequence
    # tiles, full and partial; ragged K chunks (H = 640, F = 1800), ragged vocab tile
    "mm-b16": small(name="mm16", cid=104, hidden=640, n_q=10, n_kv=2, head_dim=64, ffn=1800,
                    vocab=6007, batch=16, K=3, ctx_lo=1, ctx_hi=200),
    "mm-b17": small(name="mm17", cid=105, hidden=512, n_q=4, n_kv=4, head_dim=128, ffn=1536,
                    vocab=4099, batch=17, K=2, ctx_lo=0, ctx_hi=150),
    "mm-b33": small(name="mm33", cid=106, hidden=512, n_q=8, n_kv=1, head_dim=64, ffn=2048,
                    vocab=5000, batch=33, K=2, ctx_lo=30, ctx_hi=300),
    "mm-b64": small(name="mm64", cid=107, hidden=768, n_q=6, n_kv=2, head_dim=128, ffn=2304,
                    vocab=8192, batch=64, K=2, ctx_lo=1, ctx_hi=120),
    # bf16, B = 40 ragged caches (len 1..4000) over 8 KV heads (G = 2): 640 attention
    # items, more than the chip runs at once, so they run in the longest-first order
    "mm-b40-ragged-order": small(name="order", cid=108, hidden=256, n_q=16, n_kv=8, head_dim=64,
                                 ffn=512, vocab=2048, batch=40, K=2, ctx_lo=1, ctx_hi=4000),
    # B=40 with a 50000-row vocabulary: the lm_head runs on 256-row items (196 of them), the
    # last one ending inside its first 128-row block, so its second block reads the dummy
    "mm-b40-wide-items": small(name="w8lm", cid=109, hidden=256, n_q=4, n_kv=2, head_dim=64,
                               ffn=512, vocab=50000, batch=40, K=2, ctx_lo=1, ctx_hi=200),
    # the same vocabulary at B = 64: four 16-sequence tiles on 256-row items, whose greedy
    # lm_head streams 128-column stages
    "mm-b64-wide-items": small(name="w8lm64", cid=110, hidden=256, n_q=4, n_kv=2, head_dim=64,
                               ffn=512, vocab=50000, batch=64, K=2, ctx_lo=1, ctx_hi=200),
    # the same with H = 320: the second 256-column chunk ends inside its first half, so one
    # 128-column stage of every item lies wholly past the row end
    "mm-b64-wide-items-ragged-h": small(name="w8lm64r", cid=111, hidden=320, n_q=5, n_kv=1,
                                        head_dim=64, ffn=640, vocab=50000, batch=64, K=2,
                                        ctx_lo=1, ctx_hi=150),
    # bf16, B = 2, a cache long enough for several attention splits (len 3000..3100)
    "small-bf16-long": small(name="long", cid=103, hidden=256, n_q=4, n_kv=4, head_dim=128,
                             ffn=512, vocab=2048, batch=2, K=3, ctx_lo=3000, ctx_hi=3100),
}


@pytest.mark.parametrize("case", list(CASES))
def test_draft_parity(case):
    cfg = CASES[case]
    inp = S.make_inputs(cfg, capacity=int(S.cache_lengths(cfg).max()) + cfg.K + 7)
    g = run_draft(cfg, inp, cfg.K)
    r = oracle_forced(cfg, inp, cfg.K, g["tokens"])
    n = compare_draft(cfg, r, g["tokens"], g["hidden"], g["top2"], g["logits"])
    assert n >= 0.5 * cfg.K * cfg.batch, f"only {n} tokens above the near-tie margin"
    check_cache(cfg, inp, g, r, cfg.K, cfg.batch)


def test_draft_k1_and_k0():
    cfg = CASES["small-bf16"]
    inp = S.make_inputs(cfg, capacity=320)
    g = run_draft(cfg, inp, 1)
    r = oracle_forced(cfg, inp, 1, g["tokens"])
    compare_draft(cfg, r, g["tokens"], g["hidden"], g["top2"], g["logits"])
    head, cache = make_head(cfg, inp)
    hid = to_dev(inp.hidden, cfg.dtype)
    lt = torch.from_numpy(inp.last_tokens).cuda()
    out = head.draft(hid, lt, cache, 0)
    torch.cuda.synchronize()
    assert out.numel() == 0
    assert np.array_equal(cache.len.cpu().numpy(), inp.lens)


def test_determinism_and_batch_independence():
    """Reruns are bit-identical; a sequence's result does not depend on the rest of the
    batch (bit-exact between batch sizes served by the same kernels, within the parity
    tolerance across kernel families)."""
    cfg = CASES["small-bf16-b9-empty"].with_(ctx_lo=20, ctx_hi=90)
    inp = S.make_inputs(cfg, capacity=100)
    a = run_draft(cfg, inp, cfg.K)
    b = run_draft(cfg, inp, cfg.K)
    assert np.array_equal(a["tokens"], b["tokens"])
    assert np.array_equal(a["hidden"], b["hidden"])
    assert np.array_equal(a["k"], b["k"]) and np.array_equal(a["v"], b["v"])
    one = run_draft(cfg, inp, cfg.K, B=1)
    two = run_draft(cfg, inp, cfg.K, B=2)
    assert np.array_equal(one["tokens"][0], two["tokens"][0])
    assert np.array_equal(one["hidden"][:, 0], two["hidden"][:, 0])
    r = oracle_forced(cfg, inp, cfg.K, a["tokens"])
    for k in range(cfg.K):
        if r["margin"][k, 0] > MARGIN:
            assert one["tokens"][0, k] == a["tokens"][0, k]
    if np.array_equal(one["tokens"][0], a["tokens"][0]):
        assert np.max(np.abs(one["hidden"][:, 0] - a["hidden"][:, 0])) < TOL[cfg.dtype]


def test_poisoned_stale_slots_do_not_leak():
    cfg = CASES["small-bf16"]
    inp = S.make_inputs(cfg, capacity=320)
    ref = run_draft(cfg, inp, cfg.K)
    pk, pv = inp.k_cache.copy(), inp.v_cache.copy()
    for b in range(cfg.batch):
        pk[b, :, inp.lens[b]:] = 0x7FC0  # bf16 quiet NaN
        pv[b, :, inp.lens[b]:] = 0x7FC0
    inp2 = S.SynthInputs(cfg=cfg, capacity=inp.capacity, weights=inp.weights, hidden=inp.hidden,
                         last_tokens=inp.last_tokens, k_cache=pk, v_cache=pv, lens=inp.lens,
                         pos=inp.pos)
    got = run_draft(cfg, inp2, cfg.K)
    assert np.array_equal(got["tokens"], ref["tokens"])
    assert np.array_equal(got["hidden"], ref["hidden"])


@pytest.mark.parametrize("B,K,V", [(1, 5, 151936), (32, 3, 151936), (4, 0, 1000), (3, 7, 4099),
                                   (64, 1, 129280)])
def test_verify_parity(B, K, V):
    cfg = small(name="ver", cid=110 + K, batch=B, vocab=V, K=K, agree_lo=0.7)
    rng = np.random.default_rng(B * 100 + K)
    d = rng.integers(0, V, size=(B, K)).astype(np.int32)
    t = S.plant_target_logits(cfg, d, 0)
    # crafted ties in a few rows: two equal maxima, the lower index must win
    for b in range(0, B, 3):
        j = b % (K + 1)
        t[b, j, 7] = t[b, j, V - 3] = 50.0
    from mtp_self_speculative_amd import MtpHead  # noqa: F401
    inp = S.make_inputs(small(name="verh", cid=119, vocab=V, batch=B, K=max(K, 1), ctx_lo=1,
                              ctx_hi=None, hidden=64, n_q=2, n_kv=1, ffn=64), capacity=16)
    head, _ = make_head(inp.cfg, inp, max_batch=B, max_k=max(K, 1))
    acc, nxt = head.verify(torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda() if K else None)
    assert head.get_error() == 0
    a_o, n_o = O.verify(t, d)
    assert np.array_equal(acc.cpu().numpy(), a_o)
    assert np.array_equal(nxt.cpu().numpy(), n_o)
    # repeat: counters and keys were reset by the previous call
    acc2, nxt2 = head.verify(torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda() if K else None)
    assert np.array_equal(acc2.cpu().numpy(), a_o) and np.array_equal(nxt2.cpu().numpy(), n_o)
    head.close()


@pytest.mark.parametrize("K", [0, 1, 3, 5])
def test_rollback_parity(K):
    cfg = small(name="rb", cid=120, batch=40, K=max(K, 1), ctx_lo=10, ctx_hi=50, hidden=64, n_q=2,
                n_kv=1, ffn=64, vocab=100)
    inp = S.make_inputs(cfg, capacity=64)
    head, cache = make_head(cfg, inp)
    rng = np.random.default_rng(K)
    a = rng.integers(0, K + 1, size=cfg.batch).astype(np.int32)
    cache.len += K
    cache.pos += K
    head.rollback(cache, torch.from_numpy(a).cuda(), K)
    assert head.get_error() == 0
    ln, ps = O.kv_rollback(inp.lens + K, inp.pos + K, a, K)
    assert np.array_equal(cache.len.cpu().numpy(), ln)
    assert np.array_equal(cache.pos.cpu().numpy(), ps)
    head.close()


def test_chained_iterations():
    """draft -> planted target logits -> verify -> rollback, several iterations; the GPU
    state (len, pos, accepted lengths, cache contents) tracks the oracle's."""
    cfg = small(name="chain", cid=130, batch=4, K=3, ctx_lo=5, ctx_hi=40, agree_lo=0.7)
    iters = 6
    inp = S.make_inputs(cfg, capacity=40 + iters * cfg.K + 4)
    head, cache = make_head(cfg, inp)
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    lens, pos = inp.lens.astype(np.int64), inp.pos.astype(np.int64)
    last = inp.last_tokens.copy()
    for it in range(iters):
        hid_np = S.hidden_states(cfg, it)
        tok, hid, t2, _ = head.draft_debug(to_dev(hid_np, cfg.dtype),
                                           torch.from_numpy(last.astype(np.int32)).cuda(), cache,
                                           cfg.K)
        g_tok = tok.cpu().numpy()
        r = O.draft(cfg, W, hid_np, last, kc, vc, lens, pos, cfg.K, force_tokens=g_tok)
        compare_draft(cfg, r, g_tok, hid.cpu().numpy(), t2.cpu().numpy())
        t = S.plant_target_logits(cfg, g_tok, it)
        acc, nxt = head.verify(torch.from_numpy(t).cuda(), tok)
        head.rollback(cache, acc, cfg.K)
        a_o, n_o = O.verify(t, g_tok)
        assert np.array_equal(acc.cpu().numpy(), a_o) and np.array_equal(nxt.cpu().numpy(), n_o)
        lens, pos = O.kv_rollback(r["lens"], r["pos"], a_o, cfg.K)
        assert np.array_equal(cache.len.cpu().numpy(), lens)
        assert np.array_equal(cache.pos.cpu().numpy(), pos)
        last = n_o.astype(np.int32)
    gk = cache_to_np(cache.k, cfg.dtype)
    for b in range(cfg.batch):
        n = int(lens[b])
        assert np.allclose(O.as_float(gk[b, :, :n], "bf16"), O.as_float(kc[b, :, :n], "bf16"),
                           rtol=1e-2, atol=2e-2)
    assert head.get_error() == 0
    head.close()


def test_device_error_paths_stay_in_bounds():
    """A bad token id and a cache without room are reported through the error word;
    the kernels clamp and stay inside every buffer."""
    cfg = CASES["small-bf16"]
    inp = S.make_inputs(cfg, capacity=310)
    head, cache = make_head(cfg, inp)
    hid = to_dev(inp.hidden, cfg.dtype)
    bad = torch.tensor([0, cfg.vocab + 5, -1], dtype=torch.int32, device="cuda")
    head.draft(hid, bad, cache, 2)
    bits = head.get_error()
    assert bits & 1
    cache.len.fill_(308)
    head.draft(hid, torch.from_numpy(inp.last_tokens).cuda(), cache, 4)
    bits = head.get_error()
    assert bits & 2
    acc = torch.tensor([0, 9, -2], dtype=torch.int32, device="cuda")
    head.rollback(cache, acc, 3)
    assert head.get_error() & 4
    assert head.get_error() == 0
    head.close()


def test_host_validation_errors():
    """Out-of-range K and B are refused twice over: by the wrapper (ValueError, before the
    library) and by the library itself (status returned before any launch)."""
    import ctypes

    from mtp_self_speculative_amd import MtpError
    from mtp_self_speculative_amd import _lib as L
    cfg = CASES["small-bf16"]
    inp = S.make_inputs(cfg, capacity=320)
    head, cache = make_head(cfg, inp)
    hid = to_dev(inp.hidden, cfg.dtype)
    lt = torch.from_numpy(inp.last_tokens).cuda()
    out = torch.zeros((cfg.batch, cfg.K + 1), dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    with pytest.raises(ValueError):
        head.draft(hid, lt, cache, cfg.K + 1)          # K > max_k
    with pytest.raises(MtpError) as e:
        L.mtp_draft(head.handle, hid.data_ptr(), lt.data_ptr(), cache.kv, cfg.batch, cfg.K + 1,
                    out.data_ptr(), s)
    assert e.value.status == 4
    big = torch.zeros((cfg.batch + 1, cfg.hidden), dtype=torch.bfloat16, device="cuda")
    lt1 = torch.zeros(cfg.batch + 1, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        head.draft(big, lt1, cache, 1)
    with pytest.raises(MtpError) as e:
        L.mtp_draft(head.handle, big.data_ptr(), lt1.data_ptr(), cache.kv, cfg.batch + 1, 1,
                    out.data_ptr(), s)
    assert e.value.status == 4
    assert L.LIB.mtp_draft(head.handle, hid.data_ptr(), lt.data_ptr(), ctypes.byref(cache.kv),
                           cfg.batch, -1, out.data_ptr(), s) == 2
    head.close()


def test_q8b_full_size_parity():
    """The Qwen3-8B-shaped head at its real sizes (bf16, H=4096, V=151936, L=4096, K=5)
    in the launch configuration the benchmark times, against the full oracle: tokens,
    hidden states, the max logit and every logit of every step."""
    cfg = S.get_config("q8b")
    inp = S.make_inputs(cfg, capacity=4096 + 64)
    g = run_draft(cfg, inp, cfg.K, want_logits=True)
    r = oracle_forced(cfg, inp, cfg.K, g["tokens"])
    n = compare_draft(cfg, r, g["tokens"], g["hidden"], g["top2"], g["logits"])
    assert n >= 4
    check_cache(cfg, inp, g, r, cfg.K, cfg.batch)


def test_q8b_cache_much_larger_than_its_contents():
    """The q8b head with a 32768-slot cache holding 4096 positions: the attention chunk is
    planned on the device from the lengths (not from the capacity), and the result still
    matches the oracle."""
    cfg = S.get_config("q8b")
    inp = S.make_inputs(cfg, capacity=32768)
    g = run_draft(cfg, inp, cfg.K, want_logits=False)
    r = oracle_forced(cfg, inp, cfg.K, g["tokens"])
    n = compare_draft(cfg, r, g["tokens"], g["hidden"], g["top2"])
    assert n >= 4
    check_cache(cfg, inp, g, r, cfg.K, cfg.batch)


@pytest.mark.parametrize("kind", ["one-long", "equal"])
def test_attention_chunks_from_the_length_spread(kind):
    """Many attention items on a bf16 cache, where each call's chunk comes from the sum and
    the spread of the lengths: one sequence of 3000 positions among 47 of 1-20 (its split
    count capped by the grid's five splits), and 80 equal lengths of 1000 (one item per kv
    head and sequence, a chunk longer than the grid was sized with). Both match the oracle."""
    B, L = (48, 3000) if kind == "one-long" else (80, 1000)
    cfg = small(name="spread-" + kind, cid=230 if kind == "one-long" else 231, hidden=256,
                n_q=16, n_kv=8, head_dim=64, ffn=512, vocab=2048, batch=B, K=2, ctx_lo=1,
                ctx_hi=20)
    inp = S.make_inputs(cfg, capacity=L + cfg.K + 7)
    if kind == "one-long":
        inp.lens[:] = 1 + (np.arange(B) * 7) % 20
        inp.lens[0] = L
    else:
        inp.lens[:] = L
    inp.pos[:] = inp.lens
    g = run_draft(cfg, inp, cfg.K)
    r = oracle_forced(cfg, inp, cfg.K, g["tokens"])
    n = compare_draft(cfg, r, g["tokens"], g["hidden"], g["top2"], g["logits"])
    assert n >= 0.5 * cfg.K * cfg.batch, f"only {n} tokens above the near-tie margin"
    check_cache(cfg, inp, g, r, cfg.K, cfg.batch)


@pytest.mark.parametrize("name", ["q8b-b32", "q32b", "wide"])
def test_batched_full_size_parity(name):
    """The batched workloads at their real sizes, in the launch configuration the
    benchmark times, against one oracle run over the whole batch: every sequence's
    tokens (bit-exact above the near-tie margin, teacher-forced), hidden states, max
    logits and every logit of every step, and every sequence's new cache slots."""
    cfg = S.get_config(name)
    lens = S.cache_lengths(cfg)
    inp = S.make_inputs(cfg, capacity=int(lens.max()) + cfg.K + 8)
    print(f"full-size batched parity: {name} B={cfg.batch} K={cfg.K}", flush=True)
    g = run_draft(cfg, inp, cfg.K, want_logits=True)
    r = oracle_forced(cfg, inp, cfg.K, g["tokens"])
    n = compare_draft(cfg, r, g["tokens"], g["hidden"], g["top2"], g["logits"])
    assert n >= cfg.batch * cfg.K // 2, f"only {n} tokens above the near-tie margin"
    check_cache(cfg, inp, g, r, cfg.K, cfg.batch)


def test_speculative_decoding_with_gpu_head_equals_greedy():
    """End to end: greedy speculative decoding driven by the GPU head and GPU verify
    emits exactly the synthetic target's plain greedy tokens."""
    from oracle.tiny_target import TinyTarget, speculative_greedy
    cfg = small(name="e2e", cid=140, hidden=128, n_q=4, n_kv=2, head_dim=64, ffn=256, vocab=8,
                batch=1, K=3, ctx_lo=8, ctx_hi=None, dtype="f32")
    inp = S.make_inputs(cfg, capacity=128)
    head, cache = make_head(cfg, inp)
    tgt = TinyTarget(cfg, S.target_weights(cfg, 2), inp.weights["embed"], inp.weights["lm_head"])
    prompt = S.prompt_tokens(cfg, 6)
    cache.pos.fill_(len(prompt) - 1)
    st = {}

    def draft_fn(h, last, K, _seq):
        out = head.draft(torch.from_numpy(np.asarray(h, np.float32)[None]).cuda(),
                         torch.tensor([last], dtype=torch.int32, device="cuda"), cache, K)
        st["d"] = out
        return out[0].cpu().numpy()

    def verify_fn(rows, d):
        a, n = head.verify(torch.from_numpy(rows[None].astype(np.float32)).cuda(), st["d"])
        st["a"] = a
        return int(a[0]), int(n[0])

    def rollback_fn(a):
        head.rollback(cache, st["a"], 3)

    out, acc = speculative_greedy(tgt, prompt, 32, draft_fn, verify_fn, rollback_fn, 3)
    assert out == tgt.greedy(prompt, 32)
    assert head.get_error() == 0
    head.close()
