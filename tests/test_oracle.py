"""Pins for the oracle: it is checked against values the pages print, closed forms,
library routines (torch, transformers), invariants and brute force — never against
a retyped copy of itself.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import mtp_synth as S
from oracle import mtp_oracle as O
from oracle.tiny_target import TinyTarget, lockstep_seqk, speculative_greedy

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_cfg(**kw):
    base = dict(name="pin", cid=20, hidden=64, n_q=4, n_kv=2, head_dim=16, ffn=96, vocab=50,
                batch=2, K=3, ctx_lo=5, ctx_hi=None, agree_lo=0.8, agree_hi=None, dtype="f32")
    base.update(kw)
    return S.Config(**base)


# ----------------------------------------------------------------------------- step weights

def test_step_weights_match_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "step_weights.json")))
    a = O.step_weights(g["beta"], g["K"])
    assert np.allclose(np.round(a, g["decimals"]), g["printed"], atol=0)


def test_step_weights_closed_form():
    # beta = 3/5: weights are 25/49, 15/49, 9/49.
    assert np.allclose(O.step_weights(0.6, 3), [25 / 49, 15 / 49, 9 / 49], rtol=1e-14)
    for beta, K in [(0.3, 5), (0.9, 7), (0.6, 1)]:
        a = O.step_weights(beta, K)
        assert abs(a.sum() - 1) < 1e-14 and np.all(np.diff(a) < 0) or K == 1
        assert np.allclose(a[1:] / a[:-1], beta)
    assert np.allclose(O.step_weights(1.0, 4), 0.25)


# ----------------------------------------------------------------------------- verify

def test_verify_golden_cases():
    g = json.load(open(os.path.join(GOLDEN, "verify_cases.json")))
    for c in g["cases"]:
        t = np.array(c["logits"], np.float32)[None]
        d = np.array(c["drafts"], np.int64).reshape(1, c["K"])
        a, n = O.verify(t, d)
        assert (int(a[0]), int(n[0])) == (c["accepted_len"], c["next_token"]), c["name"]


def _verify_by_definition(t, d):
    """Largest n <= K with d_i == argmax(row i-1) for every i <= n; bonus = argmax(row n)."""
    K = len(d)
    g = [int(np.flatnonzero(r == r.max())[0]) for r in t]
    best = max(n for n in range(K + 1) if all(d[i] == g[i] for i in range(n)))
    return best, g[best]


def test_verify_brute_force_small_vocab():
    rng = np.random.default_rng(1)
    Vs, K = 5, 3
    for trial in range(6):
        t = rng.integers(0, 4, size=(K + 1, Vs)).astype(np.float32)  # integer logits: many ties
        for d in itertools.product(range(Vs), repeat=K):
            a, n = O.verify(t[None], np.array(d)[None])
            assert (int(a[0]), int(n[0])) == _verify_by_definition(t, d)


def test_verify_bounds_forced_agreement_and_k0():
    rng = np.random.default_rng(2)
    B, K, V = 7, 5, 300
    d = rng.integers(0, V, size=(B, K))
    t = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    a, n = O.verify(t, d)
    tok = O.tokens_per_iteration(a)
    assert np.all((tok >= 1) & (tok <= K + 1))
    # Target forced to agree with every draft: all K accepted, K+1 tokens per iteration.
    t2 = t.copy()
    for b in range(B):
        for j in range(K):
            t2[b, j, d[b, j]] += 1e3
    a2, n2 = O.verify(t2, d)
    assert np.all(a2 == K) and np.all(O.tokens_per_iteration(a2) == K + 1)
    assert np.all(n2 == np.argmax(t2[:, K], axis=1))
    # K = 0: verification is the target's own greedy token of row 0.
    a0, n0 = O.verify(t[:, :1], np.zeros((B, 0), np.int64))
    assert np.all(a0 == 0) and np.all(n0 == np.argmax(t[:, 0], axis=1))


@pytest.mark.parametrize("name,K,p,agree_hi,B,V,iters", [
    ("tiny-like", 3, 0.8, None, 1, 4096, 2500),
    ("b32-like", 3, 0.6, None, 32, 2048, 100),
    ("q8b-like", 5, 0.9, None, 1, 4096, 2500),
    ("q32b-like", 5, 0.5, 0.95, 8, 2048, 300),
])
def test_planted_acceptance_closed_form(name, K, p, agree_hi, B, V, iters):
    """With planted agreement p per position, E[tokens / iteration] = 1 + sum_{n=1..K} p^n
    (up to the 1/V chance agreement and the rare bump failure)."""
    cfg = small_cfg(cid=30 + K, batch=B, vocab=V, K=K, agree_lo=p, agree_hi=agree_hi)
    pb = S.agreement(cfg)
    rng = np.random.default_rng(3)
    tot = []
    for it in range(iters):
        d = rng.integers(0, V, size=(B, K))
        t = S.plant_target_logits(cfg, d, it)
        a, _ = O.verify(t, d)
        tot.append(O.tokens_per_iteration(a))
    tot = np.concatenate(tot).astype(np.float64)
    expect = np.mean([1 + sum(q ** n for n in range(1, K + 1)) for q in pb])
    se = tot.std() / math.sqrt(tot.size)
    assert abs(tot.mean() - expect) < 4 * se + 2e-3, (tot.mean(), expect, se)


# ----------------------------------------------------------------------------- building blocks

def test_rmsnorm_and_silu_match_torch():
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 256)).astype(np.float32) * 3
    g = (1 + 0.02 * rng.standard_normal(256)).astype(np.float32)
    ref = F.rms_norm(torch.from_numpy(x), (256,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.max(np.abs(O.rmsnorm(x, g, 1e-6) - ref)) < 2e-6
    ref = F.silu(torch.from_numpy(x)).numpy()
    assert np.max(np.abs(O.silu(x) - ref)) < 2e-6


def test_attention_matches_torch_sdpa_gqa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    nq, nkv, d, T = 8, 2, 64, 37
    q = rng.standard_normal((nq, d)).astype(np.float32)
    k = rng.standard_normal((nkv, T, d)).astype(np.float32)
    v = rng.standard_normal((nkv, T, d)).astype(np.float32)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        enable_gqa=True)[0, :, 0].numpy()
    assert np.max(np.abs(O.gqa_attention(q, k, v) - ref)) < 2e-6


def test_attention_special_cases():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 16)).astype(np.float32)
    k = rng.standard_normal((2, 1, 16)).astype(np.float32)
    v = rng.standard_normal((2, 1, 16)).astype(np.float32)
    o = O.gqa_attention(q, k, v)          # one slot: output is that slot's value
    assert np.array_equal(o[:2], np.repeat(v[0], 2, 0)) and np.array_equal(o[2:], np.repeat(v[1], 2, 0))
    k = np.repeat(rng.standard_normal((2, 1, 16)).astype(np.float32), 9, axis=1)
    v = rng.standard_normal((2, 9, 16)).astype(np.float32)
    o = O.gqa_attention(q, k, v)          # identical keys: uniform weights, mean of V
    assert np.allclose(o[0], v[0].mean(0), atol=1e-6) and np.allclose(o[3], v[1].mean(0), atol=1e-6)


def test_rope_invariants_and_transformers_tables():
    d, theta = 128, 1e6
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, d)).astype(np.float64)
    c0, s0 = O.rope_tables(0, d, theta, np.float64)
    assert np.array_equal(O.rope(x, c0, s0), x)
    for p1, p2 in [(1, 2), (17, 4096), (30000, 2768)]:
        c1, s1 = O.rope_tables(p1, d, theta, np.float64)
        c2, s2 = O.rope_tables(p2, d, theta, np.float64)
        c3, s3 = O.rope_tables(p1 + p2, d, theta, np.float64)
        y = O.rope(O.rope(x, c1, s1), c2, s2)
        assert np.allclose(y, O.rope(x, c3, s3), atol=1e-9)
        r = O.rope(x, c1, s1)
        h = d // 2
        assert np.allclose(r[:, :h] ** 2 + r[:, h:] ** 2, x[:, :h] ** 2 + x[:, h:] ** 2)
    # Element i of the first half pairs with element i + d/2 at frequency theta^(-2i/d).
    c, s = O.rope_tables(3, d, theta, np.float64)
    assert np.isclose(c[0], math.cos(3.0)) and np.isclose(s[1], math.sin(3.0 * theta ** (-2 / d)))
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers.models.llama.modeling_llama")
    lc = tr.LlamaConfig(hidden_size=1024, num_attention_heads=8, head_dim=d, rope_theta=theta)
    cos, sin = tr.LlamaRotaryEmbedding(lc)(torch.zeros(1, 1, 1), torch.tensor([[5, 100]]))
    for i, p in enumerate([5, 100]):
        c, s = O.rope_tables(p, d, theta)
        assert np.allclose(cos[0, i, :h].numpy(), c, atol=2e-5)
        assert np.allclose(sin[0, i, h:].numpy(), s, atol=2e-5)


# ----------------------------------------------------------------------------- whole step

def _inputs(cfg, cap=None):
    return S.make_inputs(cfg, capacity=cap)


@pytest.mark.parametrize("case", ["tiny", "bf16"])
def test_decoder_step_matches_transformers_llama_layer(case):
    """Steps 3-9 of one draft step against transformers' Llama decoder layer (a standard
    pre-norm GQA/RoPE/SwiGLU block with no biases) fed by torch's own RMSNorm / linear.
    For a bf16 head the new cache entries must be torch's round-to-nearest-even bf16 of
    the layer's rotated keys and values."""
    torch = pytest.importorskip("torch")
    tr = pytest.importorskip("transformers.models.llama.modeling_llama")
    from transformers.cache_utils import DynamicCache
    F = torch.nn.functional
    if case == "tiny":
        cfg = S.get_config("tiny")
        cap = 140
    else:
        cfg = small_cfg(cid=70, hidden=128, n_q=4, n_kv=2, head_dim=64, ffn=256, vocab=300,
                        batch=1, K=1, ctx_lo=37, dtype="bf16")
        cap = 48
    inp = _inputs(cfg, cap)
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    res = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, 1)

    def f32(a):
        return torch.from_numpy(O.as_float(a, cfg.dtype).copy())

    w = {k: f32(v) for k, v in inp.weights.items()}
    H, L = cfg.hidden, int(inp.lens[0])
    h = f32(inp.hidden)
    e = w["embed"][torch.from_numpy(inp.last_tokens.astype(np.int64))]
    cat = torch.cat([F.rms_norm(h, (H,), w["g_h"], 1e-6), F.rms_norm(e, (H,), w["g_e"], 1e-6)], 1)
    x = F.linear(cat, w["w_eh"])
    lc = tr.LlamaConfig(hidden_size=H, intermediate_size=cfg.ffn, num_attention_heads=cfg.n_q,
                        num_key_value_heads=cfg.n_kv, head_dim=cfg.head_dim, rms_norm_eps=1e-6,
                        rope_theta=cfg.rope_theta, attention_bias=False, mlp_bias=False,
                        num_hidden_layers=1, vocab_size=cfg.vocab)
    lc._attn_implementation = "eager"
    layer = tr.LlamaDecoderLayer(lc, 0)
    sd = {"self_attn.q_proj.weight": w["w_q"], "self_attn.k_proj.weight": w["w_k"],
          "self_attn.v_proj.weight": w["w_v"], "self_attn.o_proj.weight": w["w_o"],
          "mlp.gate_proj.weight": w["w_gate"], "mlp.up_proj.weight": w["w_up"],
          "mlp.down_proj.weight": w["w_down"], "input_layernorm.weight": w["g_attn"],
          "post_attention_layernorm.weight": w["g_mlp"]}
    layer.load_state_dict(sd)
    cache = DynamicCache(config=lc)
    cache.update(f32(inp.k_cache[:, :, :L]), f32(inp.v_cache[:, :, :L]), 0)
    P = int(inp.pos[0])
    cos, sin = tr.LlamaRotaryEmbedding(lc)(x[None], torch.tensor([[P]]))
    with torch.no_grad():
        x2 = layer(x[None], position_ids=torch.tensor([[P]]), past_key_values=cache,
                   use_cache=True, position_embeddings=(cos, sin))[0]
        logits = F.linear(F.rms_norm(x2, (H,), w["g_final"], 1e-6), w["lm_head"])
    newk = cache.layers[0].keys[0, :, L]
    newv = cache.layers[0].values[0, :, L]
    if cfg.dtype == "f32":
        # The pinned cache attends to the new entry in fp32; the layer's output matches.
        assert np.max(np.abs(res["hidden_steps"][0] - x2.numpy())) < 1e-4
        assert np.max(np.abs(res["logits"][0] - logits.numpy())) < 1e-4
        assert np.max(np.abs(kc[0, :, L] - newk.numpy())) < 1e-5
        assert np.max(np.abs(vc[0, :, L] - newv.numpy())) < 1e-6
        assert int(res["draft_tokens"][0, 0]) == int(torch.argmax(logits[0]))
    else:
        # bf16 cache: the oracle attends to rounded entries, the layer to fp32 ones; the
        # written entries are the nearest bf16 (ties to even) of the layer's values.
        for mine, ref in ((kc[0, :, L], newk), (vc[0, :, L], newv)):
            want = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            same = np.mean(mine == want)
            ulp = np.abs(mine.astype(np.int32) - want.astype(np.int32))
            assert same > 0.98 and ulp.max() <= 1, (same, ulp.max())
        assert np.max(np.abs(res["hidden_steps"][0] - x2.numpy())) < 2e-2


def test_identity_projection_pins():
    """W_eh = [I, 0] / [0, I] and zero W_o, W_d make the step's hidden output the
    normalised verifier state / normalised embedding: pins the concat order, the
    separate gains and both residual paths."""
    cfg = small_cfg()
    inp = _inputs(cfg, 20)
    H = cfg.hidden
    for half in (0, 1):
        w = dict(inp.weights)
        eye = np.zeros((H, 2 * H), np.float32)
        eye[:, half * H:(half + 1) * H] = np.eye(H, dtype=np.float32)
        w["w_eh"] = eye
        w["w_o"] = np.zeros_like(w["w_o"])
        w["w_down"] = np.zeros_like(w["w_down"])
        W = O.OracleWeights(cfg, w)
        r = O.draft(cfg, W, inp.hidden, inp.last_tokens, inp.k_cache.copy(), inp.v_cache.copy(),
                    inp.lens, inp.pos, 1)
        src = inp.hidden if half == 0 else w["embed"][inp.last_tokens]
        g = w["g_h"] if half == 0 else w["g_e"]
        ms = np.mean(src.astype(np.float64) ** 2, axis=1, keepdims=True)
        expect = src / np.sqrt(ms + 1e-6) * g
        assert np.max(np.abs(r["hidden_steps"][0] - expect)) < 1e-5


def test_recursion_consumes_previous_token_and_hidden():
    """Step k+1 equals a fresh 1-step draft started from (h^(k), d_k) at pos+k, len+k.
    The restart hands h^(k) over in the storage dtype (fp32 here), which is lossless
    when the oracle itself runs in fp32."""
    cfg = small_cfg()
    inp = _inputs(cfg, 20)
    W = O.OracleWeights(cfg, inp.weights, np.float32)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, 3)
    kc2, vc2 = inp.k_cache.copy(), inp.v_cache.copy()
    r1 = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc2, vc2, inp.lens, inp.pos, 1)
    r2 = O.draft(cfg, W, r1["hidden_steps"][0], r1["draft_tokens"][:, 0], kc2, vc2,
                 r1["lens"], r1["pos"], 2)
    assert np.array_equal(r["draft_tokens"][:, 1:], r2["draft_tokens"])
    assert np.allclose(r["hidden_steps"][1:], r2["hidden_steps"], atol=1e-6)
    assert np.array_equal(kc, kc2)


def test_fp64_rerun_bounds_oracle_rounding():
    cfg = S.get_config("tiny")
    inp = _inputs(cfg, 140)
    r32 = O.draft(cfg, O.OracleWeights(cfg, inp.weights), inp.hidden, inp.last_tokens,
                  inp.k_cache.copy(), inp.v_cache.copy(), inp.lens, inp.pos, 3,
                  force_tokens=None)
    r64 = O.draft(cfg, O.OracleWeights(cfg, inp.weights, np.float64), inp.hidden, inp.last_tokens,
                  inp.k_cache.copy(), inp.v_cache.copy(), inp.lens, inp.pos, 3,
                  force_tokens=r32["draft_tokens"])
    assert np.max(np.abs(r32["hidden_steps"] - r64["hidden_steps"])) < 1e-5
    assert np.max(np.abs(r32["logits"] - r64["logits"])) < 1e-5


def test_rollback_is_truncation():
    """Drafting K steps then rolling back to accepted length a leaves the cache state a
    min(a+1, K)-step draft would have left; pos moves to the last verified input."""
    cfg = small_cfg(K=4)
    inp = _inputs(cfg, 30)
    W = O.OracleWeights(cfg, inp.weights)
    K = 4
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, K)
    for a in range(K + 1):
        acc = np.full(cfg.batch, a)
        ln, ps = O.kv_rollback(r["lens"], r["pos"], acc, K)
        assert np.all(ln - inp.lens == min(a + 1, K)) and np.all(ps - inp.pos == a + 1)
        kt, vt = inp.k_cache.copy(), inp.v_cache.copy()
        rt = O.draft(cfg, W, inp.hidden, inp.last_tokens, kt, vt, inp.lens, inp.pos, min(a + 1, K))
        assert np.array_equal(rt["lens"], ln)
        for b in range(cfg.batch):
            assert np.array_equal(kc[b, :, :ln[b]], kt[b, :, :ln[b]])
            assert np.array_equal(vc[b, :, :ln[b]], vt[b, :, :ln[b]])
    ln0, ps0 = O.kv_rollback(inp.lens, inp.pos, np.zeros(cfg.batch), 0)
    assert np.array_equal(ln0, inp.lens) and np.array_equal(ps0, inp.pos + 1)


def test_poisoned_stale_slots_do_not_leak():
    cfg = small_cfg()
    inp = _inputs(cfg, 20)
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    for b in range(cfg.batch):
        kc[b, :, inp.lens[b]:] = np.nan
        vc[b, :, inp.lens[b]:] = np.nan
    r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, 3)
    r0 = O.draft(cfg, W, inp.hidden, inp.last_tokens, inp.k_cache.copy(), inp.v_cache.copy(),
                 inp.lens, inp.pos, 3)
    assert np.all(np.isfinite(r["hidden_steps"]))
    assert np.array_equal(r["hidden_steps"], r0["hidden_steps"])


def test_bf16_cache_entries_are_rounded_on_write():
    cfg = small_cfg(dtype="bf16")
    inp = _inputs(cfg, 20)
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, 2)
    assert kc.dtype == np.uint16
    w = O.OracleWeights(cfg, inp.weights, np.float64)
    r64 = O.draft(cfg, w, inp.hidden, inp.last_tokens, inp.k_cache.copy(), inp.v_cache.copy(),
                  inp.lens, inp.pos, 2, force_tokens=r["draft_tokens"])
    assert np.max(np.abs(r["hidden_steps"] - r64["hidden_steps"])) < 2e-3


# ----------------------------------------------------------------------------- end to end

@pytest.mark.parametrize("vocab,cache_len", [(4096, 0), (8, 0), (8, 8)])
def test_speculative_equals_greedy(vocab, cache_len):
    """Greedy speculative decoding with the oracle head emits exactly the target's plain
    greedy tokens (a tiny random 2-layer target sharing E and W_lm with the head)."""
    cfg = small_cfg(cid=40 + vocab + cache_len, batch=1, vocab=vocab, ctx_lo=cache_len, K=3)
    inp = _inputs(cfg, 256)
    W = O.OracleWeights(cfg, inp.weights)
    tgt = TinyTarget(cfg, S.target_weights(cfg, 2), inp.weights["embed"], inp.weights["lm_head"])
    prompt = S.prompt_tokens(cfg, 6)
    n_new = 40
    ref = tgt.greedy(prompt, n_new)
    st = {"kc": inp.k_cache.copy(), "vc": inp.v_cache.copy(),
          "len": np.array([cache_len]), "pos": np.array([len(prompt) - 1])}

    def draft_fn(h, last, K, _seq):
        r = O.draft(cfg, W, np.asarray(h, np.float32)[None], np.array([last]), st["kc"], st["vc"],
                    st["len"], st["pos"], K)
        st["len"], st["pos"] = r["lens"], r["pos"]
        return r["draft_tokens"][0]

    def rollback_fn(a):
        st["len"], st["pos"] = O.kv_rollback(st["len"], st["pos"], np.array([a]), 3)

    def verify_fn(rows, d):
        a, n = O.verify(rows[None], np.asarray(d)[None])
        return a[0], n[0]

    out, acc = speculative_greedy(tgt, prompt, n_new, draft_fn, verify_fn, rollback_fn, 3)
    assert out == ref
    assert all(0 <= a <= 3 for a in acc)


@pytest.mark.parametrize("vocab,cache_len", [(4096, 0), (8, 8)])
def test_speculative_from_hidden_states_equals_greedy(vocab, cache_len):
    """Verification from the target's hidden states (its final norm and the shared
    lm_head applied by the verifier) also reproduces plain greedy decoding exactly."""
    cfg = small_cfg(cid=70 + vocab + cache_len, batch=1, vocab=vocab, ctx_lo=cache_len, K=3)
    inp = _inputs(cfg, 256)
    W = O.OracleWeights(cfg, inp.weights)
    tw = S.target_weights(cfg, 2)
    tgt = TinyTarget(cfg, tw, inp.weights["embed"], inp.weights["lm_head"])
    prompt = S.prompt_tokens(cfg, 6)
    ref = tgt.greedy(prompt, 40)
    st = {"kc": inp.k_cache.copy(), "vc": inp.v_cache.copy(),
          "len": np.array([cache_len]), "pos": np.array([len(prompt) - 1])}

    def draft_fn(h, last, K, _seq):
        r = O.draft(cfg, W, np.asarray(h, np.float32)[None], np.array([last]), st["kc"], st["vc"],
                    st["len"], st["pos"], K)
        st["len"], st["pos"] = r["lens"], r["pos"]
        return r["draft_tokens"][0]

    def rollback_fn(a):
        st["len"], st["pos"] = O.kv_rollback(st["len"], st["pos"], np.array([a]), 3)

    def verify_fn(hid_rows, d):
        a, n, _ = O.verify_from_hidden(cfg, hid_rows[None], tw["g_final"], inp.weights["lm_head"],
                                       np.asarray(d)[None])
        return a[0], n[0]

    out, acc = speculative_greedy(tgt, prompt, 40, draft_fn, verify_fn, rollback_fn, 3,
                                  from_hidden=True)
    assert out == ref
    assert all(0 <= a <= 3 for a in acc)


def test_adapt_k_golden_cases():
    """The adaptive-length rule against hand-worked cases (cited in the fixture)."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "adapt_k_cases.json")))
    for c in gold["cases"]:
        assert O.adapt_k(c["accepted"], c["K"], c["k_min"], c["k_max"]) == c["k_next"], c


def test_speculative_with_adaptive_k_equals_greedy():
    """Changing K every iteration (draft, verify and rollback all follow it) keeps greedy
    speculative decoding exactly equal to plain greedy decoding, and K moves."""
    cfg = small_cfg(cid=80, batch=1, vocab=8, ctx_lo=4, K=3)
    inp = _inputs(cfg, 512)
    W = O.OracleWeights(cfg, inp.weights)
    tgt = TinyTarget(cfg, S.target_weights(cfg, 2), inp.weights["embed"], inp.weights["lm_head"])
    prompt = S.prompt_tokens(cfg, 6)
    ref = tgt.greedy(prompt, 60)
    st = {"kc": inp.k_cache.copy(), "vc": inp.v_cache.copy(),
          "len": np.array([4]), "pos": np.array([len(prompt) - 1]), "K": 2, "ks": []}

    def draft_fn(h, last, K, _seq):
        st["K"] = K
        st["ks"].append(K)
        r = O.draft(cfg, W, np.asarray(h, np.float32)[None], np.array([last]), st["kc"], st["vc"],
                    st["len"], st["pos"], K)
        st["len"], st["pos"] = r["lens"], r["pos"]
        return r["draft_tokens"][0]

    def rollback_fn(a):
        st["len"], st["pos"] = O.kv_rollback(st["len"], st["pos"], np.array([a]), st["K"])

    def verify_fn(rows, d):
        a, n = O.verify(rows[None], np.asarray(d)[None])
        return a[0], n[0]

    out, acc = speculative_greedy(tgt, prompt, 60, draft_fn, verify_fn, rollback_fn, 2,
                                  next_k=lambda a, K: O.adapt_k([a], K, 1, 6))
    assert out == ref
    assert len(set(st["ks"])) > 1


def _catchup_run(cfg, inp, W, tgt, prompt, n_new, K0, next_k, bad_at, init=None):
    """Greedy speculative decoding with exact catch-up. The head runs every draft step
    (writing its cache) teacher-forced on the target's own greedy continuation with one
    planted error at index bad_at(iteration, K) (none when that is K, so all K drafts are
    accepted). init: the head's starting cache state (default: empty, at the position of
    the prompt's last token). Returns the emitted tokens, accepted lengths and the head's
    cache state."""
    st = {"kc": np.zeros_like(inp.k_cache), "vc": np.zeros_like(inp.v_cache),
          "len": np.array([0]), "pos": np.array([len(prompt) - 1]), "it": 0}
    if init is not None:
        st.update(init)

    def draft_fn(h, last, K, seq):
        cont = tgt.greedy(seq, K)
        bad = bad_at(st["it"], K)
        st["it"] += 1
        if bad < K:
            cont[bad] = (cont[bad] + 1) % cfg.vocab
        st["K"] = K
        r = O.draft(cfg, W, np.asarray(h, np.float32)[None], np.array([last]), st["kc"], st["vc"],
                    st["len"], st["pos"], K, force_tokens=np.array([cont]))
        st["len"], st["pos"], st["d"] = r["lens"], r["pos"], np.array([cont])
        return cont

    def verify_fn(hid_rows, d):
        st["hid"] = hid_rows
        a, n, _ = O.verify_from_hidden(cfg, hid_rows[None], tgt_norm, inp.weights["lm_head"],
                                       np.asarray(d)[None])
        return a[0], n[0]

    def commit_fn(a):
        st["len"], st["pos"] = O.kv_catchup(cfg, W, st["hid"][None], st["d"], np.array([a]),
                                            st["kc"], st["vc"], st["len"], st["pos"], st["K"])

    tgt_norm = tgt.g_final_store
    out, acc = speculative_greedy(tgt, prompt, n_new, draft_fn, verify_fn, commit_fn, K0,
                                  from_hidden=True, next_k=next_k)
    return out, acc, st


def test_exact_catchup_cache_is_independent_of_the_speculation_schedule():
    """With exact catch-up every committed slot holds the layer's K/V of (the verifier's
    hidden state, the next committed token) at its position, so the cache over the
    committed prefix depends only on the committed tokens: two different speculative
    schedules leave identical caches, both equal to slots written one position at a time
    by single-step drafts from the target's own hidden states, and the output is still
    plain greedy decoding."""
    cfg = small_cfg(cid=90, batch=1, vocab=16, ctx_lo=0, K=4)
    inp = _inputs(cfg, 256)
    W = O.OracleWeights(cfg, inp.weights)
    tw = S.target_weights(cfg, 2)
    tgt = TinyTarget(cfg, tw, inp.weights["embed"], inp.weights["lm_head"])
    tgt.g_final_store = tw["g_final"]
    prompt = S.prompt_tokens(cfg, 6)
    n_new = 40
    ref = tgt.greedy(prompt, n_new)
    out1, acc1, s1 = _catchup_run(cfg, inp, W, tgt, prompt, n_new, 3, None,
                                  lambda it, K: it % (K + 1))
    out2, acc2, s2 = _catchup_run(cfg, inp, W, tgt, prompt, n_new, 2,
                                  lambda a, K: O.adapt_k([a], K, 1, 5),
                                  lambda it, K: K if it % 3 else it % K)
    assert out1 == ref and out2 == ref
    assert 3 in acc1 and 0 in acc1 and len(set(acc2)) > 1  # includes the a = K gap
    n = min(int(s1["len"][0]), int(s2["len"][0]))
    assert n > 20
    assert np.array_equal(s1["kc"][:, :, :n], s2["kc"][:, :, :n])
    assert np.array_equal(s1["vc"][:, :, :n], s2["vc"][:, :, :n])
    # reference: slot s is written by a one-step draft at position len(prompt)-1+s from
    # the target's hidden state there and the token after it
    seq = list(prompt) + ref
    hid, _ = tgt.forward(seq)
    kc, vc = np.zeros_like(inp.k_cache), np.zeros_like(inp.v_cache)
    for slot in range(n):
        p = len(prompt) - 1 + slot
        O.draft(cfg, W, hid[p][None], np.array([seq[p + 1]]), kc, vc, np.array([slot]),
                np.array([p]), 1)
    assert np.allclose(s1["kc"][:, :, :n], kc[:, :, :n], rtol=0, atol=1e-5)
    assert np.allclose(s1["vc"][:, :, :n], vc[:, :, :n], rtol=0, atol=1e-5)


def test_speculative_equals_greedy_with_scripted_drafts():
    """A drafter that proposes the target's own greedy continuation with one planted
    error at index i (or none) must be accepted for exactly i tokens, and the output
    must still equal plain greedy decoding."""
    cfg = small_cfg(cid=60, batch=1, vocab=16, K=4)
    inp = _inputs(cfg, 64)
    tgt = TinyTarget(cfg, S.target_weights(cfg, 2), inp.weights["embed"], inp.weights["lm_head"])
    prompt = S.prompt_tokens(cfg, 5)
    ref = tgt.greedy(prompt, 30)
    K = 4
    it = {"n": 0}

    def draft_fn(h, last, K_, seq):
        cont = tgt.greedy(seq, K_)
        bad = it["n"] % (K_ + 1)
        it["n"] += 1
        if bad < K_:
            cont[bad] = (cont[bad] + 1) % cfg.vocab
        return cont

    def verify_fn(rows, d):
        a, n = O.verify(rows[None], np.asarray(d)[None])
        return a[0], n[0]

    out, acc = speculative_greedy(tgt, prompt, 30, draft_fn, verify_fn, lambda a: None, K)
    assert out == ref
    assert acc == [i % (K + 1) for i in range(len(acc))]


# ----------------------------------------------------------------------------- prompt prefill

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_equals_one_step_drafts(dtype):
    """Prefill writes, for each prompt position s, the slot a one-step draft at s would
    write from the same pair (verifier hidden state h_s, token x_{s+1}): the layer's input
    side only, at RoPE position pos+s, slot len+s. Ragged counts leave the rows past a
    sequence's count unread (NaN there changes nothing) and its later slots untouched."""
    cfg = small_cfg(cid=93, batch=3, ctx_lo=4, ctx_hi=9, dtype=dtype)
    n = 7
    inp = _inputs(cfg, 40)
    W = O.OracleWeights(cfg, inp.weights)
    th = S.prefill_hidden(cfg, n)
    tok = S.prefill_tokens(cfg, n)
    nv = np.array([n, n - 3, 0])
    th_p = th.copy()
    if dtype == "bf16":
        th_p[1, n - 3:] = 0x7FC0
    else:
        th_p[1, n - 3:] = np.nan
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    pos0 = inp.pos + 11
    ln, ps = O.kv_prefill(cfg, W, th_p, tok, kc, vc, inp.lens, pos0, nv)
    assert np.array_equal(ln, inp.lens + nv) and np.array_equal(ps, pos0 + nv)
    rk, rv = inp.k_cache.copy(), inp.v_cache.copy()
    for b in range(cfg.batch):
        for s_ in range(int(nv[b])):
            O.draft(cfg, W, th[b:b + 1, s_], tok[b:b + 1, s_], rk[b:b + 1], rv[b:b + 1],
                    inp.lens[b:b + 1] + s_, pos0[b:b + 1] + s_, 1)
    for got, ref in ((kc, rk), (vc, rv)):
        if dtype == "bf16":
            # one-ulp rounding flips are allowed between the two evaluation orders
            g, r = O.as_float(got, "bf16"), O.as_float(ref, "bf16")
            assert np.allclose(g, r, rtol=2 ** -7, atol=1e-6)
        else:
            assert np.allclose(got, ref, rtol=0, atol=1e-6)
        for b in range(cfg.batch):
            L1 = int(inp.lens[b] + nv[b])
            assert np.array_equal(got[b, :, L1:], getattr(inp, "k_cache" if got is kc else
                                                          "v_cache")[b, :, L1:])


def test_prefill_then_exact_decoding_equals_prefill_of_the_committed_sequence():
    """From an empty cache, prefilling the prompt and then decoding speculatively with
    exact catch-up emits plain greedy decoding, and leaves the same cache as prefilling the
    whole committed sequence at once: slot s holds the pair (h_s, x_{s+1}) at position s
    whichever way the slot was written."""
    cfg = small_cfg(cid=94, batch=1, vocab=16, ctx_lo=0, K=4)
    inp = _inputs(cfg, 256)
    W = O.OracleWeights(cfg, inp.weights)
    tw = S.target_weights(cfg, 2)
    tgt = TinyTarget(cfg, tw, inp.weights["embed"], inp.weights["lm_head"])
    tgt.g_final_store = tw["g_final"]
    prompt = [int(x) for x in S.prompt_tokens(cfg, 9)]
    P = len(prompt)
    hid, _ = tgt.forward(prompt)
    kc, vc = np.zeros_like(inp.k_cache), np.zeros_like(inp.v_cache)
    ln, ps = O.kv_prefill(cfg, W, hid[None, :P - 1], np.array([prompt[1:]]), kc, vc,
                          np.array([0]), np.array([0]))
    assert int(ln[0]) == P - 1 and int(ps[0]) == P - 1
    n_new = 30
    ref = tgt.greedy(prompt, n_new)
    out, acc, st = _catchup_run(cfg, inp, W, tgt, prompt, n_new, 3, None,
                                lambda it, K: it % (K + 1),
                                init={"kc": kc, "vc": vc, "len": ln, "pos": ps})
    assert out == ref
    assert 3 in acc and 0 in acc
    n = int(st["len"][0])
    assert n > P + 10 and int(st["pos"][0]) == n
    seq = prompt + ref
    hid_all, _ = tgt.forward(seq)
    rk, rv = np.zeros_like(inp.k_cache), np.zeros_like(inp.v_cache)
    O.kv_prefill(cfg, W, hid_all[None, :n], np.array([seq[1:n + 1]]), rk, rv, np.array([0]),
                 np.array([0]))
    assert np.allclose(st["kc"][:, :, :n], rk[:, :, :n], rtol=0, atol=1e-5)
    assert np.allclose(st["vc"][:, :, :n], rv[:, :, :n], rtol=0, atol=1e-5)


# ----------------------------------------------------------------------------- per-sequence K

def test_adapt_k_seq_golden_cases():
    """The per-sequence window rule against hand-worked cases (cited in the fixture)."""
    gold = json.load(open(os.path.join(GOLDEN, "adapt_k_seq_cases.json")))
    for c in gold["cases"]:
        got = O.adapt_k_seq(c["accepted"], c["k"], c["k_min"], c["k_max"])
        assert got.tolist() == c["k_next"], c


def test_verify_seqk_reads_only_the_sequence_rows():
    """Target rows past k_b and drafts past k_b do not matter (poisoned with NaN and
    out-of-range ids); k_b = K for every sequence is the uniform verification; brute force
    over every draft in [0,4)^k_b for each k_b <= 3 against the definition."""
    rng = np.random.default_rng(7)
    B, K, V = 6, 3, 4
    t = rng.normal(size=(B, K + 1, V)).astype(np.float32)
    d = rng.integers(0, V, size=(B, K))
    ks = np.array([0, 1, 2, 3, 3, 1])
    tp, dp = t.copy(), d.copy()
    for b in range(B):
        tp[b, ks[b] + 1:] = np.nan
        dp[b, ks[b]:] = -1
    a1, n1 = O.verify_seqk(t, d, ks)
    a2, n2 = O.verify_seqk(tp, dp, ks)
    assert np.array_equal(a1, a2) and np.array_equal(n1, n2)
    assert np.all(a1 <= ks) and np.all(a1 >= 0)
    a3, n3 = O.verify_seqk(t, d, np.full(B, K))
    a4, n4 = O.verify(t, d)
    assert np.array_equal(a3, a4) and np.array_equal(n3, n4)
    for kb in range(K + 1):
        for dd in itertools.product(range(V), repeat=kb):
            dr = np.full((1, K), -1)
            dr[0, :kb] = dd
            a, n = O.verify_seqk(t[:1], dr, np.array([kb]))
            g = [int(np.argmax(t[0, j])) for j in range(K + 1)]
            ref = 0
            while ref < kb and dd[ref] == g[ref]:
                ref += 1
            assert a[0] == ref and n[0] == g[ref]


def test_seqk_draft_and_rollback_is_per_sequence_truncation():
    """Drafting k_b steps per sequence then rolling back to a_b leaves, for every sequence,
    the cache a fresh min(a_b+1, k_b)-step draft of that sequence alone would leave, and
    sequences with k_b = 0 are untouched except pos += 1 after rollback."""
    cfg = small_cfg(K=4, batch=4)
    inp = _inputs(cfg, 30)
    W = O.OracleWeights(cfg, inp.weights)
    ks = np.array([4, 0, 2, 1])
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft_seqk(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, ks, 4)
    assert np.array_equal(r["lens"], inp.lens + ks) and np.array_equal(r["pos"], inp.pos + ks)
    assert np.all(r["draft_tokens"][1] == -1) and np.all(r["draft_tokens"][3, 1:] == -1)
    a = np.array([2, 0, 2, 0])
    ln, ps = O.kv_rollback_seqk(r["lens"], r["pos"], a, ks)
    assert np.array_equal(ln - inp.lens, np.minimum(a + 1, ks))
    assert np.array_equal(ps - inp.pos, a + 1)
    for b in range(cfg.batch):
        kt, vt = inp.k_cache[b:b + 1].copy(), inp.v_cache[b:b + 1].copy()
        m = int(min(a[b] + 1, ks[b]))
        if m:
            rt = O.draft(cfg, W, inp.hidden[b:b + 1], inp.last_tokens[b:b + 1], kt, vt,
                         inp.lens[b:b + 1], inp.pos[b:b + 1], m)
            assert np.array_equal(rt["draft_tokens"][0], r["draft_tokens"][b, :m])
        assert np.array_equal(kc[b, :, :ln[b]], kt[0, :, :ln[b]])
        assert np.array_equal(vc[b, :, :ln[b]], vt[0, :, :ln[b]])
        # slots past the sequence's own draft are untouched
        assert np.array_equal(kc[b, :, inp.lens[b] + ks[b]:],
                              inp.k_cache[b, :, inp.lens[b] + ks[b]:])


def test_speculative_with_per_sequence_k_equals_greedy():
    """Each sequence of a batch drafts, verifies and rolls back with its own length, which
    the window rule moves every iteration; every sequence still emits exactly its plain
    greedy decoding, and the lengths differ across sequences and iterations."""
    cfg = small_cfg(cid=95, batch=3, vocab=2, ctx_lo=4, K=3)
    inp = _inputs(cfg, 512)
    W = O.OracleWeights(cfg, inp.weights)
    tgt = TinyTarget(cfg, S.target_weights(cfg, 2), inp.weights["embed"], inp.weights["lm_head"])
    prompts = [S.prompt_tokens(cfg, 5 + b, sub=b) for b in range(cfg.batch)]
    st = {"kc": inp.k_cache.copy(), "vc": inp.v_cache.copy(), "len": inp.lens.copy(),
          "pos": np.array([len(p) - 1 for p in prompts])}

    def draft(h, last, k, k_max):
        r = O.draft_seqk(cfg, W, h, last, st["kc"], st["vc"], st["len"], st["pos"], k, k_max)
        st["len"], st["pos"] = r["lens"], r["pos"]
        return r["draft_tokens"]

    def verify(rows, d, k):
        return O.verify_seqk(rows, d, k)

    def rollback(a, k):
        st["len"], st["pos"] = O.kv_rollback_seqk(st["len"], st["pos"], a, k)

    out, kh = lockstep_seqk(tgt, prompts, 40, 2, 3, 0, 5, draft, verify, rollback,
                            O.adapt_k_seq)
    for b in range(cfg.batch):
        assert out[b] == tgt.greedy(prompts[b], 40), b
    assert len(set(kh.reshape(-1).tolist())) > 2
    assert any(len(set(row.tolist())) > 1 for row in kh)   # lengths differ within a batch
