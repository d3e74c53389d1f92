"""Speculative length per sequence (mtp_draft_seqk, mtp_verify_seqk, mtp_kv_rollback_seqk):
HIP path against the oracle and against the uniform-length path, and GPU decoding with the
per-sequence window rule equal to plain greedy decoding."""
import numpy as np
import pytest

import mtp_synth as S
from gpu_util import MARGIN, cache_to_np, make_head, small, to_dev
from oracle import mtp_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

CASES = {
    # bf16, B = 2: pipelined GEMV
    "bf16-pipe": (small(name="sk1", cid=210, batch=2, K=3, ctx_lo=5, ctx_hi=120), [3, 1]),
    # bf16, B = 5: matrix-core path, lengths 0..K
    "bf16-mm": (small(name="sk2", cid=211, batch=5, K=4, ctx_lo=1, ctx_hi=200), [4, 0, 2, 1, 3]),
    # bf16, B = 17 over two 16-sequence tiles, many sequences at 0
    "bf16-mm-b17": (small(name="sk3", cid=212, batch=17, K=3, hidden=512, n_q=4, n_kv=4,
                          ffn=1536, vocab=4099, ctx_lo=0, ctx_hi=150), None),
    # fp32 column GEMV, G = 8
    "f32": (small(name="sk4", cid=213, hidden=256, n_q=16, n_kv=2, head_dim=64, ffn=520,
                  vocab=3000, batch=3, K=3, ctx_lo=60, ctx_hi=200, dtype="f32"), [0, 3, 2]),
    # the B = 32 ragged workload at full size, lengths drawn 0..3
    "q8b-b32": (S.get_config("q8b-b32"), None),
}


def _kseq(cfg, ks):
    if ks is None:
        ks = np.random.default_rng(cfg.cid).integers(0, cfg.K + 1, size=cfg.batch)
        ks[0], ks[-1] = cfg.K, 0
    return np.asarray(ks, np.int32)


@pytest.mark.parametrize("case", list(CASES))
def test_draft_seqk_equals_uniform_draft_prefix_and_oracle(case):
    """Sequence b's first k_b tokens and cache slots are bit-identical to the uniform
    K-step draft's (sequences are independent and the masked steps touch nothing); its
    later slots are untouched, len / pos advance by k_b; tokens agree with the oracle's
    per-sequence draft above the near-tie margin. One sequence sits so close to the cache
    end that a uniform K-step draft would overflow: masked steps need no capacity."""
    cfg, ks = CASES[case]
    K, B = cfg.K, cfg.batch
    ks = _kseq(cfg, ks)
    lens = S.cache_lengths(cfg)
    cap = int(lens.max()) + K + 8
    inp = S.make_inputs(cfg, capacity=cap)
    print(f"seqk draft {case}: B={B} K={K} k={ks.tolist()}", flush=True)
    hid = to_dev(inp.hidden, cfg.dtype)
    lt = torch.from_numpy(inp.last_tokens.astype(np.int32)).cuda()
    head, cache = make_head(cfg, inp)
    u_tok = head.draft(hid, lt, cache, K).cpu().numpy()
    uk, uv = cache_to_np(cache.k, cfg.dtype), cache_to_np(cache.v, cfg.dtype)
    head.close()
    # the sequence with the shortest own length starts at the cache end (no room for K)
    lens2 = inp.lens.copy()
    near = int(np.argmin(ks))
    lens2[near] = cap - int(ks[near])
    head, cache = make_head(cfg, inp)
    cache.len.copy_(torch.from_numpy(lens2.astype(np.int32)))
    cache.pos.copy_(torch.from_numpy(lens2.astype(np.int32)))
    # the uniform run's slots of the moved sequence do not apply to it
    s_tok = head.draft_seqk(hid, lt, cache, torch.from_numpy(ks).cuda(), K).cpu().numpy()
    assert head.get_error() == 0
    sk, sv = cache_to_np(cache.k, cfg.dtype), cache_to_np(cache.v, cfg.dtype)
    assert np.array_equal(cache.len.cpu().numpy(), lens2 + ks)
    assert np.array_equal(cache.pos.cpu().numpy(), lens2 + ks)
    head.close()
    for b in range(B):
        kb, L0 = int(ks[b]), int(lens2[b])
        if b != near:
            assert np.array_equal(s_tok[b, :kb], u_tok[b, :kb]), b
            assert np.array_equal(sk[b, :, L0:L0 + kb], uk[b, :, L0:L0 + kb])
            assert np.array_equal(sv[b, :, L0:L0 + kb], uv[b, :, L0:L0 + kb])
        assert np.array_equal(sk[b, :, L0 + kb:], inp.k_cache[b, :, L0 + kb:])
        assert np.array_equal(sv[b, :, L0 + kb:], inp.v_cache[b, :, L0 + kb:])
        assert np.array_equal(sk[b, :, :L0], inp.k_cache[b, :, :L0])
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft_seqk(cfg, W, inp.hidden, inp.last_tokens, kc, vc, lens2, lens2, ks, K)
    checked = 0
    for b in range(B):
        for k in range(int(ks[b])):
            if not np.array_equal(r["draft_tokens"][b, :k], s_tok[b, :k]):
                break
            if r["margin"][k, b] > MARGIN:
                assert r["draft_tokens"][b, k] == s_tok[b, k], (b, k)
                checked += 1
    assert checked >= int(ks.sum()) // 2


def test_draft_seqk_out_of_range_lengths_are_reported_and_clamped():
    cfg, _ = CASES["bf16-mm"]
    inp = S.make_inputs(cfg, capacity=int(S.cache_lengths(cfg).max()) + cfg.K + 8)
    head, cache = make_head(cfg, inp)
    ks = torch.tensor([cfg.K + 3, -2, 1, 0, 2], dtype=torch.int32, device="cuda")
    from mtp_self_speculative_amd import _lib as L
    head.draft_seqk(to_dev(inp.hidden, cfg.dtype),
                    torch.from_numpy(inp.last_tokens.astype(np.int32)).cuda(), cache, ks, cfg.K)
    assert head.get_error() & L.DEVERR_COUNT
    assert np.array_equal(cache.len.cpu().numpy(), inp.lens + np.array([cfg.K, 0, 1, 0, 2]))
    head.close()


@pytest.mark.parametrize("B,K,V", [(40, 5, 151936), (9, 3, 4099), (3, 0, 1000), (64, 1, 129280)])
def test_verify_seqk_parity(B, K, V):
    """Bit-exact against the oracle; target rows past k_b hold NaN and the drafts past k_b
    are out of range, so reading either would change the result."""
    cfg = small(name="vsk", cid=215 + K, batch=B, vocab=V, K=max(K, 1), agree_lo=0.7)
    rng = np.random.default_rng(B + K)
    d = rng.integers(0, V, size=(B, K)).astype(np.int32)
    t = S.plant_target_logits(cfg, d, 0)
    ks = rng.integers(0, K + 1, size=B).astype(np.int32)
    for b in range(B):
        t[b, ks[b] + 1:] = np.nan
        d[b, ks[b]:] = V + 7
    inp = S.make_inputs(small(name="vskh", cid=219, vocab=V, batch=B, K=max(K, 1), ctx_lo=1,
                              ctx_hi=None, hidden=64, n_q=2, n_kv=1, ffn=64), capacity=16)
    head, _ = make_head(inp.cfg, inp, max_batch=B, max_k=max(K, 1))
    acc, nxt = head.verify_seqk(torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda(),
                                torch.from_numpy(ks).cuda())
    assert head.get_error() == 0
    a_o, n_o = O.verify_seqk(t, d, ks)
    assert np.array_equal(acc.cpu().numpy(), a_o) and np.array_equal(nxt.cpu().numpy(), n_o)
    head.close()


def test_rollback_seqk_parity():
    cfg = small(name="rbk", cid=220, batch=40, K=5, ctx_lo=10, ctx_hi=50, hidden=64, n_q=2,
                n_kv=1, ffn=64, vocab=100)
    inp = S.make_inputs(cfg, capacity=64)
    head, cache = make_head(cfg, inp)
    rng = np.random.default_rng(9)
    ks = rng.integers(0, 6, size=cfg.batch).astype(np.int32)
    a = (rng.random(cfg.batch) * (ks + 1)).astype(np.int32)
    cache.len += torch.from_numpy(ks).cuda()
    cache.pos += torch.from_numpy(ks).cuda()
    head.rollback_seqk(cache, torch.from_numpy(a).cuda(), torch.from_numpy(ks).cuda(), 5)
    assert head.get_error() == 0
    ln, ps = O.kv_rollback_seqk(inp.lens + ks, inp.pos + ks, a, ks)
    assert np.array_equal(cache.len.cpu().numpy(), ln)
    assert np.array_equal(cache.pos.cpu().numpy(), ps)
    bad = a.copy()
    bad[0] = ks[0] + 1
    head.rollback_seqk(cache, torch.from_numpy(bad).cuda(), torch.from_numpy(ks).cuda(), 5)
    assert head.get_error() & 4
    head.close()


def test_gpu_decoding_with_per_sequence_k_equals_greedy():
    """Three sequences decoded in lock step by the GPU head, each with its own length from
    the library's window rule (mtp_adapt_k_seq): each emits its plain greedy decoding."""
    from mtp_self_speculative_amd import _lib as L
    from oracle.tiny_target import TinyTarget, lockstep_seqk
    cfg = small(name="ske", cid=221, hidden=128, n_q=4, n_kv=2, head_dim=64, ffn=256, vocab=2,
                batch=3, K=5, ctx_lo=4, ctx_hi=None, dtype="f32")
    inp = S.make_inputs(cfg, capacity=512)
    head, cache = make_head(cfg, inp)
    tgt = TinyTarget(cfg, S.target_weights(cfg, 2), inp.weights["embed"], inp.weights["lm_head"])
    prompts = [S.prompt_tokens(cfg, 5 + b, sub=b) for b in range(cfg.batch)]
    cache.pos.copy_(torch.tensor([len(p) - 1 for p in prompts], dtype=torch.int32))
    st = {}

    def draft(h, last, k, k_max):
        kt = torch.from_numpy(np.asarray(k, np.int32)).cuda()
        out = head.draft_seqk(torch.from_numpy(np.asarray(h, np.float32)).cuda(),
                              torch.from_numpy(np.asarray(last, np.int32)).cuda(), cache, kt,
                              k_max)
        st["d"], st["k"] = out, kt
        return out.cpu().numpy()

    def verify(rows, d, k):
        a, n = head.verify_seqk(torch.from_numpy(rows).cuda(), st["d"], st["k"])
        st["a"] = a
        return a.cpu().numpy(), n.cpu().numpy()

    def rollback(a, k):
        head.rollback_seqk(cache, st["a"], st["k"], 5)

    def adapt(ah, kh, kmin, kmax):
        return L.mtp_adapt_k_seq(ah.tolist(), kh.tolist(), kmin, kmax)

    out, kh = lockstep_seqk(tgt, prompts, 40, 2, 3, 0, 5, draft, verify, rollback, adapt)
    for b in range(cfg.batch):
        assert out[b] == tgt.greedy(prompts[b], 40), b
    assert head.get_error() == 0
    assert any(len(set(row.tolist())) > 1 for row in kh)
    head.close()
