"""Handles without the re-laid-out weight copy, and refreshing that copy after the weights
changed in place. The matrix-core kernels on the row-major weights and on the copy add the
same products in the same order, so both handles must agree bit for bit; the oracle checks
the lean handle as it checks every draft."""
import numpy as np
import pytest

import mtp_synth as S
from gpu_util import MARGIN, compare_draft, small, to_dev
from oracle import mtp_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

# 5 sequences: the matrix-core path (3+ sequences), ragged vocabulary
CFG = small(name="wt1", cid=190, batch=5, K=3)


def make_inputs(cfg):
    return S.make_inputs(cfg, capacity=int(S.cache_lengths(cfg).max()) + cfg.K + 4)


def head_for(cfg, inp, w, packed_copy=True):
    from mtp_self_speculative_amd import MtpHead
    return MtpHead(hidden=cfg.hidden, n_q_heads=cfg.n_q, n_kv_heads=cfg.n_kv,
                   head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=cfg.vocab, weights=w,
                   max_batch=cfg.batch, max_k=cfg.K, max_capacity=inp.capacity,
                   rope_theta=cfg.rope_theta, rms_eps=cfg.rms_eps, dtype=torch.bfloat16,
                   packed_copy=packed_copy)


def draft(head, cfg, inp):
    """One K-step draft from the inputs' own cache (a fresh device copy per call)."""
    from mtp_self_speculative_amd import MtpCache
    cache = MtpCache(to_dev(inp.k_cache, cfg.dtype), to_dev(inp.v_cache, cfg.dtype),
                     torch.from_numpy(inp.lens.astype(np.int32)).cuda(),
                     torch.from_numpy(inp.pos.astype(np.int32)).cuda())
    hid = to_dev(inp.hidden, cfg.dtype)
    lt = torch.from_numpy(inp.last_tokens.astype(np.int32)).cuda()
    tok, h, t2, _ = head.draft_debug(hid, lt, cache, cfg.K)
    assert head.get_error() == 0
    torch.cuda.synchronize()
    return tok.cpu().numpy(), h.cpu().numpy(), t2.cpu().numpy(), cache


def test_draft_without_packed_copy_matches_packed_and_oracle():
    cfg = CFG
    inp = make_inputs(cfg)
    w = {k: to_dev(v, cfg.dtype) for k, v in inp.weights.items()}
    full, lean = head_for(cfg, inp, w), head_for(cfg, inp, w, packed_copy=False)
    fi, li = full.info(), lean.info()
    assert fi["packed_weight_bytes"] > 0 and li["packed_weight_bytes"] == 0
    assert li["workspace_bytes"] <= fi["workspace_bytes"] - fi["packed_weight_bytes"]
    t1, h1, s1, c1 = draft(full, cfg, inp)
    t2, h2, s2, c2 = draft(lean, cfg, inp)
    assert np.array_equal(t1, t2)
    assert np.array_equal(h1, h2) and np.array_equal(s1, s2)
    assert torch.equal(c1.k, c2.k) and torch.equal(c1.v, c2.v)
    assert torch.equal(c1.len, c2.len) and torch.equal(c1.pos, c2.pos)
    W = O.OracleWeights(cfg, inp.weights)
    kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
    r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, cfg.K,
                force_tokens=t2)
    assert compare_draft(cfg, r, t2, h2, s2) >= cfg.batch
    full.close()
    lean.close()


def test_verify_hidden_without_packed_copy():
    """5 x 4 = 20 rows: one pass on the row-major lm_head (the default handle reads its
    copy); both agree, and agree with the oracle off near-ties."""
    cfg = CFG
    K = cfg.K
    inp = make_inputs(cfg)
    w = {k: to_dev(v, cfg.dtype) for k, v in inp.weights.items()}
    full, lean = head_for(cfg, inp, w), head_for(cfg, inp, w, packed_copy=False)
    assert lean.info()["verify_hidden_group_rows"] == cfg.batch * (K + 1)
    th, gn = S.target_hidden(cfg, K), S.target_norm(cfg)
    st = cfg.dtype
    logits = O.rmsnorm(O.as_float(th, st), O.as_float(gn, st), cfg.rms_eps) @ \
        O.as_float(inp.weights["lm_head"], st).T
    g = O.argmax_lowest(logits)
    d = g[:, :K].copy().astype(np.int32)
    d[1, 1] = (d[1, 1] + 1) % cfg.vocab  # sequence 1 stops at draft 1
    a_o, n_o, margin = O.verify_from_hidden(cfg, th, gn, inp.weights["lm_head"], d)
    thd, gnd, dd = to_dev(th, st), to_dev(gn, st), torch.from_numpy(d).cuda()
    af, nf = full.verify_hidden(thd, gnd, dd)
    al, nl = lean.verify_hidden(thd, gnd, dd)
    assert full.get_error() == 0 and lean.get_error() == 0
    af, nf, al, nl = (x.cpu().numpy() for x in (af, nf, al, nl))
    checked = 0
    for b in range(cfg.batch):
        if np.all(margin[b, :a_o[b] + 1] > MARGIN):
            assert al[b] == a_o[b] and nl[b] == n_o[b], b
            assert af[b] == a_o[b] and nf[b] == n_o[b], b
            checked += 1
    assert checked >= cfg.batch // 2
    full.close()
    lean.close()


def test_refresh_weights_after_in_place_change():
    cfg = CFG
    inp = make_inputs(cfg)
    w = {k: to_dev(v, cfg.dtype) for k, v in inp.weights.items()}
    full, lean = head_for(cfg, inp, w), head_for(cfg, inp, w, packed_copy=False)
    t0 = draft(full, cfg, inp)[0]
    # the verifier updates its lm_head in place: row v now holds the old row v - 1, so every
    # first-step argmax moves up by one
    w["lm_head"].copy_(torch.roll(w["lm_head"], 1, 0))
    torch.cuda.synchronize()
    assert np.array_equal(draft(full, cfg, inp)[0], t0)  # the copy still holds the old rows
    full.refresh_weights()
    lean.refresh_weights()  # nothing to rebuild: a no-op
    fresh = head_for(cfg, inp, w)
    tf, hf, sf, _ = draft(fresh, cfg, inp)
    assert np.array_equal(tf[:, 0], (t0[:, 0] + 1) % cfg.vocab)
    tr, hr, sr, _ = draft(full, cfg, inp)
    assert np.array_equal(tr, tf) and np.array_equal(hr, hf) and np.array_equal(sr, sf)
    tl, hl, sl, _ = draft(lean, cfg, inp)  # reads the weights in place
    assert np.array_equal(tl, tf) and np.array_equal(hl, hf) and np.array_equal(sl, sf)
    for h in (full, lean, fresh):
        assert h.get_error() == 0
        h.close()


def test_full_size_batched_draft_identical_without_packed_copy():
    """q8b-b32 shapes (H=4096, V=151936, 32 ragged sequences, K=3): the row-major
    contractions give the default handle's tokens, hidden states and top-2 logits bit for
    bit, and verification from hidden states (128 rows: the tiled contraction on the
    row-major lm_head in both handles) gives the same accepted lengths and next tokens
    wherever the oracle's margin clears the near-tie bar."""
    cfg = S.get_config("q8b-b32")
    inp = make_inputs(cfg)
    w = {k: to_dev(v, cfg.dtype) for k, v in inp.weights.items()}
    full, lean = head_for(cfg, inp, w), head_for(cfg, inp, w, packed_copy=False)
    t1, h1, s1, c1 = draft(full, cfg, inp)
    t2, h2, s2, c2 = draft(lean, cfg, inp)
    assert np.array_equal(t1, t2)
    assert np.array_equal(h1, h2) and np.array_equal(s1, s2)
    assert torch.equal(c1.k, c2.k) and torch.equal(c1.v, c2.v)
    del c1, c2
    K = cfg.K
    th, gn = S.target_hidden(cfg, K), S.target_norm(cfg)
    thd, gnd = to_dev(th, cfg.dtype), to_dev(gn, cfg.dtype)
    dd = torch.from_numpy(t1).cuda()
    af, nf = full.verify_hidden(thd, gnd, dd)
    al, nl = lean.verify_hidden(thd, gnd, dd)
    assert full.get_error() == 0 and lean.get_error() == 0
    af, nf, al, nl = (x.cpu().numpy() for x in (af, nf, al, nl))
    a_o, n_o, margin = O.verify_from_hidden(cfg, th, gn, inp.weights["lm_head"], t1)
    checked = 0
    for b in range(cfg.batch):
        if np.all(margin[b, :a_o[b] + 1] > MARGIN):
            assert (af[b], nf[b]) == (a_o[b], n_o[b]) == (al[b], nl[b]), b
            checked += 1
    assert checked >= cfg.batch // 2
    full.close()
    lean.close()
