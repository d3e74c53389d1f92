"""Greedy verification from the target's hidden states (through the target's final norm
and the shared lm_head, no logits written), HIP path against the oracle."""
import numpy as np
import pytest

import mtp_synth as S
from gpu_util import MARGIN, make_head, small, to_dev
from oracle import mtp_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

CASES = {
    # bf16, 3 x 5 rows: matrix-core lm_head; ragged vocabulary
    "bf16-mm": small(name="vh1", cid=150, batch=3, K=4),
    # bf16, 1 x 2 rows: widened rows through the pipelined GEMV
    "bf16-gemv": small(name="vh2", cid=151, batch=1, K=1, hidden=512, vocab=4099),
    # fp32, 2 x 4 rows: column-blocked GEMV
    "f32": small(name="vh3", cid=152, batch=2, K=3, hidden=256, vocab=3001, dtype="f32"),
    # bf16, 20 x 4 = 80 rows: one lm_head pass of eight 16-sequence tiles, three of them
    # partly or wholly past the rows
    "bf16-groups": small(name="vh4", cid=153, batch=20, K=3, hidden=512, vocab=4099),
    # bf16, 30 x 5 = 150 rows: two groups (128 + 22) of lm_head passes
    "bf16-two-groups": small(name="vh6", cid=155, batch=30, K=4, hidden=384, vocab=5003),
    # the same two shapes on handles without the packed lm_head copy: 80 rows and the first
    # 128 of 150 through the tiled contraction's argmax on the row-major lm_head (ragged
    # vocabulary; 384 columns end inside a 256-column chunk), the last 22 through the
    # weight-streaming kernel on the row-major lm_head
    "bf16-groups-lean": small(name="vh4", cid=153, batch=20, K=3, hidden=512, vocab=4099),
    "bf16-two-groups-lean": small(name="vh6", cid=155, batch=30, K=4, hidden=384, vocab=5003),
    # K = 0: the target's token of row 0 only
    "bf16-k0": small(name="vh5", cid=154, batch=5, K=0),
    # 3..8 rows of a handle without the packed lm_head (1-2 sequences): the pipelined GEMV
    # over all rows at once (3, 4, 7 and 8 rows, bf16 and fp32, ragged vocabulary)
    "bf16-rows3": small(name="vr3", cid=156, batch=1, K=2, hidden=512, vocab=4099),
    "bf16-rows4": small(name="vr4", cid=157, batch=2, K=1, hidden=640, vocab=5003),
    "bf16-rows7": small(name="vr7", cid=173, batch=1, K=6, hidden=384, vocab=3001),
    "bf16-rows8": small(name="vr8", cid=159, batch=2, K=3, hidden=512, vocab=4099),
    "f32-rows5": small(name="vr5", cid=180, batch=1, K=4, hidden=256, vocab=3001, dtype="f32"),
    # 2 x 4 rows too wide for the LDS of that GEMV (8 x 8192 floats): the matrix-core route
    "bf16-rows8-wide": small(name="vr9", cid=171, batch=2, K=3, hidden=8192, n_q=8, n_kv=2,
                             ffn=512, vocab=2053),
    # 16 x 4 = 64 and 12 x 4 = 48 rows over a 50021-row vocabulary: the lm_head pass on
    # 256-row items in 128-column stages (four and three 16-sequence tiles; the input
    # staging of three tiles ends in a partial pass)
    "bf16-rows64-wide-items": small(name="vw64", cid=186, batch=16, K=3, hidden=256, n_q=4,
                                    n_kv=2, head_dim=64, ffn=512, vocab=50021, ctx_hi=64),
    "bf16-rows48-wide-items": small(name="vw48", cid=187, batch=12, K=3, hidden=256, n_q=4,
                                    n_kv=2, head_dim=64, ffn=512, vocab=50021, ctx_hi=64),
    # full Qwen3-8B-shaped head (H=4096, V=151936), one sequence, K=5
    "q8b": S.get_config("q8b"),
    # same head, 32 sequences, K=3: 128 rows
    "q8b-b32": S.get_config("q8b-b32"),
}


def planted_drafts(cfg, g, rng):
    """Drafts equal to the target's tokens up to a random first mismatch per sequence."""
    B, K1 = g.shape
    K = K1 - 1
    d = g[:, :K].copy()
    stop = rng.integers(0, K + 1, size=B)
    for b in range(B):
        if stop[b] < K:
            d[b, stop[b]] = (d[b, stop[b]] + 1) % cfg.vocab
    return d.astype(np.int32), stop


@pytest.mark.parametrize("case", list(CASES))
def test_verify_hidden_parity(case):
    cfg = CASES[case]
    K = cfg.K
    inp = S.make_inputs(cfg, capacity=int(S.cache_lengths(cfg).max()) + max(K, 1) + 4)
    th = S.target_hidden(cfg, K)
    gn = S.target_norm(cfg)
    # the oracle's own tokens (and margins) give the planted drafts
    st = cfg.dtype
    logits = O.rmsnorm(O.as_float(th, st), O.as_float(gn, st), cfg.rms_eps) @ \
        O.as_float(inp.weights["lm_head"], st).T
    g = O.argmax_lowest(logits)
    rng = np.random.default_rng(cfg.cid)
    d, stop = planted_drafts(cfg, g, rng)
    a_o, n_o, margin = O.verify_from_hidden(cfg, th, gn, inp.weights["lm_head"], d)
    assert np.array_equal(a_o, stop)

    lean = case.endswith("-lean")
    head, _ = make_head(cfg, inp, max_batch=cfg.batch, max_k=max(K, 1), packed_copy=not lean)
    if lean:
        assert head.info()["packed_weight_bytes"] == 0
        assert head.info()["verify_hidden_group_rows"] == min(cfg.batch * (K + 1), 128)
    thd, gnd = to_dev(th, st), to_dev(gn, st)
    dd = torch.from_numpy(d).cuda() if K else None
    for rep in range(2):  # the second call checks that keys / counters were reset
        acc, nxt = head.verify_hidden(thd, gnd, dd)
        assert head.get_error() == 0
        acc, nxt = acc.cpu().numpy(), nxt.cpu().numpy()
        checked = 0
        for b in range(cfg.batch):
            if np.all(margin[b, :a_o[b] + 1] > MARGIN):
                assert acc[b] == a_o[b] and nxt[b] == n_o[b], (rep, b)
                checked += 1
        assert checked >= max(1, cfg.batch // 2)
    head.close()


def test_speculative_decoding_from_hidden_states_on_gpu_equals_greedy():
    """End to end: the GPU head drafts, the GPU verifies from the target's hidden states,
    and the emitted tokens equal the synthetic target's plain greedy decoding."""
    from oracle.tiny_target import TinyTarget, speculative_greedy
    cfg = small(name="e2eh", cid=141, hidden=128, n_q=4, n_kv=2, head_dim=64, ffn=256, vocab=8,
                batch=1, K=3, ctx_lo=8, ctx_hi=None, dtype="f32")
    inp = S.make_inputs(cfg, capacity=128)
    head, cache = make_head(cfg, inp)
    tw = S.target_weights(cfg, 2)
    tgt = TinyTarget(cfg, tw, inp.weights["embed"], inp.weights["lm_head"])
    gn = torch.from_numpy(np.ascontiguousarray(tw["g_final"])).cuda()
    prompt = S.prompt_tokens(cfg, 6)
    cache.pos.fill_(len(prompt) - 1)
    st = {}

    def draft_fn(h, last, K, _seq):
        out = head.draft(torch.from_numpy(np.asarray(h, np.float32)[None]).cuda(),
                         torch.tensor([last], dtype=torch.int32, device="cuda"), cache, K)
        st["d"] = out
        return out[0].cpu().numpy()

    def verify_fn(hid_rows, d):
        a, n = head.verify_hidden(torch.from_numpy(hid_rows[None].astype(np.float32)).cuda(), gn,
                                  st["d"])
        st["a"] = a
        return int(a[0]), int(n[0])

    def rollback_fn(a):
        head.rollback(cache, st["a"], 3)

    out, _ = speculative_greedy(tgt, prompt, 32, draft_fn, verify_fn, rollback_fn, 3,
                                from_hidden=True)
    assert out == tgt.greedy(prompt, 32)
    assert head.get_error() == 0
    head.close()


def test_speculative_decoding_with_adaptive_k_on_gpu_equals_greedy():
    """The GPU head drafts with a length that the library's adaptive rule changes every
    iteration; verification and rollback follow; output equals plain greedy decoding."""
    from mtp_self_speculative_amd import mtp_adapt_k
    from oracle.tiny_target import TinyTarget, speculative_greedy
    cfg = small(name="e2ek", cid=142, hidden=128, n_q=4, n_kv=2, head_dim=64, ffn=256, vocab=8,
                batch=1, K=6, ctx_lo=8, ctx_hi=None, dtype="f32")
    inp = S.make_inputs(cfg, capacity=256)
    head, cache = make_head(cfg, inp, max_k=6)
    tgt = TinyTarget(cfg, S.target_weights(cfg, 2), inp.weights["embed"], inp.weights["lm_head"])
    prompt = S.prompt_tokens(cfg, 6)
    cache.pos.fill_(len(prompt) - 1)
    st = {"ks": []}

    def draft_fn(h, last, K, _seq):
        st["K"] = K
        st["ks"].append(K)
        out = head.draft(torch.from_numpy(np.asarray(h, np.float32)[None]).cuda(),
                         torch.tensor([last], dtype=torch.int32, device="cuda"), cache, K)
        st["d"] = out
        return out[0].cpu().numpy()

    def verify_fn(rows, d):
        a, n = head.verify(torch.from_numpy(rows[None].astype(np.float32)).cuda(), st["d"])
        st["a"] = a
        return int(a[0]), int(n[0])

    def rollback_fn(a):
        head.rollback(cache, st["a"], st["K"])

    out, _ = speculative_greedy(tgt, prompt, 48, draft_fn, verify_fn, rollback_fn, 2,
                                next_k=lambda a, K: mtp_adapt_k([a], K, 1, 6))
    assert out == tgt.greedy(prompt, 48)
    assert len(set(st["ks"])) > 1
    assert head.get_error() == 0
    head.close()
