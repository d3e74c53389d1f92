"""Speculative iterations captured into a HIP graph and replayed.

The hot-path entry points launch kernels only: no allocation, no host synchronisation, no
memset. So a caller can capture whole iterations (draft, verify, rollback; or the sampling
pair) on its stream and replay them. Each case runs the iterations eagerly, captures the
same calls, and then replays the graph three times. Between replays it restores the cache
lengths with eager copies and synchronises. Every replay must give the eager tokens,
accepted lengths and cache state bit for bit."""
import numpy as np
import pytest

import mtp_synth as S
from gpu_util import make_head, small, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

ITERS = 3

CASES = {
    # fp32 weights, one sequence: the pipelined GEMV path
    "tiny": S.get_config("tiny"),
    # bf16, one sequence, several attention splits
    "bf16-b1": small(name="gr1", cid=191, batch=1, K=4, ctx_lo=200, ctx_hi=700),
    # bf16, five ragged sequences: the matrix-core path with its row kernels
    "bf16-b5": small(name="gr5", cid=192, batch=5, K=3, ctx_lo=1, ctx_hi=600),
}


def _setup(cfg):
    cap = int(S.cache_lengths(cfg).max()) + (ITERS + 2) * cfg.K + 8
    inp = S.make_inputs(cfg, capacity=cap)
    head, cache = make_head(cfg, inp)
    dev = torch.device("cuda:0")
    B, K = cfg.batch, cfg.K
    hidden = torch.stack([to_dev(S.hidden_states(cfg, it), cfg.dtype) for it in range(ITERS)])
    last0 = torch.from_numpy(inp.last_tokens.astype(np.int32)).to(dev)
    drafts = torch.zeros((ITERS, B, K), dtype=torch.int32, device=dev)
    acc = torch.zeros((ITERS, B), dtype=torch.int32, device=dev)
    nxt = torch.zeros((ITERS, B), dtype=torch.int32, device=dev)
    saved = (cache.k.clone(), cache.v.clone(), cache.len.clone(), cache.pos.clone())
    return head, cache, hidden, last0, drafts, acc, nxt, saved


def _restore(cache, saved):
    cache.k.copy_(saved[0])
    cache.v.copy_(saved[1])
    cache.len.copy_(saved[2])
    cache.pos.copy_(saved[3])


def _state(cache, *outs):
    return [t.clone() for t in (cache.k, cache.v, cache.len, cache.pos) + outs]


def _same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("case", list(CASES))
def test_greedy_iterations_replay_from_a_graph(case):
    cfg = CASES[case]
    K = cfg.K
    head, cache, hidden, last0, drafts, acc, nxt, saved = _setup(cfg)
    # target logits planted from an eager recording pass (agreement then a mismatch)
    logits = []
    last = last0
    for it in range(ITERS):
        head.draft(hidden[it], last, cache, K, out=drafts[it])
        tl = S.plant_target_logits(cfg, drafts[it].cpu().numpy(), it)
        logits.append(torch.from_numpy(tl).cuda())
        head.verify(logits[it], drafts[it], acc[it], nxt[it])
        head.rollback(cache, acc[it], K)
        last = nxt[it]
    torch.cuda.synchronize()
    assert head.get_error() == 0
    eager = _state(cache, drafts, acc, nxt)

    def iterations():
        last = last0
        for it in range(ITERS):
            head.draft(hidden[it], last, cache, K, out=drafts[it])
            head.verify(logits[it], drafts[it], acc[it], nxt[it])
            head.rollback(cache, acc[it], K)
            last = nxt[it]

    _restore(cache, saved)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iterations()
    torch.cuda.synchronize()
    for rep in range(3):
        _restore(cache, saved)
        for t in (drafts, acc, nxt):
            t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert head.get_error() == 0
        assert _same(_state(cache, drafts, acc, nxt), eager), (case, rep)
    head.close()


def test_sampling_iterations_replay_from_a_graph():
    """Temperature 1: draft_sample + verify_sample + rollback. The random streams are
    counter-based (seed, offset), so every replay draws the same numbers."""
    cfg = CASES["bf16-b5"]
    K, B = cfg.K, cfg.batch
    head, cache, hidden, last0, drafts, acc, nxt, saved = _setup(cfg)
    seeds = torch.from_numpy(S.sample_seeds(cfg).astype(np.int64)).cuda()
    dlog = torch.zeros((ITERS, B, K, cfg.vocab), dtype=torch.float32, device="cuda")
    tlog = [torch.from_numpy(S.sampling_logits(cfg, K, it)[0]).cuda() for it in range(ITERS)]

    def iterations():
        last = last0
        for it in range(ITERS):
            head.draft_sample(hidden[it], last, cache, K, 1.0, seeds, it, out=drafts[it],
                              logits=dlog[it])
            head.verify_sample(tlog[it], dlog[it], drafts[it], 1.0, seeds, it, acc[it], nxt[it])
            head.rollback(cache, acc[it], K)
            last = nxt[it]

    iterations()
    torch.cuda.synchronize()
    assert head.get_error() == 0
    eager = _state(cache, drafts, acc, nxt, dlog)
    _restore(cache, saved)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iterations()
    torch.cuda.synchronize()
    for rep in range(3):
        _restore(cache, saved)
        for t in (drafts, acc, nxt, dlog):
            t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert head.get_error() == 0
        assert _same(_state(cache, drafts, acc, nxt, dlog), eager), rep
    head.close()


@pytest.mark.parametrize("case", ["bf16-b1", "bf16-b5"])
def test_prefill_hidden_verification_and_catchup_replay_from_a_graph(case):
    """Prompt prefill, then iterations of draft, verification from the target's hidden
    states and exact cache catch-up, all captured: every replay matches the eager run."""
    cfg = CASES[case]
    K, B, n = cfg.K, cfg.batch, 70
    cap = int(S.cache_lengths(cfg).max()) + n + (ITERS + 2) * K + 8
    inp = S.make_inputs(cfg, capacity=cap)
    head, cache = make_head(cfg, inp)
    dev = torch.device("cuda:0")
    hidden = torch.stack([to_dev(S.hidden_states(cfg, it), cfg.dtype) for it in range(ITERS)])
    th = torch.stack([to_dev(S.target_hidden(cfg, K, it), cfg.dtype) for it in range(ITERS)])
    gn = to_dev(S.target_norm(cfg), cfg.dtype)
    ph = to_dev(S.prefill_hidden(cfg, n), cfg.dtype)
    pt = torch.from_numpy(S.prefill_tokens(cfg, n)).to(dev)
    last0 = torch.from_numpy(inp.last_tokens.astype(np.int32)).to(dev)
    drafts = torch.zeros((ITERS, B, K), dtype=torch.int32, device=dev)
    acc = torch.zeros((ITERS, B), dtype=torch.int32, device=dev)
    nxt = torch.zeros((ITERS, B), dtype=torch.int32, device=dev)
    saved = (cache.k.clone(), cache.v.clone(), cache.len.clone(), cache.pos.clone())

    def chain():
        head.prefill(cache, ph, pt)
        last = last0
        for it in range(ITERS):
            head.draft(hidden[it], last, cache, K, out=drafts[it])
            head.verify_hidden(th[it], gn, drafts[it], acc[it], nxt[it])
            head.catchup(cache, th[it], drafts[it], acc[it])
            last = nxt[it]

    chain()
    torch.cuda.synchronize()
    assert head.get_error() == 0
    eager = _state(cache, drafts, acc, nxt)
    _restore(cache, saved)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for rep in range(3):
        _restore(cache, saved)
        for t in (drafts, acc, nxt):
            t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert head.get_error() == 0
        assert _same(_state(cache, drafts, acc, nxt), eager), (case, rep)
    head.close()
