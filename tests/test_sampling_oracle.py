"""Pins of the sampling-verification oracle (CPU).

The random numbers are pinned to NumPy's own Philox4x64-10 generator; the sampling rules
are pinned by what they must produce statistically: Gumbel-max draws follow softmax(z/T),
speculative sampling leaves the target's distribution unchanged and accepts with the
closed-form probability sum_v min(p(v), q(v)) (Leviathan, Kalman and Matias, ICML 2023,
Theorem 3.5 / Definition 3.1), and decoding a tiny random target with the oracle MTP head
as drafter reproduces the target's exact sequence probabilities.
Every statistical test uses fixed seeds, so it is deterministic; thresholds are 5 standard
errors (or a chi-square tail of 1e-5).
"""
import numpy as np
import pytest
from scipy import stats

import mtp_synth as S
from oracle import mtp_oracle as O
from oracle import sampling as SP
from oracle.tiny_target import TinyTarget, softmax_rows, speculative_sample_batch

MASK = (1 << 64) - 1


def _plus_one(ctr):
    out, carry = [], 1
    for w in ctr:
        s = w + carry
        out.append(s & MASK)
        carry = s >> 64
    return out


@pytest.mark.parametrize("key,ctr", [
    ((0, 0), (0, 0, 0, 0)),
    ((123, 456), (7, 8, 9, 10)),
    ((MASK, MASK), (MASK - 1, MASK, MASK, MASK)),   # carry through every counter word
    ((0xDEADBEEF12345678, 0), (MASK, 3, 0, 1)),
    ((2 ** 63 + 5, 2 ** 40), (1 << 62, 1 << 61, 1 << 60, 1 << 59)),
])
def test_philox_matches_numpy_generator(key, ctr):
    """NumPy's Philox bit generator bumps its 256-bit counter before each block and then
    returns the four words of Philox4x64-10(counter, key)."""
    g = np.random.Philox(key=np.array(key, np.uint64), counter=np.array(ctr, np.uint64))
    raw = g.random_raw(8)
    c1 = _plus_one(ctr)
    c2 = _plus_one(c1)
    for c, want in ((c1, raw[:4]), (c2, raw[4:])):
        got = SP.philox4x64_10(*[np.uint64(x) for x in c], np.uint64(key[0]), np.uint64(key[1]))
        assert [int(w[0]) for w in got] == [int(x) for x in want]


def test_philox_vectorised_equals_elementwise():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 2 ** 63, size=(4, 37), dtype=np.uint64)
    k = rng.integers(0, 2 ** 63, size=(2, 37), dtype=np.uint64)
    vec = SP.philox4x64_10(*c, *k)
    for i in range(37):
        one = SP.philox4x64_10(*[x[i] for x in c], k[0, i], k[1, i])
        assert all(int(vec[w][i]) == int(one[w][0]) for w in range(4))


def test_uniforms_are_odd_multiples_in_open_interval():
    u = SP.vocab_uniforms(np.arange(64), 3, 0, 1, 1001)
    m = u * 2.0 ** 24
    assert np.all(m == np.round(m)) and np.all(m.astype(np.int64) % 2 == 1)
    assert u.min() > 0 and u.max() < 1
    assert abs(u.mean() - 0.5) < 5 * np.sqrt(1 / 12 / u.size)
    # word v & 3 of block v >> 2: entry v of the table is that word
    w = SP.philox4x64_10(np.uint64(5), np.uint64(1), np.uint64(0), np.uint64(3), np.uint64(7))
    assert SP.vocab_uniforms([7], 3, 0, 1, 24)[0, 21] == SP.to_uniform(w[1])[0]


def _freq(tokens, V):
    return np.bincount(np.asarray(tokens).ravel(), minlength=V) / np.asarray(tokens).size


def _close(freq, p, n):
    se = np.sqrt(np.maximum(p * (1 - p), 1e-12) / n)
    return np.all(np.abs(freq - p) <= 5 * se + 1e-12)


@pytest.mark.parametrize("T", [1.0, 0.6, 2.5])
def test_gumbel_max_draws_follow_softmax(T):
    z = np.array([[0.3, -1.2, 2.0, 0.0, 1.1, -0.4]])
    n = 200_000
    seeds = np.arange(n, dtype=np.uint64)
    tok, gap = SP.sample_tokens(np.repeat(z, n, 0), T, seeds, 11, 2)
    p = softmax_rows(z, T)[0]
    assert _close(_freq(tok, 6), p, n)
    assert np.all(gap >= 0)


def test_streams_are_independent_across_rows_purposes_and_offsets():
    z = np.zeros((1, 8))
    n = 100_000
    seeds = np.arange(n, dtype=np.uint64) * 7919
    t0, _ = SP.sample_tokens(np.repeat(z, n, 0), 1.0, seeds, 0, 0)
    t1, _ = SP.sample_tokens(np.repeat(z, n, 0), 1.0, seeds, 0, 1)
    t2, _ = SP.sample_tokens(np.repeat(z, n, 0), 1.0, seeds, 1, 0)
    for other in (t1, t2):
        joint = np.bincount(t0 * 8 + other, minlength=64) / n
        assert _close(joint, np.full(64, 1 / 64), n)
    u = SP.accept_uniforms(seeds[:2000], 0, 3)
    assert abs(np.corrcoef(u[:, 0], u[:, 1])[0, 1]) < 5 / np.sqrt(2000)


def _scheme_trials(tl, zl, T, n, offset=0):
    """n independent verifications of the same target / draft rows, drafts drawn from the
    draft distributions with the oracle's own noise."""
    K = zl.shape[0]
    seeds = np.arange(n, dtype=np.uint64) + 1000
    d = np.stack([SP.sample_tokens(np.repeat(zl[j][None], n, 0), T, seeds, offset, j)[0]
                  for j in range(K)], axis=1)
    r = SP.verify_sample(np.repeat(tl[None], n, 0), np.repeat(zl[None], n, 0), d, T, seeds,
                         offset)
    return d, r


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_speculative_sampling_preserves_target_distribution(T):
    """Rows here do not depend on the drafted tokens, so each emitted position must follow
    its own target row: first token ~ p_0; given d_1 accepted, second ~ p_1; given both
    accepted, the bonus ~ p_2. Acceptance of d_1 happens with probability sum min(p_0, q_0)."""
    rng = np.random.default_rng(3)
    V, K, n = 5, 2, 200_000
    tl = rng.normal(0, 1.5, size=(K + 1, V))
    zl = tl[:K] + rng.normal(0, 1.0, size=(K, V))
    d, r = _scheme_trials(tl, zl, T, n)
    a, nxt = r["accepted_len"], r["next_token"]
    p, q = softmax_rows(tl, T), softmax_rows(zl, T)
    first = np.where(a >= 1, d[:, 0], nxt)
    assert _close(_freq(first, V), p[0], n)
    acc_rate = np.minimum(p[0], q[0]).sum()
    assert abs((a >= 1).mean() - acc_rate) <= 5 * np.sqrt(acc_rate * (1 - acc_rate) / n)
    m1 = a >= 1
    second = np.where(a[m1] >= 2, d[m1, 1], nxt[m1])
    assert _close(_freq(second, V), p[1], m1.sum())
    m2 = a == 2
    assert _close(_freq(nxt[m2], V), p[2], m2.sum())
    # the draft tokens themselves follow q
    assert _close(_freq(d[:, 0], V), q[0], n)


def test_identical_distributions_accept_everything():
    rng = np.random.default_rng(4)
    tl = rng.normal(0, 2, size=(4, 7))
    d, r = _scheme_trials(tl, tl[:3].copy(), 1.0, 5000)
    assert np.all(r["accepted_len"] == 3)
    assert _close(_freq(r["next_token"], 7), softmax_rows(tl, 1.0)[3], 5000)


def test_draft_mass_where_target_has_none_is_always_rejected():
    tl = np.array([[0.0, 0.5, 1.0, -60.0], [0.0, 0.0, 0.0, 0.0]])
    zl = np.array([[-60.0, -60.0, -60.0, 0.0]])  # the draft always proposes token 3
    d, r = _scheme_trials(tl, zl, 1.0, 20_000)
    assert np.all(d[:, 0] == 3)
    assert np.all(r["accepted_len"] == 0) and np.all(r["residual"])
    assert _close(_freq(r["next_token"], 4), softmax_rows(tl[:1], 1.0)[0], 20_000)


def test_k0_draws_the_bonus_from_the_target():
    tl = np.array([[1.0, 0.0, -1.0, 0.5]])
    n = 50_000
    r = SP.verify_sample(np.repeat(tl[None], n, 0), np.zeros((n, 0, 4)), np.zeros((n, 0)), 0.9,
                         np.arange(n), 2)
    assert np.all(r["accepted_len"] == 0)
    assert _close(_freq(r["next_token"], 4), softmax_rows(tl, 0.9)[0], n)


def test_sampled_drafting_with_the_head_reproduces_target_sequence_probabilities():
    """End to end: many independent generations from one prompt, each drafted by the
    oracle MTP head (sampling at T) and verified by speculative sampling against a tiny
    random target; the empirical distribution of the first three emitted tokens equals
    the target's exact sequence probabilities p(x1) p(x2|x1) p(x3|x1,x2)."""
    V, K, T, n = 4, 2, 1.0, 4000
    cfg = S.Config(name="samp", cid=77, hidden=64, n_q=4, n_kv=2, head_dim=16, ffn=96, vocab=V,
                   batch=n, K=K, ctx_lo=0, ctx_hi=None, agree_lo=0.8, agree_hi=None, dtype="f32")
    inp = S.make_inputs(cfg, capacity=16)
    W = O.OracleWeights(cfg, inp.weights)
    tgt = TinyTarget(cfg, S.target_weights(cfg, 2), inp.weights["embed"], inp.weights["lm_head"])
    prompt = [int(x) for x in S.prompt_tokens(cfg, 5)]
    seeds = np.arange(n, dtype=np.uint64) * 31 + 9
    p1 = softmax_rows(tgt.forward(prompt)[1][-1:], T)[0]
    first = np.random.default_rng(12).choice(V, size=n, p=p1)
    st = {"kc": np.zeros_like(inp.k_cache), "vc": np.zeros_like(inp.v_cache),
          "len": np.zeros(n, np.int64), "pos": np.full(n, len(prompt) - 1, np.int64)}

    def draft_fn(h, last, K_, it):
        r = O.draft(cfg, W, h.astype(np.float32), last, st["kc"], st["vc"], st["len"], st["pos"],
                    K_, sample={"T": T, "seeds": seeds, "offset": it})
        st["len"], st["pos"] = r["lens"], r["pos"]
        return r["draft_tokens"], np.transpose(r["logits"], (1, 0, 2))

    def verify_fn(rows, d, dl, it):
        r = SP.verify_sample(rows, dl, d, T, seeds, it)
        return r["accepted_len"], r["next_token"]

    def commit_fn(a):
        st["len"], st["pos"] = O.kv_rollback(st["len"], st["pos"], a, K)

    out, acc = speculative_sample_batch(tgt, prompt, 3, first, draft_fn, verify_fn, commit_fn, K)
    # exact probabilities of every 3-token continuation
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
    if not keep.all():  # pool the rare continuations into one cell
        obs = np.append(obs, counts[~keep].sum())
        exp = np.append(exp, expect[~keep].sum())
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert stats.chi2.sf(chi2, len(obs) - 1) > 1e-5, chi2
    rate = np.concatenate(acc).mean() / K
    assert 0.05 < rate < 0.95  # both outcomes occur: the test exercises accept and reject
