#!/usr/bin/env python3
"""Benchmark of the MTP draft / verify / rollback path on one MI355X.

One step = one speculative iteration over the batch: K recursive draft steps
(mtp_draft), greedy verification against target logits (mtp_verify) and the MTP
cache rollback (mtp_kv_rollback). Inputs are seeded and synthetic. The target
logits of every iteration are planted from the drafts of an untimed recording
pass and are resident in HBM before the timed pass replays the identical chain
(the kernels are deterministic; the replay is checked against the recording).

Prints one JSON line: draft-steps/s (value), verified tokens/s, the HBM roofline
fraction of the whole iteration and of the lm_head kernel (HIP events on the
library's stream), and the oracle timed on the host's cores. The headline workload
is the Qwen3-8B-shaped head at batch 1; the same run also times the other workloads
(B=32 ragged, the Qwen3-32B shape at 32K context, the wide B=64 head and the tiny
fp32 head) under "workloads", each with its own throughput, HBM fraction, lm_head
fraction and device memory; the batched ones also replay the same iterations on a
handle without the re-laid-out weight copy ("without_packed_copy"). Every workload
also replays its timed iterations from one captured HIP graph ("graph_replay": the same
kernels without host-side launch work, checked against the recording); the headline
value stays the eager replay.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "lm_head_argmax_q8b_counters.md")
LMHEAD_SOURCES = ("mtp_self_speculative_amd/csrc/gemv_pipe.hip",
                  "mtp_self_speculative_amd/csrc/common.h",
                  "mtp_self_speculative_amd/csrc/kernels.h")
METRIC = "MTP draft-steps/s + verified tok/s at 1 GPU; % of HBM roofline"
LMHEAD_BIT = 1 << 6
DESCR = {
    "tiny": "tiny fp32 MTP head: H=256, 4/2 heads x 64, FFN 768, V=4096, B=1, L=128, K=3",
    "q8b": "Qwen3-8B-shaped MTP head, bf16: H=4096, 32/8 heads x 128, FFN 12288, V=151936, "
           "B=1, KV context 4096, K=5, planted agreement 0.9",
    "q8b-b32": "Qwen3-8B-shaped MTP head, bf16, B=32 ragged KV context U{512..8192}, K=3, "
               "planted agreement 0.6",
    "q32b": "Qwen3-32B-shaped MTP head, bf16: H=5120, 64/8 heads x 128, FFN 25600, V=151936, "
            "B=8, KV context 32768, K=5",
    "wide": "wide dense MTP head, bf16: H=7168, 56/8 heads x 128, FFN 18432, V=129280, B=64, "
            "KV context 4096, K=1",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(cfg, lens0, K: int, acc_sum_rows: int) -> dict:
    """Bytes one iteration must move at least: every weight once per draft step, the
    gathered embedding rows, the KV cache read (including the new slot) and written,
    and the target-logit rows verification needs."""
    s = 2 if cfg.dtype == "bf16" else 4
    H, F, V, d = cfg.hidden, cfg.ffn, cfg.vocab, cfg.head_dim
    qd, kvd = cfg.n_q * d, cfg.n_kv * d
    B = cfg.batch
    w_layer = (2 * H * H + qd * H + 2 * kvd * H + H * qd + 3 * F * H + 5 * H) * s
    lm = V * H * s
    per_step_w = w_layer + lm
    kv_read = sum(2 * kvd * (int(L) + k + 1) * s for L in lens0 for k in range(K))
    kv_write = B * K * 2 * kvd * s
    emb = B * K * H * s
    io = B * H * s + B * 4 * (2 + K)
    verify = acc_sum_rows * V * 4
    return {"per_step_weights": per_step_w, "lm_head": lm + H * s + B * H * 4 + B * 8,
            "iteration": K * per_step_w + kv_read + kv_write + emb + io + verify}


def lmhead_source_hash() -> str:
    """Hash of the lm_head kernel's sources with comments and blank lines removed, so that
    only a change of code (not of its comments) retires the recorded counters."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in LMHEAD_SOURCES:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        lines = [ln.rstrip() for ln in src.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def measured_traffic(config: str):
    """HBM bytes per lm_head launch from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE scaled by the copy-kernel calibration), or None when the
    summary is missing, is for another workload, or the kernel source changed since."""
    if config != "q8b" or not os.path.exists(TRAFFIC_SUMMARY):
        return None
    vals = {}
    for line in open(TRAFFIC_SUMMARY):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256_16") != lmhead_source_hash():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3) -> None:
    """A plain device-to-device copy of known size, run under rocprofv3 --pmc to scale
    FETCH_SIZE / WRITE_SIZE readings to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def cpu_baseline(cfg, inp, K: int, iter_bytes: int, budget32: float = 8.0,
                 budget64: float = 4.0) -> dict:
    """The oracle (plain NumPy, untuned) on the host cores: one speculative iteration of the
    same workload (K draft steps + verify + rollback), 1 warm-up then the median of as many
    timed iterations as fit the time budget (at least 3); the stated value is the float32
    oracle, the float64 one is reported beside it. Input generation and the widening of the
    weights are not timed."""
    import numpy as np

    import mtp_synth as S
    from oracle import mtp_oracle as O
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        if info:
            threads = max(int(i.get("num_threads", 1)) for i in info)
            blas = ", ".join(f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                             for i in info)
    except Exception:  # pragma: no cover
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        affinity = os.cpu_count() or 1

    def timed(dt, budget):
        W = O.OracleWeights(cfg, inp.weights, dt=dt)
        times = []
        rep = -1
        while rep < 3 or (sum(times) < budget and rep < 200):
            rep += 1
            kc, vc = inp.k_cache.copy(), inp.v_cache.copy()
            t0 = time.perf_counter()
            r = O.draft(cfg, W, inp.hidden, inp.last_tokens, kc, vc, inp.lens, inp.pos, K)
            t1 = time.perf_counter()
            tl = S.plant_target_logits(cfg, r["draft_tokens"], 0)
            t2 = time.perf_counter()
            a, _ = O.verify(tl, r["draft_tokens"])
            O.kv_rollback(r["lens"], r["pos"], a, K)
            t3 = time.perf_counter()
            if rep:
                times.append((t1 - t0) + (t3 - t2))
        log(f"cpu oracle ({np.dtype(dt).name}): median {statistics.median(times):.3f} s "
            f"per iteration over {len(times)}")
        return statistics.median(times), len(times)

    t32, reps32 = timed(np.float32, budget32)
    t64, reps64 = timed(np.float64, budget64)
    return {"value": round(K / t32, 4), "unit": "draft-steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{reps32} timed iterations (after 1 warm-up) of {K} draft steps + verify "
                      f"+ rollback of the same workload, float32 NumPy oracle, median "
                      f"{t32:.3f} s per iteration",
            "effective_gb_per_s": round(iter_bytes / t32 / 1e9, 3),
            "float64": {"value": round(K / t64, 4), "unit": "draft-steps/s",
                        "median_s_per_iteration": round(t64, 4), "reps": reps64,
                        "effective_gb_per_s": round(iter_bytes / t64 / 1e9, 3)},
            "host": {"os_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
                     "blas": blas, "blas_threads": threads}}


def sampling_pass(args, cfg, head, cache, hidden, last0, len0, pos0, up) -> dict:
    """Temperature sampling at T = 1, timed like the greedy pass: the draft samples each
    token in the lm_head kernel (draft logits written); the target's rows are the draft's
    logits plus N(0, 1) noise (row K: N(0, 1.3^2)), which gives about 60% acceptance per
    draft; speculative-sampling verification decides and the cache is rolled back. The
    iteration index is the random-stream offset, so the replay reproduces the recording."""
    import numpy as np
    import torch

    import mtp_synth as S
    from mtp_self_speculative_amd._lib import KERNEL_CLASSES
    dev = hidden.device
    B, K, V = cfg.batch, cfg.K, cfg.vocab
    iters = args.warmup + args.steps
    T = 1.0
    seeds = torch.from_numpy(S.sample_seeds(cfg).view(np.int64)).to(dev)
    toks = torch.empty((iters, B, K), dtype=torch.int32, device=dev)
    dlog = torch.empty((iters, B, K, V), dtype=torch.float32, device=dev)
    tlog = torch.empty((iters, B, K + 1, V), dtype=torch.float32, device=dev)
    acc = torch.empty((iters, B), dtype=torch.int32, device=dev)
    nxt = torch.empty((iters, B), dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg.cid * 1000 + 17)

    def run(it, last, plant=False):
        head.draft_sample(hidden[it], last, cache, K, T, seeds, it, out=toks[it], logits=dlog[it])
        if plant:
            tlog[it, :, :K] = dlog[it] + torch.randn((B, K, V), generator=gen, device=dev)
            tlog[it, :, K] = 1.3 * torch.randn((B, V), generator=gen, device=dev)
        head.verify_sample(tlog[it], dlog[it], toks[it], T, seeds, it, acc[it], nxt[it])
        head.rollback(cache, acc[it], K)
        return nxt[it]

    def replay(mask, plant=False):
        cache.len.copy_(len0)
        cache.pos.copy_(pos0)
        last = last0
        head.set_profiling(0)
        for it in range(args.warmup):
            last = run(it, last, plant)
        torch.cuda.synchronize()
        head.set_profiling(mask)
        t0 = time.perf_counter()
        for it in range(args.warmup, iters):
            last = run(it, last, plant)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        head.set_profiling(0)
        return t1 - t0, head.get_profile()

    replay(0, plant=True)
    rec_t, rec_a = toks.clone(), acc.clone()
    assert head.get_error() == 0
    elapsed, _ = replay(0)
    if not (torch.equal(toks, rec_t) and torch.equal(acc, rec_a)):
        raise RuntimeError("timed sampling replay diverged from the recording pass")
    mask = (1 << KERNEL_CLASSES.index("lm_head_argmax")) | (1 << KERNEL_CLASSES.index("verify"))
    _, prof = replay(mask)
    a = acc[args.warmup:].cpu().numpy().astype(np.int64)
    lm_ms, lm_n = prof["lm_head_argmax"]
    v_ms, v_n = prof["verify"]
    log(f"sampling pass: {args.steps} iterations in {elapsed * 1e3:.2f} ms, "
        f"acceptance {a.mean() / K:.3f}")
    out = {"temperature": T, "draft_steps_per_s": round(K * args.steps / elapsed, 3),
           "verified_tok_per_s": round(float((a + 1).sum()) / elapsed, 2),
           "acceptance_per_draft": round(float(a.mean()) / K, 4),
           "lm_head_sample_us": round(lm_ms * 1e3 / lm_n, 2),
           "verify_sample_us": round(v_ms * 1e3 / v_n, 2)}
    cache.len.copy_(len0)
    cache.pos.copy_(pos0)
    del dlog, tlog
    torch.cuda.empty_cache()
    return out


def large_cache_probe(args, cfg, w, head, cache, hidden, last0, len0, pos0,
                      capacity: int = 32768) -> dict:
    """Attention + merge per launch (HIP events on the library's stream) with the bench's
    cache and with a copy of it in a cache of `capacity` slots holding the same lengths:
    the chunk is planned from the lengths, so the two should take about the same time."""
    import torch

    from mtp_self_speculative_amd import MtpCache, MtpHead
    from mtp_self_speculative_amd._lib import KERNEL_CLASSES
    bit = 1 << KERNEL_CLASSES.index("attention")
    B, K = cfg.batch, cfg.K
    cap0 = cache.capacity
    k2 = torch.zeros((B, cfg.n_kv, capacity, cfg.head_dim), dtype=cache.k.dtype,
                     device=cache.k.device)
    v2 = torch.zeros_like(k2)
    k2[:, :, :cap0] = cache.k
    v2[:, :, :cap0] = cache.v
    big = MtpCache(k2, v2, cache.len.clone(), cache.pos.clone())
    head2 = MtpHead(hidden=cfg.hidden, n_q_heads=cfg.n_q, n_kv_heads=cfg.n_kv,
                    head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=cfg.vocab, weights=w,
                    max_batch=B, max_k=K, max_capacity=capacity, rope_theta=cfg.rope_theta,
                    rms_eps=cfg.rms_eps, dtype=cache.k.dtype)
    out = {"capacity": capacity, "len": int(len0.max())}
    for key, hd, cc in (("us_cache_as_filled", head, cache), ("us_cache_32768", head2, big)):
        hd.set_profiling(0)
        for it in range(args.warmup + args.steps):
            cc.len.copy_(len0)
            cc.pos.copy_(pos0)
            if it == args.warmup:
                torch.cuda.synchronize()
                hd.set_profiling(bit)
            hd.draft(hidden[it], last0, cc, K)
        torch.cuda.synchronize()
        hd.set_profiling(0)
        ms, n = hd.get_profile()["attention"]
        out[key] = round(ms * 1e3 / max(n, 1), 2)
    out["capacity_as_filled"] = cap0
    head2.close()
    cache.len.copy_(len0)
    cache.pos.copy_(pos0)
    del k2, v2, big
    torch.cuda.empty_cache()
    log(f"attention + merge with a {capacity}-slot cache: {out}")
    return out


def run_workload(name: str, args, full: bool) -> dict:
    """Record, then replay and time `args.steps` speculative iterations of one workload.

    full (the headline workload): also the lm_head's own HIP-event roofline, per-call
    latency percentiles, the optional per-kernel breakdown, verification from hidden states,
    exact catch-up, prompt prefill and the sampling pass. Otherwise: throughput, HBM
    fraction, the lm_head fraction, verification from hidden states and catch-up."""
    import numpy as np
    import torch

    import mtp_synth as S
    from mtp_self_speculative_amd import MtpCache, MtpHead

    dev = torch.device("cuda:0")
    cfg = S.get_config(name)
    B, K = cfg.batch, cfg.K
    iters = args.warmup + args.steps
    hot = args.hot_only
    lens0 = S.cache_lengths(cfg)
    cap = int(lens0.max()) + (iters + 2) * K + 8
    t0 = time.time()
    inp = S.make_inputs(cfg, capacity=cap)
    log(f"generated {name} inputs in {time.time() - t0:.1f} s")
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    esz = 2 if cfg.dtype == "bf16" else 4

    def up(a):
        if cfg.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    w = {k: up(v) for k, v in inp.weights.items()}
    head = MtpHead(hidden=cfg.hidden, n_q_heads=cfg.n_q, n_kv_heads=cfg.n_kv,
                   head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=cfg.vocab, weights=w, max_batch=B,
                   max_k=K, max_capacity=cap, rope_theta=cfg.rope_theta, rms_eps=cfg.rms_eps,
                   dtype=tdt)
    cache = MtpCache(up(inp.k_cache), up(inp.v_cache), torch.from_numpy(inp.lens).to(dev),
                     torch.from_numpy(inp.pos).to(dev))
    hidden = torch.stack([up(S.hidden_states(cfg, it)) for it in range(iters)])
    last0 = torch.from_numpy(inp.last_tokens).to(dev)
    len0, pos0 = cache.len.clone(), cache.pos.clone()
    drafts = torch.empty((iters, B, K), dtype=torch.int32, device=dev)
    acc = torch.empty((iters, B), dtype=torch.int32, device=dev)
    nxt = torch.empty((iters, B), dtype=torch.int32, device=dev)
    info = head.info()
    shared = int(w["embed"].numel() + w["lm_head"].numel()) * esz
    memory = {"weights_bytes": int(sum(t.numel() for t in w.values())) * esz,
              "of_which_shared_embed_lm_head_bytes": shared,
              "workspace_bytes": info["workspace_bytes"],
              "of_which_packed_copy_bytes": info["packed_weight_bytes"],
              "kv_cache_bytes": int(cache.k.numel() + cache.v.numel()) * esz}
    log(f"{name}: inputs resident on the device; memory {memory}")

    # Recording pass: plant each iteration's target logits from the drafts it produced.
    logits = []
    last = last0
    for it in range(iters):
        head.draft(hidden[it], last, cache, K, out=drafts[it])
        tl = S.plant_target_logits(cfg, drafts[it].cpu().numpy(), it)
        logits.append(torch.from_numpy(tl).to(dev))
        head.verify(logits[it], drafts[it], acc[it], nxt[it])
        head.rollback(cache, acc[it], K)
        last = nxt[it]
    torch.cuda.synchronize()
    rec_drafts, rec_acc = drafts.clone(), acc.clone()
    assert head.get_error() == 0
    log(f"{name}: recording pass done")

    def run(it, last):
        head.draft(hidden[it], last, cache, K, out=drafts[it])
        head.verify(logits[it], drafts[it], acc[it], nxt[it])
        head.rollback(cache, acc[it], K)
        return nxt[it]

    def replay(mask: int):
        cache.len.copy_(len0)
        cache.pos.copy_(pos0)
        last = last0
        head.set_profiling(0)
        for it in range(args.warmup):
            last = run(it, last)
        torch.cuda.synchronize()
        head.set_profiling(mask)
        t0 = time.perf_counter()
        for it in range(args.warmup, iters):
            last = run(it, last)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        head.set_profiling(0)
        return t1 - t0, head.get_profile()

    elapsed, _ = replay(0)
    if not (torch.equal(drafts, rec_drafts) and torch.equal(acc, rec_acc)):
        raise RuntimeError("timed replay diverged from the recording pass")
    log(f"{name}: timed pass: {args.steps} iterations in {elapsed * 1e3:.2f} ms")
    # Same replay with HIP events around every lm_head launch (on the library's stream).
    el_ev, prof = replay(LMHEAD_BIT)
    log(f"{name}: lm_head-event pass: {args.steps} iterations in {el_ev * 1e3:.2f} ms")

    acc_np = acc[args.warmup:].cpu().numpy().astype(np.int64)
    tokens = int((acc_np + 1).sum())
    ab = algorithmic_bytes(cfg, lens0, K, tokens // max(1, args.steps))
    it_s = elapsed / args.steps
    lm_ms, lm_n = prof["lm_head_argmax"]
    lm_avg_s = lm_ms / 1e3 / lm_n
    lm_gbs = ab["lm_head"] / lm_avg_s / 1e9
    res = {"workload": DESCR[name], "dtype": cfg.dtype, "batch": B, "K": K,
           "steps": args.steps, "warmup": args.warmup,
           "draft_steps_per_s": round(K * args.steps / elapsed, 3),
           "ms_per_iteration": round(it_s * 1e3, 4),
           "us_per_draft_step": round(it_s * 1e6 / K, 2),
           "verified_tok_per_s": round(tokens / elapsed, 2),
           "tokens_per_iteration": round(tokens / (args.steps * B), 4),
           "hbm_roofline_frac": round(ab["iteration"] / it_s / 1e9 / HBM_PEAK_GBS, 4),
           "algorithmic_bytes_per_iteration": int(ab["iteration"]),
           "lm_head": {"avg_launch_us": round(lm_avg_s * 1e6, 2), "launches": lm_n,
                       "achieved_gb_per_s": round(lm_gbs, 1),
                       "frac": round(lm_gbs / HBM_PEAK_GBS, 4),
                       "algorithmic_bytes_per_launch": int(ab["lm_head"])},
           "device_memory": memory}

    # The timed iterations captured once into a HIP graph (the entry points only launch
    # kernels) and replayed: the same kernels with no host-side launch work between them.
    # Capture runs nothing, so the state before each replay is the one after the eager
    # warm-up; the first replay is untimed, the second is timed and checked against the
    # recording.
    def graph_state():
        cache.len.copy_(len0)
        cache.pos.copy_(pos0)
        last = last0
        for it in range(args.warmup):
            last = run(it, last)
        drafts[args.warmup:].fill_(-1)
        acc[args.warmup:].fill_(-1)
        torch.cuda.synchronize()
        return last

    def graph_pass() -> dict:
        head.set_profiling(0)
        last_g = graph_state()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            lg = last_g
            for it in range(args.warmup, iters):
                lg = run(it, lg)
        torch.cuda.synchronize()
        graph.replay()
        graph_state()
        t0g = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        el_graph = time.perf_counter() - t0g
        same = torch.equal(drafts, rec_drafts) and torch.equal(acc, rec_acc)
        assert head.get_error() == 0
        del graph
        if not same:
            return {"error": "the graph replay diverged from the recording pass"}
        return {"draft_steps_per_s": round(K * args.steps / el_graph, 3),
                "ms_per_iteration": round(el_graph / args.steps * 1e3, 4),
                "hbm_roofline_frac": round(ab["iteration"] / (el_graph / args.steps) / 1e9
                                           / HBM_PEAK_GBS, 4),
                "vs_eager": round(elapsed / el_graph, 4),
                "tokens_identical": True}

    try:
        if not hot:
            res["graph_replay"] = graph_pass()
    except RuntimeError as e:  # a capture the runtime refuses: reported, the eager line stands
        res["graph_replay"] = {"error": str(e)[:200]}
    log(f"{name}: graph replay: {res.get('graph_replay', 'not run')}")

    if not full and info["packed_weight_bytes"] and not hot:
        # The same recorded iterations on a handle without the re-laid-out weight copy
        # (MTP_CREATE_NO_PACKED_COPY): the trade of workspace for speed, and a check that
        # the row-major path reproduces the recorded tokens bit for bit.
        lean = MtpHead(hidden=cfg.hidden, n_q_heads=cfg.n_q, n_kv_heads=cfg.n_kv,
                       head_dim=cfg.head_dim, ffn=cfg.ffn, vocab=cfg.vocab, weights=w,
                       max_batch=B, max_k=K, max_capacity=cap, rope_theta=cfg.rope_theta,
                       rms_eps=cfg.rms_eps, dtype=tdt, packed_copy=False)
        cache.len.copy_(len0)
        cache.pos.copy_(pos0)
        last = last0
        for it in range(iters):
            if it == args.warmup:
                torch.cuda.synchronize()
                t0l = time.perf_counter()
            lean.draft(hidden[it], last, cache, K, out=drafts[it])
            lean.verify(logits[it], drafts[it], acc[it], nxt[it])
            lean.rollback(cache, acc[it], K)
            last = nxt[it]
        torch.cuda.synchronize()
        el_lean = time.perf_counter() - t0l
        if not (torch.equal(drafts, rec_drafts) and torch.equal(acc, rec_acc)):
            raise RuntimeError("the handle without the packed copy diverged from the recording")
        assert lean.get_error() == 0
        # its verification from hidden states (row-major lm_head) on the same drafts
        th_l, tn_l = up(S.target_hidden(cfg, K)), up(S.target_norm(cfg))
        va = torch.empty(B, dtype=torch.int32, device=dev)
        vn = torch.empty(B, dtype=torch.int32, device=dev)
        for it in range(3):
            lean.verify_hidden(th_l, tn_l, drafts[it], va, vn)
        torch.cuda.synchronize()
        t0l = time.perf_counter()
        for it in range(args.steps):
            lean.verify_hidden(th_l, tn_l, drafts[args.warmup + it], va, vn)
        torch.cuda.synchronize()
        vh_lean_us = (time.perf_counter() - t0l) / args.steps * 1e6
        assert lean.get_error() == 0
        res["without_packed_copy"] = {
            "draft_steps_per_s": round(K * args.steps / el_lean, 3),
            "hbm_roofline_frac": round(ab["iteration"] / (el_lean / args.steps) / 1e9
                                       / HBM_PEAK_GBS, 4),
            "workspace_bytes": lean.info()["workspace_bytes"],
            "verify_from_hidden_us_per_call": round(vh_lean_us, 2),
            "verify_hidden_group_rows": lean.info()["verify_hidden_group_rows"],
            "tokens_identical": True}
        del th_l, tn_l
        log(f"{name}: without the packed copy: {res['without_packed_copy']}")
        lean.close()

    if full and not hot:
        # Per-call latency: HIP events (torch's current stream, which the library runs on)
        # bracket each ABI call of the same replay; median and 10th / 90th percentiles.
        cache.len.copy_(len0)
        cache.pos.copy_(pos0)
        last = last0
        for it in range(args.warmup):
            last = run(it, last)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
        for j, it in enumerate(range(args.warmup, iters)):
            e = ev[j]
            e[0].record()
            head.draft(hidden[it], last, cache, K, out=drafts[it])
            e[1].record()
            head.verify(logits[it], drafts[it], acc[it], nxt[it])
            e[2].record()
            head.rollback(cache, acc[it], K)
            e[3].record()
            last = nxt[it]
        torch.cuda.synchronize()

        def pct(vals):
            q = np.percentile(np.asarray(vals) * 1e3, [10, 50, 90])
            return {"p10": round(float(q[0]), 2), "p50": round(float(q[1]), 2),
                    "p90": round(float(q[2]), 2)}

        res["latency_us"] = {"samples": args.steps,
                             "draft": pct([e[0].elapsed_time(e[1]) for e in ev]),
                             "verify": pct([e[1].elapsed_time(e[2]) for e in ev]),
                             "rollback": pct([e[2].elapsed_time(e[3]) for e in ev]),
                             "iteration": pct([e[0].elapsed_time(e[3]) for e in ev])}
        log(f"{name}: per-call latency (us): {res['latency_us']}")
        if args.breakdown:
            _, bprof = replay((1 << 9) - 1)
            res["kernel_us_per_launch"] = {k: round(ms * 1e3 / n, 2)
                                           for k, (ms, n) in bprof.items() if n}
            log(f"{name}: per-kernel us/launch: {res['kernel_us_per_launch']}")
        res["_lm_head_prof"] = (lm_avg_s, lm_n, int(ab["lm_head"]), lm_gbs)

    if full:
        res.setdefault("_lm_head_prof", (lm_avg_s, lm_n, int(ab["lm_head"]), lm_gbs))

    if cfg.dtype == "bf16" and not hot:
        # Verification from the target's hidden states (the alternative to mtp_verify that
        # never materialises target logits): one call per recorded iteration's drafts.
        th = up(S.target_hidden(cfg, K))
        tn = up(S.target_norm(cfg))
        vacc = torch.empty(B, dtype=torch.int32, device=dev)
        vnxt = torch.empty(B, dtype=torch.int32, device=dev)
        for it in range(3):
            head.verify_hidden(th, tn, drafts[it], vacc, vnxt)
        torch.cuda.synchronize()
        t0v = time.perf_counter()
        for it in range(args.steps):
            head.verify_hidden(th, tn, drafts[args.warmup + it], vacc, vnxt)
        torch.cuda.synchronize()
        vh_us = (time.perf_counter() - t0v) / args.steps * 1e6
        vh_group = info["verify_hidden_group_rows"]
        vh_passes = -(-(B * (K + 1)) // vh_group)
        vh_bytes = vh_passes * cfg.vocab * cfg.hidden * esz + B * (K + 1) * cfg.hidden * esz
        res["verify_from_hidden"] = {
            "us_per_call": round(vh_us, 2), "rows": B * (K + 1), "rows_per_pass": vh_group,
            "algorithmic_bytes": int(vh_bytes),
            "hbm_frac": round(vh_bytes / (vh_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"{name}: verify from hidden states: {vh_us:.2f} us per call")
        # Exact cache catch-up (the alternative to rollback), on the recorded drafts and
        # accepted lengths, from the state right after a K-step draft.
        len_k, pos_k = len0 + K, pos0 + K
        cu_ms = []
        for it in range(args.steps + 2):
            cache.len.copy_(len_k)
            cache.pos.copy_(pos_k)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            head.catchup(cache, th, drafts[args.warmup + it % args.steps],
                         acc[args.warmup + it % args.steps])
            e1.record()
            e1.synchronize()
            if it >= 2:
                cu_ms.append(e0.elapsed_time(e1))
        res["kv_catchup"] = {"us_per_call": round(float(np.median(cu_ms)) * 1e3, 2),
                             "candidate_rows": B * K}
        assert head.get_error() == 0
        log(f"{name}: exact cache catch-up: {res['kv_catchup']['us_per_call']} us per call")

    if full and cfg.dtype == "bf16" and not hot:
        # Prompt prefill: a 4096-token prompt per sequence into an emptied cache.
        n = min(4096, cap)
        ph = up(S.prefill_hidden(cfg.with_(batch=1), n)).expand(B, n, cfg.hidden).contiguous()
        pt = torch.from_numpy(S.prefill_tokens(cfg.with_(batch=1), n)).to(dev).expand(B, n).contiguous()
        pf_ms = []
        for it in range(5):
            cache.len.zero_()
            cache.pos.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            head.prefill(cache, ph, pt)
            e1.record()
            e1.synchronize()
            if it >= 1:
                pf_ms.append(e0.elapsed_time(e1))
        assert head.get_error() == 0
        pf_us = float(np.median(pf_ms)) * 1e3
        H, kvd = cfg.hidden, cfg.n_kv * cfg.head_dim
        pf_bytes = (2 * H * H + 2 * kvd * H) * esz + B * n * (H * esz + 4 + H * esz + 2 * kvd * esz)
        # every prompt row goes through eh_proj (2H -> H) and the K / V projections (H -> 2 kvd):
        # with thousands of rows the call is bound by these multiply-adds, not by HBM
        pf_flops = 2.0 * B * n * (2 * H * H + 2 * kvd * H)
        pf_tflops = pf_flops / (pf_us * 1e-6) / 1e12
        res["prefill"] = {"prompt_tokens": n, "sequences": B, "us_per_call": round(pf_us, 1),
                          "prompt_tok_per_s": round(B * n / (pf_us * 1e-6), 1),
                          "rows_per_pass": info["catchup_group_rows"],
                          "algorithmic_flops": int(pf_flops),
                          "tflop_per_s": round(pf_tflops, 2),
                          "mfma_frac": round(pf_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                          "algorithmic_bytes": int(pf_bytes),
                          "hbm_frac": round(pf_bytes / (pf_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"{name}: prefill of {n} prompt tokens: {pf_us:.1f} us")
        del ph, pt

    if full and name == "q8b" and not hot:
        res["attention_large_cache"] = large_cache_probe(args, cfg, w, head, cache, hidden,
                                                         last0, len0, pos0)
    if full and not hot:
        res["sampling"] = sampling_pass(args, cfg, head, cache, hidden, last0, len0, pos0, up)
    if full:
        res["_inp"] = inp
    head.close()
    del w, cache, hidden, logits
    torch.cuda.empty_cache()
    return res


EXTRA_WORKLOADS = ("q8b-b32", "q32b", "wide", "tiny")


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="q8b", choices=sorted(DESCR))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time only the headline workload (not the other workloads)")
    ap.add_argument("--breakdown", action="store_true",
                    help="extra untimed pass with HIP events around every kernel class")
    ap.add_argument("--hot-only", action="store_true",
                    help="only the timed draft / verify / rollback iterations and the lm_head "
                         "events (no graph, lean-handle, verification-from-hidden, catch-up, "
                         "prefill, large-cache or sampling passes), for clean kernel traces")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU; --gpus must be 1 "
                                   "(the path shards by sequence with no exchange step)"}))
        return 2

    import mtp_synth as S

    cfg = S.get_config(args.config)
    head_res = run_workload(args.config, args, full=True)
    inp = head_res.pop("_inp")
    lm_avg_s, lm_n, lm_bytes, lm_gbs = head_res.pop("_lm_head_prof")
    out = {
        "metric": METRIC,
        "value": head_res["draft_steps_per_s"],
        "unit": "draft-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head_res["ms_per_iteration"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": DESCR[args.config], "name": args.config, "batch": cfg.batch,
                   "K": cfg.K},
        "verified_tok_per_s": head_res["verified_tok_per_s"],
        "tokens_per_iteration": head_res["tokens_per_iteration"],
        "hbm_roofline_frac": head_res["hbm_roofline_frac"],
        "algorithmic_bytes_per_iteration": head_res["algorithmic_bytes_per_iteration"],
        "roofline": {"bound": "hbm", "kernel": "lm_head_argmax",
                     "achieved": round(lm_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(lm_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(args.config),
                     "avg_launch_us": round(lm_avg_s * 1e6, 2), "launches": lm_n,
                     "algorithmic_bytes_per_launch": lm_bytes},
    }
    for k in ("us_per_draft_step", "latency_us", "kernel_us_per_launch", "verify_from_hidden",
              "kv_catchup", "prefill", "attention_large_cache", "sampling", "graph_replay",
              "device_memory"):
        if k in head_res:
            out[k] = head_res[k]
    if not args.no_extra:
        out["workloads"] = {}
        for name in EXTRA_WORKLOADS:
            if name == args.config:
                continue
            r = run_workload(name, args, full=False)
            out["workloads"][name] = r
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp, cfg.K, out["algorithmic_bytes_per_iteration"])
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
