"""The C-ABI library loads, exports every symbol include/mtp.h declares, and rejects bad
arguments on the host before touching a device. No device call is made here; the one
host-only computation (the step weights) is checked against its printed values."""
import ctypes
import subprocess

import numpy as np

import pytest

from mtp_self_speculative_amd import _lib as L


def cfg(**kw):
    base = dict(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288, vocab=151936,
                rope_theta=1e6, rms_eps=1e-6, dtype=L.MTP_BF16)
    base.update(kw)
    return L.make_config(**base)


def test_every_declared_symbol_is_exported():
    names = L.declared_symbols()
    assert {"mtp_draft", "mtp_verify", "mtp_kv_rollback"} <= set(names)
    for n in names:
        assert hasattr(L.LIB, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_no_unresolved_internal_symbols():
    out = subprocess.run(["nm", "-D", "--undefined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    assert "mtp" not in out, out


def test_status_strings():
    for s in range(8):
        assert L.mtp_status_string(s)
    assert "unknown" in L.mtp_status_string(99)


def _ws_status(c, mb=1, mk=5, cap=4416):
    n = ctypes.c_size_t(0)
    return L.LIB.mtp_workspace_size(ctypes.byref(c) if c is not None else None, mb, mk, cap,
                                    ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,mb,mk,cap,status", [
    (dict(), 1, 5, 4416, 0),
    (dict(dtype=7), 1, 5, 4416, 3),
    (dict(head_dim=96), 1, 5, 4416, 5),
    (dict(n_q_heads=30), 1, 5, 4416, 2),
    (dict(n_q_heads=64, n_kv_heads=4), 1, 5, 4416, 5),   # 16 query heads per KV head
    (dict(hidden=4100), 1, 5, 4416, 5),
    (dict(hidden=0), 1, 5, 4416, 2),
    (dict(rms_eps=0.0), 1, 5, 4416, 1),
    (dict(), 0, 5, 4416, 2),
    (dict(), 1, 101, 4416, 4),
    (dict(), 1, 5, 1 << 20, 4),
    (dict(), 1, -1, 4416, 2),
])
def test_workspace_size_validation(kw, mb, mk, cap, status):
    st, n = _ws_status(cfg(**kw), mb, mk, cap)
    assert st == status
    if status == 0:
        assert n > 0


def test_workspace_grows_with_batch_and_k():
    sizes = [L.mtp_workspace_size(cfg(), b, k, 4416) for b, k in [(1, 5), (8, 5), (8, 100)]]
    assert sizes[0] < sizes[1] < sizes[2]
    assert all(s % 256 == 0 for s in sizes)


def test_null_arguments_rejected_before_any_device_call():
    h = ctypes.c_void_p(0)
    w = L.mtp_weights()
    c = cfg()
    assert L.LIB.mtp_create(ctypes.byref(c), ctypes.byref(w), 1, 5, 4416, None, 0,
                            ctypes.byref(h)) == 1
    assert h.value is None
    assert L.LIB.mtp_create(None, ctypes.byref(w), 1, 5, 4416, None, 0, ctypes.byref(h)) == 1
    kv = L.mtp_kv()
    assert L.LIB.mtp_draft(None, None, None, ctypes.byref(kv), 1, 1, None, None) == 1
    assert L.LIB.mtp_draft_debug(None, None, None, ctypes.byref(kv), 1, 1, None, None, None,
                                 None, None) == 1
    assert L.LIB.mtp_verify(None, None, None, 1, 1, None, None, None) == 1
    assert L.LIB.mtp_verify_hidden(None, None, None, None, 1, 1, None, None, None) == 1
    assert L.LIB.mtp_kv_rollback(None, ctypes.byref(kv), None, 1, 1, None) == 1
    assert L.LIB.mtp_kv_catchup(None, ctypes.byref(kv), None, None, None, 1, 1, None) == 1
    assert L.LIB.mtp_draft_sample(None, None, None, ctypes.byref(kv), 1, 1, 1.0, None, 0, None,
                                  None, None) == 1
    assert L.LIB.mtp_verify_sample(None, None, None, None, 1, 1, 1.0, None, 0, None, None,
                                   None) == 1
    assert L.LIB.mtp_get_error(None, None, None) == 1
    L.LIB.mtp_destroy(None)


def test_python_wrapper_raises_mtp_error():
    with pytest.raises(L.MtpError) as e:
        L.mtp_workspace_size(cfg(head_dim=32), 1, 1, 16)
    assert e.value.status == 5


def test_step_weights_entry_point():
    """The library's host helper against the printed values and the closed form
    (speculators user guide, "MTP (Multi-Token Prediction)", Step Weight Formula)."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "step_weights.json")))
    w = L.mtp_step_weights(0.6, 3)
    assert [round(x, 2) for x in w] == [0.51, 0.31, 0.18]
    assert [round(x, 2) for x in w] == gold["printed"]
    assert np.allclose(w, [25 / 49, 15 / 49, 9 / 49], rtol=0, atol=1e-7)
    assert np.allclose(L.mtp_step_weights(1.0, 4), [0.25] * 4, atol=1e-7)
    w = L.mtp_step_weights(0.3, 100)
    assert abs(sum(w) - 1.0) < 1e-5 and all(a > b for a, b in zip(w, w[1:]) if b > 0)
    out = (ctypes.c_float * 4)(*([7.0] * 4))
    for beta, K, st in [(0.0, 3, 1), (-1.0, 3, 1), (float("nan"), 3, 1), (float("inf"), 3, 1),
                        (0.6, 0, 2), (0.6, 101, 2)]:
        assert L.LIB.mtp_step_weights(beta, K, out) == st
    assert list(out) == [7.0] * 4
    assert L.LIB.mtp_step_weights(0.6, 3, None) == 1


def test_adapt_k_entry_point():
    """The library's host rule against the hand-worked cases and the oracle."""
    import json
    import os
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "adapt_k_cases.json")))
    for c in gold["cases"]:
        assert L.mtp_adapt_k(c["accepted"], c["K"], c["k_min"], c["k_max"]) == c["k_next"], c
    out = ctypes.c_int32(-7)
    arr = (ctypes.c_int32 * 2)(1, 6)
    assert L.LIB.mtp_adapt_k(arr, 2, 5, 1, 8, ctypes.byref(out)) == 1  # accepted > K
    assert L.LIB.mtp_adapt_k(None, 2, 5, 1, 8, ctypes.byref(out)) == 1
    assert L.LIB.mtp_adapt_k(arr, 0, 5, 1, 8, ctypes.byref(out)) == 2
    assert L.LIB.mtp_adapt_k(arr, 2, 5, 4, 3, ctypes.byref(out)) == 2
    assert L.LIB.mtp_adapt_k(arr, 2, 5, 1, 101, ctypes.byref(out)) == 2
    assert out.value == -7


def _cpu_head(B=3, K=4, H=64, V=100, n_q=2, n_kv=1, d=64, F=128, dtype=None):
    """An MtpHead whose checks accept CPU tensors and whose handle is null: a call that
    passes the host-side checks reaches the library, which rejects the null handle."""
    import torch
    from mtp_self_speculative_amd.head import MtpHead
    h = object.__new__(MtpHead)
    h._device_type = "cpu"
    h.dtype = dtype or torch.bfloat16
    h.cfg = L.make_config(H, n_q, n_kv, d, F, V, 1e6, 1e-6, L.MTP_BF16)
    h.max_batch, h.max_k, h.max_capacity = B, K, 64
    h.handle = None
    return h


class _Stream:
    cuda_stream = 0


def test_head_rejects_mismatched_tensors_before_the_library():
    """Wrong shape, dtype, device or layout raises ValueError on the host (the kernels
    would otherwise read or write past the buffers); well-formed arguments reach the
    library, which returns MTP_ERR_INVALID_ARG for the null handle."""
    import torch
    from mtp_self_speculative_amd.head import MtpCache
    B, K, H, V = 3, 4, 64, 100
    h = _cpu_head(B, K, H, V)
    s = _Stream()
    i32 = torch.int32
    cache = MtpCache(torch.zeros((B, 1, 16, 64), dtype=torch.bfloat16),
                     torch.zeros((B, 1, 16, 64), dtype=torch.bfloat16),
                     torch.zeros(B, dtype=i32), torch.zeros(B, dtype=i32))
    hid = torch.zeros((B, H), dtype=torch.bfloat16)
    lt = torch.zeros(B, dtype=i32)
    logits = torch.zeros((B, K + 1, V), dtype=torch.float32)
    d = torch.zeros((B, K), dtype=i32)
    acc = torch.zeros(B, dtype=i32)
    th = torch.zeros((B, K + 1, H), dtype=torch.bfloat16)
    tn = torch.zeros(H, dtype=torch.bfloat16)
    bad = [
        lambda: h.verify(torch.zeros((B, K + 1, V - 1)), d, stream=s),        # short rows
        lambda: h.verify(logits.double(), d, stream=s),                        # dtype
        lambda: h.verify(logits, d.long(), stream=s),                          # int64 drafts
        lambda: h.verify(logits, d[:, :K - 1].contiguous(), stream=s),         # drafts short
        lambda: h.verify(logits, d, acc[:B - 1], stream=s),                    # accepted short
        lambda: h.verify(logits, None, stream=s),                              # drafts missing
        lambda: h.verify(torch.zeros((B, K + 2, V)), None, stream=s),          # K > max_k
        lambda: h.verify(logits.transpose(0, 1).contiguous().transpose(0, 1), d, stream=s),
        lambda: h.draft(hid.float(), lt, cache, K, stream=s),                  # hidden dtype
        lambda: h.draft(hid[:, :H - 8].contiguous(), lt, cache, K, stream=s),  # hidden width
        lambda: h.draft(hid, lt.long(), cache, K, stream=s),                   # token dtype
        lambda: h.draft(hid, lt[:2].contiguous(), cache, K, stream=s),         # tokens short
        lambda: h.draft(hid, lt, cache, K + 1, stream=s),                      # K > max_k
        lambda: h.verify_hidden(th.float(), tn, d, stream=s),
        lambda: h.verify_hidden(th, tn[:H // 2].contiguous(), d, stream=s),
        lambda: h.verify_hidden(th[:, :, :H - 8].contiguous(), tn, d, stream=s),
        lambda: h.catchup(cache, th, d, acc.long(), stream=s),
        lambda: h.catchup(cache, th[:, :1].contiguous(), d[:, :0].contiguous(), acc, stream=s),
        lambda: h.rollback(cache, acc.long(), K, stream=s),
        lambda: h.rollback(cache, torch.zeros(B + 1, dtype=i32), K, stream=s),
        lambda: h.draft_sample(hid, lt, cache, K, 1.0, torch.zeros(B, dtype=i32), 0, stream=s),
        lambda: h.verify_sample(logits, torch.zeros((B, K, V - 1)), d, 1.0,
                                torch.zeros(B, dtype=torch.int64), 0, stream=s),
    ]
    for i, f in enumerate(bad):
        with pytest.raises(ValueError):
            f()
    bad_cache = MtpCache(torch.zeros((B, 2, 16, 64), dtype=torch.bfloat16),
                         torch.zeros((B, 2, 16, 64), dtype=torch.bfloat16),
                         torch.zeros(B, dtype=i32), torch.zeros(B, dtype=i32))
    with pytest.raises(ValueError):                                            # n_kv mismatch
        h.draft(hid, lt, bad_cache, K, stream=s)
    with pytest.raises(ValueError):
        MtpCache(torch.zeros((B, 1, 16, 64)), torch.zeros((B, 1, 16, 64)),
                 torch.zeros(B, dtype=torch.int64), torch.zeros(B, dtype=i32))
    good = [
        lambda: h.verify(logits, d, stream=s),
        lambda: h.draft(hid, lt, cache, K, stream=s),
        lambda: h.verify_hidden(th, tn, d, stream=s),
        lambda: h.catchup(cache, th, d, acc, stream=s),
        lambda: h.rollback(cache, acc, K, stream=s),
    ]
    for f in good:
        with pytest.raises(L.MtpError) as e:
            f()
        assert e.value.status == 1


def test_get_info_rejects_null():
    info = L.mtp_info()
    assert L.LIB.mtp_get_info(None, ctypes.byref(info)) == 1


def test_verify_noalloc_host_checks():
    """Argument checks of the allocation-free verification happen before any device call."""
    p = ctypes.c_void_p(16)
    assert L.LIB.mtp_verify_noalloc(None, p, 1, 1, 8, p, p, None) == 1
    assert L.LIB.mtp_verify_noalloc(p, None, 1, 1, 8, p, p, None) == 1
    assert L.LIB.mtp_verify_noalloc(p, p, 0, 1, 8, p, p, None) == 2
    assert L.LIB.mtp_verify_noalloc(p, p, 1, -1, 8, p, p, None) == 2
    assert L.LIB.mtp_verify_noalloc(p, p, 1, 1, 0, p, p, None) == 2
    assert L.LIB.mtp_verify_noalloc(p, p, 257, 1, 8, p, p, None) == 4
    assert L.LIB.mtp_verify_noalloc(p, p, 1, 101, 8, p, p, None) == 4


def test_prefill_host_checks():
    """mtp_kv_prefill refuses a null handle and bad shapes before any device call."""
    kv = L.mtp_kv()
    p = ctypes.c_void_p(16)
    assert L.LIB.mtp_kv_prefill(None, ctypes.byref(kv), p, p, None, 1, 4, None) == 1


def test_adapt_k_seq_entry_point():
    """The library's per-sequence window rule against the hand-worked cases and the oracle."""
    import json
    import os
    from oracle import mtp_oracle as O
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "adapt_k_seq_cases.json")))
    for c in gold["cases"]:
        assert L.mtp_adapt_k_seq(c["accepted"], c["k"], c["k_min"], c["k_max"]) == c["k_next"], c
    rng = np.random.default_rng(3)
    for _ in range(200):
        W, B = int(rng.integers(1, 6)), int(rng.integers(1, 9))
        k = rng.integers(0, 9, size=(W, B))
        a = (rng.random((W, B)) * (k + 1)).astype(int)
        kmin = int(rng.integers(0, 3))
        kmax = int(rng.integers(kmin, 12))
        assert L.mtp_adapt_k_seq(a.tolist(), k.tolist(), kmin, kmax) == \
            O.adapt_k_seq(a, k, kmin, kmax).tolist()
    out = (ctypes.c_int32 * 2)(-7, -7)
    a = (ctypes.c_int32 * 2)(1, 3)
    k = (ctypes.c_int32 * 2)(2, 2)                      # accepted 3 > k 2
    assert L.LIB.mtp_adapt_k_seq(a, k, 1, 2, 1, 5, out) == 1
    assert L.LIB.mtp_adapt_k_seq(None, k, 1, 2, 1, 5, out) == 1
    assert L.LIB.mtp_adapt_k_seq(a, k, 0, 2, 1, 5, out) == 2
    assert L.LIB.mtp_adapt_k_seq(a, k, 1, 2, 3, 2, out) == 2
    assert L.LIB.mtp_adapt_k_seq(a, k, 1, 2, 1, 101, out) == 2
    assert list(out) == [-7, -7]


def test_seqk_entry_points_reject_null_arguments():
    kv = L.mtp_kv()
    p = ctypes.c_void_p(16)
    assert L.LIB.mtp_draft_seqk(None, p, p, ctypes.byref(kv), p, 1, 1, p, None) == 1
    assert L.LIB.mtp_verify_seqk(None, p, p, p, 1, 1, p, p, None) == 1
    assert L.LIB.mtp_kv_rollback_seqk(None, ctypes.byref(kv), p, p, 1, 1, None) == 1


def _packed_bytes(c):
    """Size of the re-laid-out copy: 128 x 256 blocks of every matrix of the batched path."""
    def blocks(rows, cols):
        return -(-rows // 128) * -(-cols // 256) * 128 * 256 * 2
    H, qd, kvd = c.hidden, c.n_q_heads * c.head_dim, c.n_kv_heads * c.head_dim
    return (blocks(H, 2 * H) + blocks(qd + 2 * kvd, H) + blocks(H, qd) + blocks(2 * c.ffn, H)
            + blocks(H, c.ffn) + blocks(c.vocab, H))


def test_workspace_without_packed_copy():
    c = cfg()
    assert L.mtp_workspace_size_ex(c, 8, 5, 4416, 0) == L.mtp_workspace_size(c, 8, 5, 4416)
    full = L.mtp_workspace_size(c, 8, 5, 4416)
    lean = L.mtp_workspace_size_ex(c, 8, 5, 4416, L.CREATE_NO_PACKED_COPY)
    assert lean % 256 == 0
    # the copy (1.7 GB here) goes; the 128-row verification group shrinks to 64 rows
    assert full - lean >= _packed_bytes(c)
    assert full - lean < _packed_bytes(c) + (64 << 20)
    # handles that never hold the copy are unchanged by the flag
    for c2, mb in ((cfg(), 2), (cfg(dtype=L.MTP_F32), 8)):
        assert (L.mtp_workspace_size_ex(c2, mb, 5, 4416, L.CREATE_NO_PACKED_COPY)
                == L.mtp_workspace_size(c2, mb, 5, 4416))


def test_unknown_create_flags_rejected_before_any_device_call():
    c = cfg()
    n = ctypes.c_size_t(0)
    assert L.LIB.mtp_workspace_size_ex(ctypes.byref(c), 8, 5, 4416, 2, ctypes.byref(n)) == 1
    h = ctypes.c_void_p(0)
    w = L.mtp_weights()
    assert L.LIB.mtp_create_ex(ctypes.byref(c), ctypes.byref(w), 8, 5, 4416, 0x80000000, None, 0,
                               ctypes.byref(h)) == 1
    assert h.value is None
    assert L.LIB.mtp_create_ex(ctypes.byref(c), ctypes.byref(w), 8, 5, 4416,
                               L.CREATE_NO_PACKED_COPY, None, 0, ctypes.byref(h)) == 1
    assert L.LIB.mtp_refresh_weights(None, None) == 1
