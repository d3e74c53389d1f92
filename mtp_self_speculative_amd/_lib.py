"""ctypes binding of libmtp.so (the C ABI in include/mtp.h).

Argument marshalling only: every step of the draft / verify / rollback path runs
in the library's HIP kernels. Functions keep the C names; tensors are passed as
device pointers (``tensor.data_ptr()``) and the stream as a hipStream_t handle.
There is no fallback: if the library is missing or fails to load, importing this
module raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MTP_LIB", os.path.join(_HERE, "libmtp.so"))
HEADER = os.path.join(os.path.dirname(_HERE), "include", "mtp.h")

MTP_OK = 0
MTP_F32, MTP_BF16 = 0, 1
DEVERR_TOKEN, DEVERR_CAPACITY, DEVERR_ACCEPT, DEVERR_COUNT = 1, 2, 4, 8
CREATE_NO_PACKED_COPY = 1  # MTP_CREATE_NO_PACKED_COPY

STATUS_NAMES = {0: "MTP_OK", 1: "MTP_ERR_INVALID_ARG", 2: "MTP_ERR_SHAPE", 3: "MTP_ERR_DTYPE",
                4: "MTP_ERR_CAPACITY", 5: "MTP_ERR_UNSUPPORTED", 6: "MTP_ERR_HIP",
                7: "MTP_ERR_DEVICE"}

WEIGHT_FIELDS = ("g_h", "g_e", "w_eh", "g_attn", "w_q", "w_k", "w_v", "w_o", "g_mlp", "w_gate",
                 "w_up", "w_down", "g_final", "embed", "lm_head")


class MtpError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, where: str, message: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({message})")


class mtp_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class mtp_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class mtp_kv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_void_p),
                ("pos", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("capacity", ctypes.c_int32)]


class mtp_info(ctypes.Structure):
    _fields_ = [("workspace_bytes", ctypes.c_size_t), ("packed_weight_bytes", ctypes.c_size_t),
                ("verify_hidden_group_rows", ctypes.c_int32),
                ("catchup_group_rows", ctypes.c_int32),
                ("matrix_core_min_batch", ctypes.c_int32),
                ("matrix_core_max_batch", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SIGS = {
    "mtp_workspace_size": (_I, [ctypes.POINTER(mtp_config), _I, _I, _I,
                                ctypes.POINTER(ctypes.c_size_t)]),
    "mtp_create": (_I, [ctypes.POINTER(mtp_config), ctypes.POINTER(mtp_weights), _I, _I, _I, _P,
                        ctypes.c_size_t, ctypes.POINTER(_P)]),
    "mtp_workspace_size_ex": (_I, [ctypes.POINTER(mtp_config), _I, _I, _I, ctypes.c_uint32,
                                   ctypes.POINTER(ctypes.c_size_t)]),
    "mtp_create_ex": (_I, [ctypes.POINTER(mtp_config), ctypes.POINTER(mtp_weights), _I, _I, _I,
                           ctypes.c_uint32, _P, ctypes.c_size_t, ctypes.POINTER(_P)]),
    "mtp_refresh_weights": (_I, [_P, _P]),
    "mtp_draft": (_I, [_P, _P, _P, ctypes.POINTER(mtp_kv), _I, _I, _P, _P]),
    "mtp_draft_debug": (_I, [_P, _P, _P, ctypes.POINTER(mtp_kv), _I, _I, _P, _P, _P, _P, _P]),
    "mtp_verify": (_I, [_P, _P, _P, _I, _I, _P, _P, _P]),
    "mtp_verify_hidden": (_I, [_P, _P, _P, _P, _I, _I, _P, _P, _P]),
    "mtp_draft_sample": (_I, [_P, _P, _P, ctypes.POINTER(mtp_kv), _I, _I, ctypes.c_float, _P,
                              ctypes.c_uint64, _P, _P, _P]),
    "mtp_verify_sample": (_I, [_P, _P, _P, _P, _I, _I, ctypes.c_float, _P, ctypes.c_uint64, _P,
                               _P, _P]),
    "mtp_kv_catchup": (_I, [_P, ctypes.POINTER(mtp_kv), _P, _P, _P, _I, _I, _P]),
    "mtp_kv_rollback": (_I, [_P, ctypes.POINTER(mtp_kv), _P, _I, _I, _P]),
    "mtp_kv_prefill": (_I, [_P, ctypes.POINTER(mtp_kv), _P, _P, _P, _I, _I, _P]),
    "mtp_get_error": (_I, [_P, _P, ctypes.POINTER(ctypes.c_uint32)]),
    "mtp_get_info": (_I, [_P, ctypes.POINTER(mtp_info)]),
    "mtp_verify_noalloc": (_I, [_P, _P, _I, _I, _I, _P, _P, _P]),
    "mtp_set_profiling": (_I, [_P, ctypes.c_uint32]),
    "mtp_get_profile": (_I, [_P, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_I), _I]),
    "mtp_destroy": (None, [_P]),
    "mtp_status_string": (ctypes.c_char_p, [_I]),
    "mtp_step_weights": (_I, [ctypes.c_float, _I, ctypes.POINTER(ctypes.c_float)]),
    "mtp_adapt_k": (_I, [ctypes.POINTER(_I), _I, _I, _I, _I, ctypes.POINTER(_I)]),
    "mtp_adapt_k_seq": (_I, [ctypes.POINTER(_I), ctypes.POINTER(_I), _I, _I, _I, _I,
                             ctypes.POINTER(_I)]),
    "mtp_draft_seqk": (_I, [_P, _P, _P, ctypes.POINTER(mtp_kv), _P, _I, _I, _P, _P]),
    "mtp_verify_seqk": (_I, [_P, _P, _P, _P, _I, _I, _P, _P, _P]),
    "mtp_kv_rollback_seqk": (_I, [_P, ctypes.POINTER(mtp_kv), _P, _P, _I, _I, _P]),
}


def declared_symbols(header: str = HEADER) -> list[str]:
    """Names of the functions include/mtp.h declares."""
    txt = open(header).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(mtp_[a-z_]+)\s*\(", txt)))


def _hip_runtimes() -> set[str]:
    try:
        with open("/proc/self/maps") as f:
            return {ln.split()[-1] for ln in f if "libamdhip64" in ln}
    except OSError:  # pragma: no cover
        return set()


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmtp.so not found at {LIB_PATH}; build it with "
                          "`python -m mtp_self_speculative_amd.build` (hipcc, gfx950)")
    # Device memory and streams come from PyTorch, so the library must bind to the HIP
    # runtime PyTorch loaded: load torch first, and the library's libamdhip64.so.7
    # dependency resolves (by soname) to that same runtime instead of a second copy.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    if len(_hip_runtimes()) > 1:
        raise ImportError("two HIP runtimes are loaded in this process "
                          f"({sorted(_hip_runtimes())}); libmtp.so must share PyTorch's")
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def status_string(st: int) -> str:
    return LIB.mtp_status_string(st).decode()


def _check(st: int, where: str) -> None:
    if st != MTP_OK:
        raise MtpError(st, where, status_string(st))


def make_config(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, rope_theta, rms_eps,
                dtype) -> mtp_config:
    return mtp_config(hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab, rope_theta, rms_eps,
                      dtype)


def mtp_workspace_size(cfg: mtp_config, max_batch: int, max_k: int, max_capacity: int) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.mtp_workspace_size(ctypes.byref(cfg), max_batch, max_k, max_capacity,
                                  ctypes.byref(n)), "mtp_workspace_size")
    return int(n.value)


def mtp_create(cfg: mtp_config, weights: mtp_weights, max_batch: int, max_k: int,
               max_capacity: int, workspace: int, workspace_bytes: int) -> int:
    h = ctypes.c_void_p(0)
    _check(LIB.mtp_create(ctypes.byref(cfg), ctypes.byref(weights), max_batch, max_k,
                          max_capacity, workspace, workspace_bytes, ctypes.byref(h)),
           "mtp_create")
    return h.value


def mtp_workspace_size_ex(cfg: mtp_config, max_batch: int, max_k: int, max_capacity: int,
                          flags: int) -> int:
    n = ctypes.c_size_t(0)
    _check(LIB.mtp_workspace_size_ex(ctypes.byref(cfg), max_batch, max_k, max_capacity, flags,
                                     ctypes.byref(n)), "mtp_workspace_size_ex")
    return int(n.value)


def mtp_create_ex(cfg: mtp_config, weights: mtp_weights, max_batch: int, max_k: int,
                  max_capacity: int, flags: int, workspace: int, workspace_bytes: int) -> int:
    h = ctypes.c_void_p(0)
    _check(LIB.mtp_create_ex(ctypes.byref(cfg), ctypes.byref(weights), max_batch, max_k,
                             max_capacity, flags, workspace, workspace_bytes, ctypes.byref(h)),
           "mtp_create_ex")
    return h.value


def mtp_refresh_weights(handle: int, stream: int | None) -> None:
    _check(LIB.mtp_refresh_weights(handle, stream), "mtp_refresh_weights")


def mtp_draft(handle: int, hidden: int, last_tokens: int, kv: mtp_kv, B: int, K: int,
              draft_tokens: int, stream: int | None) -> None:
    _check(LIB.mtp_draft(handle, hidden, last_tokens, ctypes.byref(kv), B, K, draft_tokens,
                         stream), "mtp_draft")


def mtp_draft_debug(handle: int, hidden: int, last_tokens: int, kv: mtp_kv, B: int, K: int,
                    draft_tokens: int, hidden_out: int | None, top2_out: int | None,
                    logits_out: int | None, stream: int | None) -> None:
    _check(LIB.mtp_draft_debug(handle, hidden, last_tokens, ctypes.byref(kv), B, K, draft_tokens,
                               hidden_out, top2_out, logits_out, stream), "mtp_draft_debug")


def mtp_verify(handle: int, target_logits: int, draft_tokens: int | None, B: int, K: int,
               accepted_len: int, next_token: int, stream: int | None) -> None:
    _check(LIB.mtp_verify(handle, target_logits, draft_tokens, B, K, accepted_len, next_token,
                          stream), "mtp_verify")


def mtp_verify_noalloc(target_logits: int, draft_tokens: int | None, B: int, K: int, vocab: int,
                       accepted_len: int, next_token: int, stream: int | None) -> None:
    _check(LIB.mtp_verify_noalloc(target_logits, draft_tokens, B, K, vocab, accepted_len,
                                  next_token, stream), "mtp_verify_noalloc")


def mtp_draft_sample(handle: int, hidden: int, last_tokens: int, kv: mtp_kv, B: int, K: int,
                     temperature: float, seeds: int | None, offset: int, draft_tokens: int,
                     draft_logits: int | None, stream: int | None) -> None:
    _check(LIB.mtp_draft_sample(handle, hidden, last_tokens, ctypes.byref(kv), B, K, temperature,
                                seeds, offset, draft_tokens, draft_logits, stream),
           "mtp_draft_sample")


def mtp_verify_sample(handle: int, target_logits: int, draft_logits: int | None,
                      draft_tokens: int | None, B: int, K: int, temperature: float,
                      seeds: int | None, offset: int, accepted_len: int, next_token: int,
                      stream: int | None) -> None:
    _check(LIB.mtp_verify_sample(handle, target_logits, draft_logits, draft_tokens, B, K,
                                 temperature, seeds, offset, accepted_len, next_token, stream),
           "mtp_verify_sample")


def mtp_verify_hidden(handle: int, target_hidden: int, target_norm: int,
                      draft_tokens: int | None, B: int, K: int, accepted_len: int,
                      next_token: int, stream: int | None) -> None:
    _check(LIB.mtp_verify_hidden(handle, target_hidden, target_norm, draft_tokens, B, K,
                                 accepted_len, next_token, stream), "mtp_verify_hidden")


def mtp_kv_catchup(handle: int, kv: mtp_kv, target_hidden: int, draft_tokens: int,
                   accepted_len: int, B: int, K: int, stream: int | None) -> None:
    _check(LIB.mtp_kv_catchup(handle, ctypes.byref(kv), target_hidden, draft_tokens,
                              accepted_len, B, K, stream), "mtp_kv_catchup")


def mtp_kv_prefill(handle: int, kv: mtp_kv, target_hidden: int, tokens: int,
                   n_valid: int | None, B: int, n: int, stream: int | None) -> None:
    _check(LIB.mtp_kv_prefill(handle, ctypes.byref(kv), target_hidden, tokens, n_valid, B, n,
                              stream), "mtp_kv_prefill")


def mtp_kv_rollback(handle: int, kv: mtp_kv, accepted_len: int, B: int, K: int,
                    stream: int | None) -> None:
    _check(LIB.mtp_kv_rollback(handle, ctypes.byref(kv), accepted_len, B, K, stream),
           "mtp_kv_rollback")


def mtp_get_error(handle: int, stream: int | None) -> int:
    """Synchronise, read and clear the device error word; returns its bits (0 = none)."""
    bits = ctypes.c_uint32(0)
    st = LIB.mtp_get_error(handle, stream, ctypes.byref(bits))
    if st not in (MTP_OK, 7):
        _check(st, "mtp_get_error")
    return int(bits.value)


def mtp_get_info(handle: int) -> dict:
    """Workspace bytes, packed-copy bytes and row grouping of a handle (host only)."""
    info = mtp_info()
    _check(LIB.mtp_get_info(handle, ctypes.byref(info)), "mtp_get_info")
    return {n: int(getattr(info, n)) for n, _ in mtp_info._fields_}


KERNEL_CLASSES = ("eh_proj", "qkv", "attention", "o_proj", "gate_up", "down", "lm_head_argmax",
                  "verify", "rollback")


def mtp_set_profiling(handle: int, mask: int) -> None:
    _check(LIB.mtp_set_profiling(handle, mask), "mtp_set_profiling")


def mtp_get_profile(handle: int) -> dict:
    """{kernel class: (summed ms, launches)} since the previous call."""
    n = len(KERNEL_CLASSES)
    ms = (ctypes.c_float * n)()
    cnt = (_I * n)()
    _check(LIB.mtp_get_profile(handle, ms, cnt, n), "mtp_get_profile")
    return {KERNEL_CLASSES[i]: (float(ms[i]), int(cnt[i])) for i in range(n)}


def mtp_destroy(handle: int) -> None:
    if handle:
        LIB.mtp_destroy(handle)


def mtp_status_string(st: int) -> str:
    return status_string(st)


def mtp_adapt_k(accepted_len, K: int, k_min: int, k_max: int) -> int:
    """Next speculative length from the accepted lengths (host sequence of ints)."""
    a = [int(x) for x in accepted_len]
    arr = (_I * max(len(a), 1))(*a)
    out = _I(0)
    _check(LIB.mtp_adapt_k(arr, len(a), int(K), int(k_min), int(k_max), ctypes.byref(out)),
           "mtp_adapt_k")
    return int(out.value)


def mtp_step_weights(beta: float, K: int) -> list:
    """Training-loss weights of the K MTP steps (host computation in the library)."""
    out = (ctypes.c_float * max(int(K), 1))()
    _check(LIB.mtp_step_weights(float(beta), int(K), out), "mtp_step_weights")
    return [float(out[i]) for i in range(int(K))]


def mtp_draft_seqk(handle: int, hidden: int, last_tokens: int, kv: mtp_kv, k_seq: int, B: int,
                   K_max: int, draft_tokens: int, stream: int | None) -> None:
    _check(LIB.mtp_draft_seqk(handle, hidden, last_tokens, ctypes.byref(kv), k_seq, B, K_max,
                              draft_tokens, stream), "mtp_draft_seqk")


def mtp_verify_seqk(handle: int, target_logits: int, draft_tokens: int | None, k_seq: int, B: int,
                    K_max: int, accepted_len: int, next_token: int, stream: int | None) -> None:
    _check(LIB.mtp_verify_seqk(handle, target_logits, draft_tokens, k_seq, B, K_max,
                               accepted_len, next_token, stream), "mtp_verify_seqk")


def mtp_kv_rollback_seqk(handle: int, kv: mtp_kv, accepted_len: int, k_seq: int, B: int,
                         K_max: int, stream: int | None) -> None:
    _check(LIB.mtp_kv_rollback_seqk(handle, ctypes.byref(kv), accepted_len, k_seq, B, K_max,
                                    stream), "mtp_kv_rollback_seqk")


def mtp_adapt_k_seq(accepted_hist, k_hist, k_min: int, k_max: int) -> list:
    """Per-sequence lengths from the last W iterations' accepted lengths and lengths
    (host nested sequences [W][B])."""
    a = [[int(x) for x in row] for row in accepted_hist]
    k = [[int(x) for x in row] for row in k_hist]
    W, B = len(a), len(a[0]) if a else 0
    fa = (_I * max(W * B, 1))(*[x for row in a for x in row])
    fk = (_I * max(W * B, 1))(*[x for row in k for x in row])
    out = (_I * max(B, 1))()
    _check(LIB.mtp_adapt_k_seq(fa, fk, W, B, int(k_min), int(k_max), out), "mtp_adapt_k_seq")
    return [int(out[i]) for i in range(B)]
