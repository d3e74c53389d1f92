"""The allocation-free verification entry point (mtp_verify_noalloc) against the
workspace-backed one (mtp_verify) and the oracle, through the C ABI: bit-exact accepted
lengths and next tokens on consecutive calls, the later ones smaller, so that whatever an
earlier call left in the shared device array cannot leak into a later one."""
import numpy as np
import pytest

import mtp_synth as S
from gpu_util import make_head, small
from oracle import mtp_oracle as O

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from mtp_self_speculative_amd import _lib as L  # noqa: E402


def _case(B, K, V, seed):
    cfg = small(name="na", cid=190 + seed, batch=B, vocab=V, K=max(K, 1), agree_lo=0.8)
    rng = np.random.default_rng(seed)
    d = rng.integers(0, V, size=(B, K)).astype(np.int32)
    t = S.plant_target_logits(cfg, d, seed)[:, :K + 1]
    for b in range(0, B, 5):  # two equal maxima: the lower index must win
        j = b % (K + 1)
        t[b, j, 3] = t[b, j, V - 2] = 60.0
    return np.ascontiguousarray(t), d


def _noalloc(t, d, B, K, V):
    tl = torch.from_numpy(t).cuda()
    dt = torch.from_numpy(d).cuda() if K else None
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    nxt = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    L.mtp_verify_noalloc(tl.data_ptr(), None if dt is None else dt.data_ptr(), B, K, V,
                         acc.data_ptr(), nxt.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), nxt.cpu().numpy()


def _with_handle(t, d, B, K, V):
    inp = S.make_inputs(small(name="nah", cid=199, vocab=V, batch=B, K=max(K, 1), ctx_lo=1,
                              ctx_hi=None, hidden=64, n_q=2, n_kv=1, ffn=64), capacity=128)
    head, _ = make_head(inp.cfg, inp, max_batch=B, max_k=max(K, 1))
    acc, nxt = head.verify(torch.from_numpy(t).cuda(), torch.from_numpy(d).cuda() if K else None)
    torch.cuda.synchronize()
    assert head.get_error() == 0
    out = acc.cpu().numpy(), nxt.cpu().numpy()
    head.close()
    return out


def test_noalloc_matches_mtp_verify_on_consecutive_calls():
    # the largest batch first, then smaller ones (fewer rows, a shorter key stride, K = 0)
    for (B, K, V, seed) in [(256, 3, 5003, 1), (64, 5, 151936, 2), (7, 2, 4099, 3),
                            (3, 0, 1000, 4), (2, 100, 257, 5)]:
        t, d = _case(B, K, V, seed)
        print(f"noalloc case B={B} K={K} V={V}", flush=True)
        a_n, n_n = _noalloc(t, d, B, K, V)
        a_h, n_h = _with_handle(t, d, B, K, V)
        a_o, n_o = O.verify(t, d)
        assert np.array_equal(a_n, a_h) and np.array_equal(n_n, n_h), (B, K, V)
        assert np.array_equal(a_n, a_o) and np.array_equal(n_n, n_o), (B, K, V)
        # the same call again gives the same result (the array was cleared and reused)
        a2, n2 = _noalloc(t, d, B, K, V)
        assert np.array_equal(a2, a_n) and np.array_equal(n2, n_n)


def test_noalloc_host_limits():
    z = torch.zeros(4, dtype=torch.int32, device="cuda")
    f = torch.zeros((1, 2, 8), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert L.LIB.mtp_verify_noalloc(f.data_ptr(), z.data_ptr(), 257, 1, 8, z.data_ptr(),
                                    z.data_ptr(), s) == 4
    assert L.LIB.mtp_verify_noalloc(f.data_ptr(), z.data_ptr(), 1, 101, 8, z.data_ptr(),
                                    z.data_ptr(), s) == 4
    assert L.LIB.mtp_verify_noalloc(f.data_ptr(), None, 1, 1, 8, z.data_ptr(), z.data_ptr(),
                                    s) == 1
