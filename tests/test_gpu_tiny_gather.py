"""GPU checks of the tiny loop's compacted cache: vc_gather_evict, which
computes the kept positions from the committed length on the device, and
vc_gather_rows, which takes them as a list, copy exactly the rows of the
oracle's kept set (bit for bit, K token-major and V in 32-token blocks) and
set the kept count, for committed lengths from 0 to a full cache."""
import numpy as np
import pytest

from oracle import tiny

pytestmark = pytest.mark.gpu


def _caches(Hkv, cap, D, seed):
    import torch
    g = np.random.default_rng(seed)
    k = torch.from_numpy(g.standard_normal((Hkv, cap, D), dtype=np.float32)).cuda()
    v = torch.from_numpy(g.standard_normal((Hkv, D, cap), dtype=np.float32)).cuda()
    return k, v


def _check(dk, dv, dl, k, v, kept):
    n = len(kept)
    Hkv, _, D = k.shape
    np.testing.assert_array_equal(dl.cpu().numpy(), np.full(Hkv, n))
    dk, dv, k, v = (t.cpu().numpy() for t in (dk, dv, k, v))
    np.testing.assert_array_equal(dk[:, :n], k[:, kept])
    dv_tok = dv.transpose(0, 1, 3, 2).reshape(Hkv, -1, D)        # [Hkv][ccap][D]
    np.testing.assert_array_equal(dv_tok[:, :n], v.transpose(0, 2, 1)[:, kept])


@pytest.mark.parametrize("rule", [(4, 128, 8), (4, 32, 8), (0, 0, 1)])
def test_gather_evict_equals_oracle_kept_rows(rule):
    import torch
    from lossless_speculative_decoding_vc_amd.tiny_loop import evict_kept_count, gather_evict
    Hkv, cap, D = 2, 1152, 64
    k, v = _caches(Hkv, cap, D, 5)
    ccap = (evict_kept_count(cap, *rule) + 63) // 64 * 64
    for T in (0, 1, 100, 131, 132, 133, 140, 1000, 1151, cap):
        dk = torch.full((Hkv, ccap, D), float("nan"), device="cuda")
        dv = torch.full((Hkv, ccap // 32, D, 32), float("nan"), device="cuda")
        dl = torch.full((Hkv,), -1, dtype=torch.int32, device="cuda")
        src_len = torch.tensor([T, 12345], dtype=torch.int32, device="cuda")   # only entry 0 is read
        gather_evict(src_len, *rule, k, v, dk, dv, dl)
        torch.cuda.synchronize()
        _check(dk, dv, dl, k, v, tiny.kept_positions(T, *rule))


def test_gather_rows_with_a_list():
    import torch
    from lossless_speculative_decoding_vc_amd.tiny_loop import _setup_lib
    from lossless_speculative_decoding_vc_amd import _check as ok
    L = _setup_lib()
    Hkv, cap, D, ccap = 2, 700, 128, 320
    k, v = _caches(Hkv, cap, D, 6)
    kept = np.sort(np.random.default_rng(7).choice(cap, 301, replace=False)).astype(np.int32)
    idx = torch.from_numpy(kept).cuda()
    dk = torch.zeros((Hkv, ccap, D), device="cuda")
    dv = torch.zeros((Hkv, ccap // 32, D, 32), device="cuda")
    dl = torch.zeros(Hkv, dtype=torch.int32, device="cuda")
    ok(L.vc_gather_rows(Hkv, D, len(kept), idx.data_ptr(), k.data_ptr(), v.data_ptr(), cap, dk.data_ptr(),
                        dv.data_ptr(), ccap, dl.data_ptr(), None))
    torch.cuda.synchronize()
    _check(dk, dv, dl, k, v, kept)
