"""GPU parity of vc_compact_kv (eviction compaction into the drafter's main
segment) against the oracle: bit-exact rows, zero rows for indices outside
the source, untouched rows past n_kept, lengths; and draft attention over the
compacted cache against the oracle's attention over the full cache with the
evicted tokens masked."""
import numpy as np
import pytest

import synthetic as S
from oracle import attention as A
from oracle.compress import compact_kv

from .helpers import TOL, assert_close, bf16_dev_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _run(dtype, D, B=2, Hkv=3, src_cap=300, cap=128, n_kept=(100, 37), seed=7):
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    rng = np.random.default_rng(seed)
    kf = S.normal_f32((B, Hkv, src_cap, D), seed, S.TID["k"])
    vf = S.normal_f32((B, Hkv, src_cap, D), seed, S.TID["v"])
    stride = 120
    idx = np.full((B, stride), -7, np.int32)
    for b, n in enumerate(n_kept):
        idx[b, :n] = np.sort(rng.choice(src_cap, n, replace=False))
    idx[1, 5] = src_cap + 3          # outside the source: a zero row
    if dtype == "bf16":
        kb, vb = S.f32_to_bf16_bits(kf), S.f32_to_bf16_bits(vf)
        sk, sv = to_dev_bf16(kb), to_dev_bf16(np.ascontiguousarray(np.swapaxes(vb, -1, -2)))
        tdt = torch.bfloat16
    else:
        kb, vb = kf, vf
        sk, sv = to_dev(kf), to_dev(np.ascontiguousarray(np.swapaxes(vf, -1, -2)))
        tdt = torch.float32
    dk = torch.full((B, Hkv, cap, D), 3.0, dtype=tdt, device="cuda")
    dv = torch.full((B, Hkv, cap // 32, D, 32), 3.0, dtype=tdt, device="cuda")
    dl = torch.full((B, Hkv), -1, dtype=torch.int32, device="cuda")
    vc.compact_kv(sk, sv, to_dev(idx), to_dev(np.asarray(n_kept, np.int32)), dk, dv, dst_len=dl)
    torch.cuda.synchronize()
    view = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) if dtype == "bf16" else \
        (lambda t: t.cpu().numpy())
    gk, gv = view(dk), view(dv)
    # unblock V: [cap/32][D][32] -> [cap][D]
    gv_t = gv.transpose(0, 1, 2, 4, 3).reshape(B, Hkv, cap, D)
    fill = view(torch.full((1,), 3.0, dtype=tdt))[0]
    for b, n in enumerate(n_kept):
        ref_k, ref_v = compact_kv(kb[b], vb[b], idx[b, :n])
        np.testing.assert_array_equal(gk[b, :, :n], ref_k)
        np.testing.assert_array_equal(gv_t[b, :, :n], ref_v)
        assert np.all(gk[b, :, n:] == fill) and np.all(gv_t[b, :, n:] == fill)
    assert dl.cpu().numpy().tolist() == [[n] * Hkv for n in n_kept]
    return dk, dv, kb, vb, idx


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
def test_compact_bit_exact(dtype, D):
    _run(dtype, D)


def test_draft_over_compacted_cache_is_masked_full_attention():
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hq, Hkv, D, n_kept = 2, 12, 3, 128, (100, 37)
    dk, dv, kb, vb, idx = _run("bf16", D, n_kept=n_kept, seed=9)
    qb = S.f32_to_bf16_bits(S.normal_f32((B, Hq, D), 9, S.TID["q"], std=3.0, slice_dims=1))
    ml = np.array([[n] * Hkv for n in n_kept], np.int32)
    out = vc.draft_attn(to_dev_bf16(qb), dk, dv, to_dev(ml))
    torch.cuda.synchronize()
    from oracle.formats import bf16_to_f64
    q, k, v = bf16_to_f64(qb), bf16_to_f64(kb), bf16_to_f64(vb)
    ref = np.empty((B, Hq, D))
    G = Hq // Hkv
    for b, n in enumerate(n_kept):
        keep = idx[b, :n]
        ok = keep < k.shape[2]
        mask = np.full(k.shape[2], -np.inf)
        mask[keep[ok]] = 0.0
        for h in range(Hq):
            kk, vv = k[b, h // G], v[b, h // G]
            extra_k = np.zeros((int((~ok).sum()), D))   # an out-of-range index compacts to a zero row
            o, _ = A.attend(q[b, h], np.concatenate([kk, extra_k]), np.concatenate([vv, extra_k]), D ** -0.5,
                            bias=np.concatenate([mask, np.zeros(len(extra_k))]))
            ref[b, h] = o
    assert_close(bf16_dev_to_f64(out), ref, TOL["bf16"], "draft over compacted cache")


def test_full_size_sampled_slices_bit_exact():
    # The launch configuration of the 128K cohort's compaction: 16 requests x
    # 8 KV heads, a 131072-token full cache, 32768 kept tokens per request (a
    # sorted random subset, as the bench times it).  Three sampled slices are
    # compared with the oracle bit for bit.
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hkv, D, n, kept = 16, 8, 128, 131072, 32768
    dev = "cuda"
    K = S.torch_normal((B, Hkv, n, D), 81, dev, torch.bfloat16, 1.0)
    Vt = S.torch_normal((B, Hkv, D, n), 82, dev, torch.bfloat16, 1.0)
    rng = np.random.default_rng(83)
    idx = np.stack([np.sort(rng.choice(n, kept, replace=False)) for _ in range(B)]).astype(np.int32)
    dk = torch.empty((B, Hkv, kept, D), dtype=torch.bfloat16, device=dev)
    dv = torch.empty((B, Hkv, kept // 32, D, 32), dtype=torch.bfloat16, device=dev)
    dl = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    vc.compact_kv(K, Vt, to_dev(idx), to_dev(np.full(B, kept, np.int32)), dk, dv, dst_len=dl)
    torch.cuda.synchronize()
    assert np.all(dl.cpu().numpy() == kept)
    host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    for b, h in [(0, 0), (9, 4), (15, 7)]:
        ref_k, ref_v = compact_kv(host(K[b, h]), host(Vt[b, h].t()), idx[b])
        np.testing.assert_array_equal(host(dk[b, h]), ref_k)
        np.testing.assert_array_equal(host(dv[b, h]).transpose(0, 2, 1).reshape(kept, D), ref_v)
