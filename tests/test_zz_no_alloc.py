"""vc_draft_attn_noalloc, the draft entry point for callers that cannot
allocate: its split partials live in the library's static per-GPU array.
Through the C ABI it must give exactly the bits vc_draft_attn gives with a
caller-provided workspace (same kernels, same split plan), on two calls in a
row, the second smaller than the first (the array keeps the first call's
partials, which the second must not read), and refuse a call whose split
scratch exceeds the array before enqueueing anything."""
import ctypes

import numpy as np
import pytest

import synthetic as S

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, cap, tcap, seed, packed=False):
    import torch
    dev = "cuda"
    D = 128
    q = S.torch_normal((B, Hq, D), seed, dev, torch.bfloat16, 2.0)
    if packed:
        k = S.torch_randint((B, Hkv, cap // 32, 5120), 0, 256, seed + 1, dev, torch.int32).to(torch.uint8)
        g = torch.Generator(device=dev)
        g.manual_seed(seed + 2)
        for j in range(2):   # K and V scale/zero pieces: scales in [0.3, 0.5), zeros -7.5 scale
            sc = (torch.rand((B, Hkv, cap // 32, 128), generator=g, device=dev) * 0.2 + 0.3).half()
            k[..., 4096 + 512 * j:4352 + 512 * j] = sc.view(torch.uint8)
            k[..., 4352 + 512 * j:4608 + 512 * j] = (sc.float() * -7.5).half().view(torch.uint8)
        v, deg = None, None
    else:
        k = S.torch_normal((B, Hkv, cap, D), seed + 1, dev, torch.bfloat16)
        v = S.torch_normal((B, Hkv, cap // 32, D, 32), seed + 2, dev, torch.bfloat16)
        deg = S.torch_randint((B, 1, cap), 1, 5, seed + 3, dev, torch.int32).float()
    ml = S.torch_randint((B, Hkv), cap // 2, cap + 1, seed + 4, dev, torch.int32)
    tk = S.torch_normal((B, Hkv, tcap, D), seed + 5, dev, torch.bfloat16)
    tv = S.torch_normal((B, Hkv, D, tcap), seed + 6, dev, torch.bfloat16)
    tl = S.torch_randint((B,), 0, tcap + 1, seed + 7, dev, torch.int32)
    return dict(q=q, k=k, v=v, main_len=ml, degree=deg, tail_k=tk, tail_v=tv, tail_len=tl)


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_equals_workspace_entry_point_twice(packed):
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    fmt = vc.VC_KV_INT4_PACKED if packed else vc.VC_KV_DENSE
    # the first call splits a batch-4 slice set 8 ways; the second is smaller (batch 2, 3 splits)
    for B, Hq, Hkv, cap, tcap, splits, seed in ((4, 32, 8, 4096, 40, 8, 11), (2, 8, 2, 1024, 24, 3, 12)):
        x = _inputs(B, Hq, Hkv, cap, tcap, seed, packed)
        assert vc.draft_workspace_size(B=B, Hq=Hq, Hkv=Hkv, D=128, dtype=0, fmt=fmt, scale=0.088,
                                       num_splits=splits, cap=cap, tcap=tcap) > 0
        ref_out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
        ref_lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        vc.draft_attn(x["q"], x["k"], x["v"], x["main_len"], degree=x["degree"], tail_k=x["tail_k"],
                      tail_v=x["tail_v"], tail_len=x["tail_len"], out=ref_out, out_lse=ref_lse, num_splits=splits,
                      fmt=fmt)
        vc.draft_attn_noalloc(x["q"], x["k"], x["v"], x["main_len"], degree=x["degree"], tail_k=x["tail_k"],
                              tail_v=x["tail_v"], tail_len=x["tail_len"], out=out, out_lse=lse, num_splits=splits,
                              fmt=fmt)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), (B, splits)
        assert torch.equal(lse, ref_lse), (B, splits)


def test_noalloc_refuses_more_than_its_array():
    import lossless_speculative_decoding_vc_amd as vc
    L = vc.lib()
    cap = L.vc_draft_noalloc_max_scratch()
    assert cap == 16 << 20
    fake = 1 << 20   # aligned, never dereferenced: the size check comes first
    a = vc.DraftArgs()
    a.B, a.Hq, a.Hkv, a.D, a.dtype, a.fmt, a.scale, a.cap, a.num_splits = 64, 64, 8, 128, 0, 0, 0.088, 65536, 64
    a.q, a.out, a.main_len, a.k, a.v = fake, fake, fake, fake, fake
    assert L.vc_draft_workspace_size(ctypes.byref(a)) > cap
    assert L.vc_draft_attn_noalloc(ctypes.byref(a), None) == vc.VC_EINVAL
    assert b"static array" in L.vc_last_error()
