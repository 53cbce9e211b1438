"""CPU checks of the binding's argument validation: the C ABI receives raw
device pointers, so every tensor's shape and dtype is compared with the
layout written in include/vc.h before anything is enqueued.  Each mismatch
below must raise ValueError naming the tensor; a call whose shapes are all
right gets as far as the device check (these tensors live on the CPU)."""
import pytest
import torch

import lossless_speculative_decoding_vc_amd as vc

B, Hq, Hkv, D, CAP, TCAP = 2, 8, 2, 128, 128, 32
bf, f32, i32, u8, i16 = torch.bfloat16, torch.float32, torch.int32, torch.uint8, torch.int16


def e(*shape, dtype=bf):
    return torch.empty(shape, dtype=dtype)


def draft_kw(**over):
    kw = dict(q=e(B, Hq, D), k=e(B, Hkv, CAP, D), v=e(B, Hkv, CAP // 32, D, 32), main_len=e(B, Hkv, dtype=i32),
              degree=e(B, 1, CAP, dtype=f32), tail_k=e(B, Hkv, TCAP, D), tail_v=e(B, Hkv, D, TCAP),
              tail_len=e(B, dtype=i32), out=e(B, Hq, D), out_lse=e(B, Hq, dtype=f32))
    kw.update(over)
    return kw


def run_draft(kw):
    kw = dict(kw)
    q, k, v, ml = kw.pop("q"), kw.pop("k"), kw.pop("v"), kw.pop("main_len")
    return vc.draft_attn(q, k, v, ml, **kw)


def test_draft_correct_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        run_draft(draft_kw())


@pytest.mark.parametrize("name,bad,msg", [
    ("q", e(B, Hq, D, 1), "q must be"),
    ("q", e(B, Hq, D, dtype=torch.float16), "q must be"),
    ("k", e(B, Hkv, CAP, 64), "k must be"),
    ("k", e(B, Hkv, CAP, D, dtype=f32), "k must be"),
    ("k", e(B + 1, Hkv, CAP, D), "k must start"),
    ("k", e(B, 3, CAP, D), "multiple of the KV heads"),
    ("v", e(B, Hkv, D, CAP), "v must be"),
    ("v", e(B, Hkv, CAP // 32 - 1, D, 32), "v must be"),
    ("main_len", e(B, dtype=i32), "main_len must be"),
    ("main_len", e(B, Hkv, dtype=torch.int64), "main_len must be"),
    ("degree", e(B, Hkv + 1, CAP, dtype=f32), "degree must be"),
    ("degree", e(B, 1, CAP - 64, dtype=f32), "degree must be"),
    ("degree", e(B, 1, CAP, dtype=bf), "degree must be"),
    ("tail_k", e(B, Hkv, TCAP, D // 2), "tail_k must be"),
    ("tail_v", e(B, Hkv, TCAP, D), "tail_v must be"),
    ("tail_v", None, "go together"),
    ("tail_len", e(B, 1, dtype=i32), "tail_len must be"),
    ("out", e(B, Hq, D, dtype=f32), "out must be"),
    ("out", e(B, Hq - 1, D), "out must be"),
    ("out_lse", e(B, Hq), "out_lse must be"),
])
def test_draft_rejects_mismatch(name, bad, msg):
    with pytest.raises(ValueError, match=msg):
        run_draft(draft_kw(**{name: bad}))


def test_draft_int4_layouts():
    i4 = dict(k=e(B, Hkv, CAP, D // 2, dtype=u8), v=e(B, Hkv, CAP // 32, D, 16, dtype=u8),
              k_scale=e(B, Hkv, CAP // 32, D, dtype=i16), k_zero=e(B, Hkv, CAP // 32, D, dtype=torch.float16),
              v_scale=e(B, Hkv, CAP // 32, D // 32, 32, dtype=i16), v_zero=e(B, Hkv, CAP // 32, D // 32, 32, dtype=i16),
              fmt=vc.VC_KV_INT4)
    with pytest.raises(ValueError, match="GPU tensor"):
        run_draft(draft_kw(**i4))
    for name, bad in (("k", e(B, Hkv, CAP, D, dtype=u8)), ("v", e(B, Hkv, CAP // 32, D, 32, dtype=u8)),
                      ("k_scale", e(B, Hkv, CAP // 32, D, dtype=f32)), ("v_zero", e(B, Hkv, CAP // 32, D, dtype=i16)),
                      ("k_zero", None)):
        with pytest.raises(ValueError, match=name):
            run_draft(draft_kw(**dict(i4, **{name: bad})))
    packed = dict(k=e(B, Hkv, CAP // 32, vc.INT4_PACKED_BLOCK, dtype=u8), v=None, fmt=vc.VC_KV_INT4_PACKED)
    with pytest.raises(ValueError, match="GPU tensor"):
        run_draft(draft_kw(**packed))
    with pytest.raises(ValueError, match="k must be"):
        run_draft(draft_kw(**dict(packed, k=e(B, Hkv, CAP // 32, 4096, dtype=u8))))
    with pytest.raises(ValueError, match="k alone"):
        run_draft(draft_kw(**dict(packed, v=e(B, Hkv, CAP // 32, D, 16, dtype=u8))))
    with pytest.raises(ValueError, match="int4 cache only"):
        run_draft(draft_kw(k_scale=e(B, Hkv, CAP // 32, D, dtype=i16)))


M, CCAP = 9, 256


def verify_kw(**over):
    kw = dict(q=e(B, M, Hq, D), ctx_k=e(B, Hkv, CCAP, D), ctx_v=e(B, Hkv, D, CCAP), ctx_len=e(B, dtype=i32),
              blk_k=e(B, Hkv, M, D), blk_v=e(B, Hkv, D, M), out=e(B, M, Hq, D), out_lse=e(B, M, Hq, dtype=f32))
    kw.update(over)
    return kw


def run_verify(kw):
    kw = dict(kw)
    args = [kw.pop(n) for n in ("q", "ctx_k", "ctx_v", "ctx_len", "blk_k", "blk_v")]
    return vc.verify_attn(*args, **kw)


def test_verify_correct_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        run_verify(verify_kw())


@pytest.mark.parametrize("name,bad,msg", [
    ("q", e(B, M, Hq), "q must be"),
    ("ctx_k", e(B, Hkv + 1, CCAP, D), "ctx_k must be"),
    ("ctx_k", e(B, Hkv, CCAP, D, dtype=f32), "ctx_k must be"),
    ("ctx_v", e(B, Hkv, CCAP, D), "ctx_v must be"),
    ("ctx_v", None, "go together"),
    ("ctx_len", e(B, 1, dtype=i32), "ctx_len must be"),
    ("blk_k", e(B, 3, M, D), "multiple of the KV heads"),
    ("blk_k", e(B, Hkv, M + 1, D), "blk_k must be"),
    ("blk_v", e(B, Hkv, M, D), "blk_v must be"),
    ("out", e(B, M, Hq, D, dtype=f32), "out must be"),
    ("out_lse", e(B, M, Hq + 1, dtype=f32), "out_lse must be"),
])
def test_verify_rejects_mismatch(name, bad, msg):
    with pytest.raises(ValueError, match=msg):
        run_verify(verify_kw(**{name: bad}))


def commit_kw(**over):
    kw = dict(blk_k=e(B, Hkv, M, D), blk_v=e(B, Hkv, D, M), n_out=e(B, dtype=i32), dst_k=e(B, Hkv, CCAP, D),
              dst_v=e(B, Hkv, D, CCAP), length=e(B, Hkv, dtype=i32), degree=e(B, Hkv, CCAP, dtype=f32))
    kw.update(over)
    return kw


def test_commit_rows_checks():
    with pytest.raises(ValueError, match="GPU tensor"):
        vc.commit_rows(**commit_kw())
    with pytest.raises(ValueError, match="GPU tensor"):
        vc.commit_rows(**commit_kw(dst_v=e(B, Hkv, CCAP // 32, D, 32)), v_blocked=True)
    for name, bad, extra in (("dst_v", e(B, Hkv, CCAP // 32, D, 32), {}),
                             ("dst_v", e(B, Hkv, D, CCAP), {"v_blocked": True}),
                             ("blk_v", e(B, Hkv, M, D), {}),
                             ("dst_k", e(B, Hkv, CCAP, D, dtype=f32), {}),
                             ("n_out", e(B, 1, dtype=i32), {}),
                             ("length", e(B, dtype=i32), {}),
                             ("degree", e(B, Hkv, CCAP + 32, dtype=f32), {})):
        with pytest.raises(ValueError, match=name):
            vc.commit_rows(**commit_kw(**{name: bad}), **extra)
