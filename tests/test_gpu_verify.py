"""GPU parity of vc_verify_attn against the oracle: block rows causal among
themselves, full context visible, ragged context lengths, head groupings,
forced split counts, causal prefill (empty context), bf16 and fp32."""
import numpy as np
import pytest

import synthetic as S
from oracle import attention as A
from oracle.formats import bf16_to_f64

from .helpers import TOL, assert_close, bf16_dev_to_f64, rel_l2, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(B, M, Hq, Hkv, D, ccap, dtype, seed, qstd):
    arrs = {
        "q": (S.normal_f32((B, M, Hq, D), seed, S.TID["q"], std=qstd, slice_dims=1), False),
        "ctx_k": (S.normal_f32((B, Hkv, ccap, D), seed, S.TID["k"]), False),
        "ctx_v": (S.normal_f32((B, Hkv, ccap, D), seed, S.TID["v"]), True),
        "blk_k": (S.normal_f32((B, Hkv, M, D), seed, S.TID["blk_k"]), False),
        "blk_v": (S.normal_f32((B, Hkv, M, D), seed, S.TID["blk_v"]), True),
    }
    dev, ref = {}, {}
    for name, (arr, chan_major) in arrs.items():
        if dtype == "bf16":
            bits = S.f32_to_bf16_bits(arr)
            ref[name] = bf16_to_f64(bits)
            dev[name] = to_dev_bf16(np.ascontiguousarray(np.swapaxes(bits, -1, -2) if chan_major else bits))
        else:
            ref[name] = arr.astype(np.float64)
            dev[name] = to_dev(np.ascontiguousarray(np.swapaxes(arr, -1, -2) if chan_major else arr))
    return dev, ref


def _check(B, M, Hq, Hkv, D, ccap, ctx_len, dtype="bf16", seed=0, splits=0, qstd=1.0, rows=None):
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    dev, ref = _inputs(B, M, Hq, Hkv, D, ccap, dtype, seed, qstd)
    cl = np.asarray(ctx_len, np.int32)
    lse = torch.empty((B, M, Hq), dtype=torch.float32, device="cuda")
    out = vc.verify_attn(dev["q"], dev["ctx_k"], dev["ctx_v"], to_dev(cl), dev["blk_k"], dev["blk_v"],
                         out_lse=lse, num_splits=splits)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out) if dtype == "bf16" else out.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = A.verify_attn(ref["q"], ref["ctx_k"], ref["ctx_v"], cl, ref["blk_k"], ref["blk_v"],
                                   rows=rows)
    if rows is not None:
        sel = tuple(np.array(rows).T)
        got, o_ref = got[sel], o_ref[sel]
        lse_got, lse_ref = lse.cpu().numpy()[sel], lse_ref[sel]
    else:
        lse_got = lse.cpu().numpy()
    assert_close(got, o_ref, TOL[dtype], "out")
    assert_close(lse_got, lse_ref, TOL[dtype] * 0.1, "lse")
    return got, o_ref


@pytest.mark.parametrize("M", [1, 9, 32, 33, 41])
@pytest.mark.parametrize("G", [2, 4, 5, 8])
def test_blocks_and_groupings(M, G):
    Hkv = 2
    _check(2, M, G * Hkv, Hkv, 128, 1280, [1100, 1234], seed=M * 100 + G, qstd=2.0)


@pytest.mark.parametrize("splits", [1, 2, 5, 16])
def test_forced_splits_peaked(splits):
    got, ref = _check(2, 33, 10, 2, 128, 2048, [2048, 1537], seed=5, splits=splits, qstd=4.0)
    assert rel_l2(got, ref) <= 2e-2 and np.abs(ref).mean() > 0.05


def test_head_dim_64_and_many_rows():
    # R = M*G = 400 packed rows -> several row tiles
    _check(1, 50, 16, 2, 64, 640, [600], seed=9, qstd=2.0)


def test_causal_prefill_empty_context():
    _check(2, 100, 8, 2, 128, 0, [0, 0], seed=11, qstd=2.0)


def test_short_context_and_zero_for_one_request():
    _check(2, 9, 4, 2, 128, 64, [3, 0], seed=12)


@pytest.mark.parametrize("G", [2, 5])
def test_fp32_mode(G):
    _check(1, 9, 2 * G, 2, 64, 1152, [1087], dtype="fp32", seed=13, qstd=3.0)


def test_fp32_prefill():
    _check(1, 130, 4, 2, 64, 0, [0], dtype="fp32", seed=14)


def test_sixteen_query_heads_per_kv_head():
    # G = 16 (the largest grouping): 33 block rows -> 528 packed rows, three row groups
    _check(1, 33, 32, 2, 128, 1280, [1201], seed=15, qstd=2.0)
    # 12 rows -> 192 packed rows, one row group of 48 rows per SIMD (token split)
    _check(2, 12, 16, 1, 128, 640, [640, 77], seed=16, qstd=2.0)


@pytest.mark.parametrize("M,G,splits", [(33, 5, 0), (20, 5, 3), (40, 4, 1)])
def test_token_split_head_dim_64(M, G, splits):
    # 165, 100 and 160 packed rows at head_dim 64: the token-split kernel with three and two column tiles
    _check(2, M, G * 2, 2, 64, 1280, [1280, 700], seed=19 + M, splits=splits, qstd=2.0)


def test_token_split_prefill_and_short_contexts():
    # 160 packed rows with no context (every tile holds block keys), then contexts shorter than one tile
    _check(1, 40, 8, 2, 128, 0, [0], seed=23, qstd=2.0)
    _check(2, 33, 10, 2, 128, 64, [50, 0], seed=24, qstd=2.0)


def test_token_split_one_tile_per_split():
    # 11 tiles over 11 splits: every split holds a single tile (one full tile or the block's tail)
    got, ref = _check(2, 33, 10, 2, 128, 640, [640, 576], seed=25, splits=11, qstd=3.0)
    assert rel_l2(got, ref) <= 2e-2


def test_prefill_of_1024_rows():
    # the largest block: a 1024-token causal prefill, then 1024 rows after a short context
    _check(1, 1024, 4, 2, 128, 0, [0], seed=17, qstd=2.0)
    _check(1, 1024, 2, 1, 64, 192, [130], seed=18, qstd=2.0)


@pytest.mark.parametrize("M,G", [(20, 5), (33, 5), (45, 5)])
def test_capacity_beyond_32bit_offsets(M, G):
    # A capacity of 2^23 tokens puts the V channel rows of one head 16 MiB
    # apart, 2 GiB in all: beyond the 32-bit offsets of the ping-pong kernel,
    # so the four-wave kernel serves every row count here (R = 100, 165 and
    # 225: 32- and 48-row waves, one and two row groups).  Only the first
    # 3000 context tokens are valid, so the oracle reads a small cache.
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hkv, D, cl, small, big = 1, 1, 128, 3000, 3008, 1 << 23
    Hq = G * Hkv
    dev, ref = _inputs(B, M, Hq, Hkv, D, small, "bf16", 40 + M, 2.0)
    ck = torch.zeros((B, Hkv, big, D), dtype=torch.bfloat16, device="cuda")
    cv = torch.zeros((B, Hkv, D, big), dtype=torch.bfloat16, device="cuda")
    ck[:, :, :small] = dev["ctx_k"]
    cv[..., :small] = dev["ctx_v"]
    cl_arr = np.array([cl], np.int32)
    lse = torch.empty((B, M, Hq), dtype=torch.float32, device="cuda")
    out = vc.verify_attn(dev["q"], ck, cv, to_dev(cl_arr), dev["blk_k"], dev["blk_v"], out_lse=lse)
    torch.cuda.synchronize()
    del ck, cv
    o_ref, lse_ref = A.verify_attn(ref["q"], ref["ctx_k"], ref["ctx_v"], cl_arr, ref["blk_k"], ref["blk_v"])
    assert_close(bf16_dev_to_f64(out), o_ref, TOL["bf16"], "out")
    assert_close(lse.cpu().numpy(), lse_ref, TOL["bf16"] * 0.1, "lse")
