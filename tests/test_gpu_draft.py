"""GPU parity of vc_draft_attn against the oracle (bf16 2e-2, fp32 1e-4),
over head groupings, ragged lengths, merge degrees, the draft tail, forced
split counts and the degenerate cases (empty main segment, tail only)."""
import numpy as np
import pytest

import synthetic as S
from oracle import attention as A
from oracle.formats import bf16_to_f64

from .helpers import TOL, assert_close, bf16_dev_to_f64, blocked32, rel_l2, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, D, cap, main_len, tcap, tail_len, dtype, deg_mode, seed, qstd=1.0):
    """Seeded inputs in both layouts: oracle side float64 [.., tokens, D]."""
    qf = S.normal_f32((B, Hq, D), seed, S.TID["q"], std=qstd, slice_dims=1)
    kf = S.normal_f32((B, Hkv, cap, D), seed, S.TID["k"])
    vf = S.normal_f32((B, Hkv, cap, D), seed, S.TID["v"])
    tkf = S.normal_f32((B, Hkv, tcap, D), seed, S.TID["tail_k"]) if tcap else None
    tvf = S.normal_f32((B, Hkv, tcap, D), seed, S.TID["tail_v"]) if tcap else None
    deg = None
    if deg_mode == "shared":
        deg = S.degrees((B, 1, cap), seed)
    elif deg_mode == "per_head":
        deg = S.degrees((B, Hkv, cap), seed)
    dev, ref = {}, {}
    # main V in 32-token blocks, tail V channel-major
    for name, arr, lay in (("q", qf, None), ("k", kf, None), ("v", vf, "blocked"),
                           ("tail_k", tkf, None), ("tail_v", tvf, "chan")):
        if arr is None:
            dev[name] = ref[name] = None
            continue
        if dtype == "bf16":
            bits = S.f32_to_bf16_bits(arr)
            ref[name] = bf16_to_f64(bits)
            dbits = blocked32(bits) if lay == "blocked" else (np.swapaxes(bits, -1, -2) if lay == "chan" else bits)
            dev[name] = to_dev_bf16(np.ascontiguousarray(dbits))
        else:
            ref[name] = arr.astype(np.float64)
            darr = blocked32(arr) if lay == "blocked" else (np.swapaxes(arr, -1, -2) if lay == "chan" else arr)
            dev[name] = to_dev(np.ascontiguousarray(darr))
    ml = np.asarray(main_len, np.int32).reshape(B, Hkv)
    tl = None if tcap == 0 else np.asarray(tail_len, np.int32).reshape(B)
    return dev, ref, ml, tl, deg


def _check(B, Hq, Hkv, D, cap, main_len, tcap=0, tail_len=None, dtype="bf16", deg_mode=None,
           seed=0, splits=0, qstd=1.0, min_rel_l2=None):
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    dev, ref, ml, tl, deg = _case(B, Hq, Hkv, D, cap, main_len, tcap, tail_len, dtype, deg_mode, seed, qstd)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out = vc.draft_attn(dev["q"], dev["k"], dev["v"], to_dev(ml),
                        degree=None if deg is None else to_dev(deg),
                        tail_k=dev["tail_k"], tail_v=dev["tail_v"],
                        tail_len=None if tl is None else to_dev(tl),
                        out_lse=lse, num_splits=splits)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out) if dtype == "bf16" else out.cpu().numpy().astype(np.float64)
    o_ref, lse_ref = A.draft_attn(ref["q"], ref["k"], ref["v"], ml, deg, ref["tail_k"], ref["tail_v"], tl)
    assert_close(got, o_ref, TOL[dtype], "out")
    assert_close(lse.cpu().numpy(), lse_ref, TOL[dtype] * 0.1, "lse")
    if min_rel_l2 is not None:
        assert rel_l2(got, o_ref) <= min_rel_l2
    return got, o_ref


@pytest.mark.parametrize("G", [1, 4, 5, 8, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_groupings_ragged(G, D):
    Hkv = 2
    _check(2, G * Hkv, Hkv, D, 1024, [[1000, 777], [1024, 65]], 16, [5, 0],
           deg_mode="shared", seed=G * 10 + D)


@pytest.mark.parametrize("deg_mode", [None, "shared", "per_head"])
@pytest.mark.parametrize("splits", [0, 1, 3, 7])
def test_degrees_and_splits_peaked(deg_mode, splits):
    # q std 4: scores spread widely, outputs O(0.1-1), so the tolerance bites
    got, ref = _check(3, 12, 3, 128, 2048, [[2048, 1999, 1500], [700, 64, 1], [0, 33, 2047]], 40,
                      [40, 7, 1], deg_mode=deg_mode, seed=7, splits=splits, qstd=4.0, min_rel_l2=2e-2)
    assert np.abs(ref).mean() > 0.05        # non-vacuous comparison


def test_tail_only_and_main_only():
    # main_len 0 everywhere for request 0: keys come from the tail alone
    _check(2, 8, 2, 128, 512, [[0, 0], [512, 100]], 24, [24, 0], deg_mode="shared", seed=3)


@pytest.mark.parametrize("G", [2, 4])
def test_fp32_mode(G):
    _check(2, 2 * G, 2, 64, 320, [[300, 257], [1, 320]], 9, [9, 3], dtype="fp32",
           deg_mode="shared", seed=21, qstd=3.0)


def test_fp32_no_tail_no_degree():
    _check(1, 4, 2, 64, 256, [[243, 200]], 0, None, dtype="fp32", seed=22)


# ---------------------------------------------------------------------------
# int4 main segment (the quantizing drafter): the oracle reconstructs
# x = c * s + z in fp64 and runs dense attention over the reconstruction.
def _int4_check(B, Hq, Hkv, cap, main_len, tcap, tail_len, deg_mode, seed, splits=0, qstd=1.0, packed=False):
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    from oracle import quant as Q
    from oracle.formats import f16_to_f64
    D = 128
    g = S.int4_grid(B, Hkv, cap, D, seed)
    qf = S.normal_f32((B, Hq, D), seed, S.TID["q"], std=qstd, slice_dims=1)
    qbits = S.f32_to_bf16_bits(qf)
    tkf = S.normal_f32((B, Hkv, tcap, D), seed, S.TID["tail_k"]) if tcap else None
    tvf = S.normal_f32((B, Hkv, tcap, D), seed, S.TID["tail_v"]) if tcap else None
    deg = None
    if deg_mode == "shared":
        deg = S.degrees((B, 1, cap), seed)
    k_ref = np.empty((B, Hkv, cap, D))
    v_ref = np.empty((B, Hkv, cap, D))
    for b in range(B):
        for h in range(Hkv):
            k_ref[b, h] = Q.dequantize_k(g["k_c"][b, h], f16_to_f64(g["k_scale"][b, h]), f16_to_f64(g["k_zero"][b, h]))
            v_ref[b, h] = Q.dequantize_v(g["v_c"][b, h], f16_to_f64(g["v_scale_td"][b, h]),
                                         f16_to_f64(g["v_zero_td"][b, h]))
    tk_ref = tv_ref = tk_dev = tv_dev = None
    if tcap:
        tkb, tvb = S.f32_to_bf16_bits(tkf), S.f32_to_bf16_bits(tvf)
        tk_ref, tv_ref = bf16_to_f64(tkb), bf16_to_f64(tvb)
        tk_dev = to_dev_bf16(tkb)
        tv_dev = to_dev_bf16(np.ascontiguousarray(np.swapaxes(tvb, -1, -2)))
    ml = np.asarray(main_len, np.int32).reshape(B, Hkv)
    tl = None if tcap == 0 else np.asarray(tail_len, np.int32)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    as_dev16 = lambda a: to_dev(np.ascontiguousarray(a).view(np.int16))
    common = dict(degree=None if deg is None else to_dev(deg), tail_k=tk_dev, tail_v=tv_dev,
                  tail_len=None if tl is None else to_dev(tl), out_lse=lse, num_splits=splits)
    if packed:   # the same cache, one interleaved 5120-byte block per 32 tokens
        blk = S.pack_int4_blocks(g["k_codes"], g["v_codes"], g["k_scale"], g["k_zero"], g["v_scale"], g["v_zero"])
        out = vc.draft_attn(to_dev_bf16(qbits), to_dev(blk), None, to_dev(ml), fmt=vc.VC_KV_INT4_PACKED, **common)
    else:
        out = vc.draft_attn(to_dev_bf16(qbits), to_dev(g["k_codes"]), to_dev(g["v_codes"]), to_dev(ml),
                            fmt=vc.VC_KV_INT4, k_scale=as_dev16(g["k_scale"]), k_zero=as_dev16(g["k_zero"]),
                            v_scale=as_dev16(g["v_scale"]), v_zero=as_dev16(g["v_zero"]), **common)
    torch.cuda.synchronize()
    got = bf16_dev_to_f64(out)
    o_ref, lse_ref = A.draft_attn(bf16_to_f64(qbits), k_ref, v_ref, ml, deg, tk_ref, tv_ref, tl)
    assert_close(got, o_ref, TOL["bf16"], "out")
    assert_close(lse.cpu().numpy(), lse_ref, TOL["bf16"] * 0.1, "lse")
    return got, o_ref


@pytest.mark.parametrize("splits", [0, 1, 5])
def test_int4_main_segment(splits):
    _int4_check(2, 8, 2, 1024, [[1024, 1000], [64, 333]], 12, [12, 3], "shared", seed=31, splits=splits)


def test_int4_peaked_no_tail():
    got, ref = _int4_check(2, 16, 4, 512, [[512, 480, 96, 1], [200, 511, 32, 256]], 0, None, None,
                           seed=32, qstd=1.0)
    assert rel_l2(got, ref) <= 2e-2


def test_int4_tail_only():
    _int4_check(1, 4, 1, 256, [[0]], 20, [20], "shared", seed=33)


@pytest.mark.parametrize("splits", [0, 3])
def test_int4_packed_main_segment(splits):
    # the packed layout: same codes and parameters, one contiguous block per 32 tokens
    _int4_check(2, 8, 2, 1024, [[1024, 1000], [64, 333]], 12, [12, 3], "shared", seed=31, splits=splits,
                packed=True)
    got, ref = _int4_check(2, 16, 4, 512, [[512, 480, 96, 1], [200, 511, 32, 256]], 0, None, None, seed=32,
                           packed=True)
    assert rel_l2(got, ref) <= 2e-2


@pytest.mark.parametrize("G", [1, 5, 8, 16])
@pytest.mark.parametrize("packed", [False, True])
def test_int4_head_groupings(G, packed):
    # 1 to 16 query heads per KV head fill 1 to 16 of the 16 MFMA columns (the rest is padding); degrees, a
    # partial last chunk, a tail and forced splits
    _int4_check(2, 2 * G, 2, 512, [[512, 300], [33, 480]], 8, [8, 5], "shared", seed=40 + G, splits=3,
                qstd=2.0, packed=packed)


def test_split_calls_share_one_workspace():
    # One workspace serves draft calls of different shapes and split counts
    # (2 .. 64 splits, 1 .. 16 query heads per KV head) back to back: every
    # call writes its partials before its merge reads them.
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    ws = vc.new_workspace(1 << 24, "cuda")
    cases = [(3, 12, 3, 2048, [[2048, 1999, 1500], [700, 64, 1], [0, 33, 2047]], 40, [40, 7, 1], 64),
             (2, 32, 2, 4096, [[4096, 4000], [37, 2500]], 0, None, 2),
             (1, 16, 1, 4096, [[4093]], 16, [16], 33),
             (2, 8, 8, 1024, [[1024] * 8, [1, 2, 3, 4, 5, 6, 7, 1000]], 0, None, 0)]
    for i, (B, Hq, Hkv, cap, ml, tcap, tl, splits) in enumerate(cases):
        dev, ref, mlen, tlen, deg = _case(B, Hq, Hkv, 128, cap, ml, tcap, tl, "bf16", "shared", 90 + i, 3.0)
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        out = vc.draft_attn(dev["q"], dev["k"], dev["v"], to_dev(mlen), degree=to_dev(deg),
                            tail_k=dev["tail_k"], tail_v=dev["tail_v"],
                            tail_len=None if tlen is None else to_dev(tlen), out_lse=lse, num_splits=splits,
                            workspace=ws)
        torch.cuda.synchronize()
        o_ref, lse_ref = A.draft_attn(ref["q"], ref["k"], ref["v"], mlen, deg, ref["tail_k"], ref["tail_v"], tlen)
        assert_close(bf16_dev_to_f64(out), o_ref, TOL["bf16"], f"out, case {i}")
        assert_close(lse.cpu().numpy(), lse_ref, TOL["bf16"] * 0.1, f"lse, case {i}")
