"""GPU parity of vc_quantize_int4 against the oracle quantizer: codes, binary16
scales and zeros bit-exact, groups outside the call untouched, rounding ties
and constant groups decided as the exact evaluation decides, and the cache it
writes read back by vc_draft_attn (attention over the oracle's reconstruction,
bf16 tolerance)."""
import numpy as np
import pytest

import synthetic as S
from oracle import attention as A
from oracle import quant as Q
from oracle.formats import bf16_to_f64, f16_to_f64, unpack_int4

from .helpers import TOL, assert_close, bf16_dev_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu

D = 128
SENT8, SENT16 = 0xA5, 0x7BCD   # fill of the destination before the call


def _alloc(B, Hkv, cap):
    import torch
    dev = "cuda"
    u8 = lambda *s: torch.full(s, SENT8, dtype=torch.uint8, device=dev)
    i16 = lambda *s: torch.full(s, SENT16, dtype=torch.int16, device=dev)
    return dict(k_codes=u8(B, Hkv, cap, D // 2), k_scale=i16(B, Hkv, cap // 32, D), k_zero=i16(B, Hkv, cap // 32, D),
                v_codes=u8(B, Hkv, cap // 32, D, 16), v_scale=i16(B, Hkv, cap // 32, D // 32, 32),
                v_zero=i16(B, Hkv, cap // 32, D // 32, 32))


def _run(kbits, vbits, src_start, dst_start, n_groups, cap):
    """kbits/vbits: bf16 bits [B][Hkv][src_cap][D] (token-major both); returns host copies of the cache."""
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hkv = kbits.shape[:2]
    out = _alloc(B, Hkv, cap)
    vc.quantize_int4(to_dev_bf16(kbits), to_dev_bf16(np.ascontiguousarray(np.swapaxes(vbits, -1, -2))),
                     to_dev(np.asarray(src_start, np.int32).reshape(B, Hkv)), n_groups,
                     to_dev(np.asarray(dst_start, np.int32).reshape(B, Hkv)), **out)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}, out


def _check(kbits, vbits, src_start, dst_start, n_groups, cap, valid):
    got, _ = _run(kbits, vbits, src_start, dst_start, n_groups, cap)
    B, Hkv = kbits.shape[:2]
    ss = np.asarray(src_start).reshape(B, Hkv)
    ds = np.asarray(dst_start).reshape(B, Hkv)
    for b in range(B):
        for h in range(Hkv):
            written = np.zeros(cap // 32, bool)
            if valid[b][h]:
                s0, d0 = int(ss[b, h]), int(ds[b, h])
                x_k = bf16_to_f64(kbits[b, h, s0:s0 + 32 * n_groups])
                x_v = bf16_to_f64(vbits[b, h, s0:s0 + 32 * n_groups])
                kc, ks, kz = Q.quantize_k(x_k)
                vc_, vs, vz = Q.quantize_v(x_v)
                blk = slice(d0 // 32, d0 // 32 + n_groups)
                written[blk] = True
                # K: codes [tokens][D], scales [groups][D]
                got_kc = unpack_int4(got["k_codes"][b, h, d0:d0 + 32 * n_groups])
                np.testing.assert_array_equal(got_kc, kc)
                np.testing.assert_array_equal(got["k_scale"][b, h, blk].view(np.uint16), ks.view(np.uint16))
                np.testing.assert_array_equal(got["k_zero"][b, h, blk].view(np.uint16), kz.view(np.uint16))
                # V: codes [blk][D][32 tokens] -> [tokens][D]; scales [blk][D/32][32] -> [tokens][D/32]
                got_vc = unpack_int4(got["v_codes"][b, h, blk]).transpose(0, 2, 1).reshape(-1, D)
                np.testing.assert_array_equal(got_vc, vc_)
                gvs = got["v_scale"][b, h, blk].view(np.uint16).transpose(0, 2, 1).reshape(-1, D // 32)
                gvz = got["v_zero"][b, h, blk].view(np.uint16).transpose(0, 2, 1).reshape(-1, D // 32)
                np.testing.assert_array_equal(gvs, vs.view(np.uint16))
                np.testing.assert_array_equal(gvz, vz.view(np.uint16))
            # everything outside the written groups keeps the fill
            rows = np.repeat(~written, 32)
            assert np.all(got["k_codes"][b, h, rows] == SENT8)
            assert np.all(got["v_codes"][b, h, ~written] == SENT8)
            for key in ("k_scale", "k_zero", "v_scale", "v_zero"):
                assert np.all(got[key][b, h, ~written].view(np.uint16) == SENT16), key


def test_quantize_matches_oracle_bit_exact():
    B, Hkv, src_cap, cap, n = 2, 3, 160, 256, 3
    kf = S.normal_f32((B, Hkv, src_cap, D), 41, S.TID["k"], std=1.5)
    vf = S.normal_f32((B, Hkv, src_cap, D), 41, S.TID["v"], std=0.7)
    kbits, vbits = S.f32_to_bf16_bits(kf), S.f32_to_bf16_bits(vf)
    src = [[0, 7, 64], [31, 0, 64]]
    dst = [[0, 96, 160], [64, 160, 32]]
    _check(kbits, vbits, src, dst, n, cap, [[True] * 3] * 2)


def test_quantize_skips_invalid_slices():
    B, Hkv, src_cap, cap, n = 1, 4, 96, 128, 2
    kbits = S.f32_to_bf16_bits(S.normal_f32((B, Hkv, src_cap, D), 42, S.TID["k"]))
    vbits = S.f32_to_bf16_bits(S.normal_f32((B, Hkv, src_cap, D), 42, S.TID["v"]))
    # slice 1: dst not a multiple of 32; slice 2: source runs past src_cap; slice 3: dst runs past cap
    src = [[0, 0, 40, 0]]
    dst = [[32, 16, 0, 96]]
    _check(kbits, vbits, src, dst, n, cap, [[True, False, False, False]])


def test_quantize_ties_and_constant_groups():
    # group built so that (x - z) / s hits exact half-integers: min 0, max 15 -> s = 1, z = 0
    B, Hkv, cap = 1, 1, 64
    k = np.zeros((B, Hkv, 64, D), np.float32)
    v = np.zeros((B, Hkv, 64, D), np.float32)
    ramp = np.array([0.0, 15.0, 2.5, 3.5, 0.5, 1.5, 14.5, 7.5] + [4.25] * 24, np.float32)
    k[0, 0, :32, 0] = ramp                 # K channel 0 of group 0
    k[0, 0, :32, 1] = 2.0                  # constant channel: s = 0 -> codes 0, z = 2
    k[0, 0, 32:, :] = np.linspace(-3, 3, 32 * D, dtype=np.float32).reshape(32, D)
    v[0, 0, 0, :32] = ramp                 # V token 0, channel group 0
    v[0, 0, 1, :] = -1.25                  # constant token
    v[0, 0, 32:, :] = np.linspace(5, -5, 32 * D, dtype=np.float32).reshape(32, D)
    kbits, vbits = S.f32_to_bf16_bits(k), S.f32_to_bf16_bits(v)
    _check(kbits, vbits, [[0]], [[0]], 2, cap, [[True]])
    got, _ = _run(kbits, vbits, [[0]], [[0]], 2, cap)
    codes = unpack_int4(got["k_codes"][0, 0, :32])[:, 0]
    assert codes[:8].tolist() == [0, 15, 2, 4, 0, 2, 14, 8]   # ties to even
    assert np.all(unpack_int4(got["k_codes"][0, 0, :32])[:, 1] == 0)


def test_quantized_cache_feeds_draft_attention():
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hq, Hkv, cap = 2, 8, 2, 256
    kbits = S.f32_to_bf16_bits(S.normal_f32((B, Hkv, cap, D), 43, S.TID["k"]))
    vbits = S.f32_to_bf16_bits(S.normal_f32((B, Hkv, cap, D), 43, S.TID["v"]))
    qbits = S.f32_to_bf16_bits(S.normal_f32((B, Hq, D), 43, S.TID["q"], std=2.0, slice_dims=1))
    _, cache = _run(kbits, vbits, [[0, 0], [0, 0]], [[0, 0], [0, 0]], cap // 32, cap)
    k_ref = np.empty((B, Hkv, cap, D))
    v_ref = np.empty((B, Hkv, cap, D))
    for b in range(B):
        for h in range(Hkv):
            c, s, z = Q.quantize_k(bf16_to_f64(kbits[b, h]))
            k_ref[b, h] = Q.dequantize_k(c, f16_to_f64(s.view(np.uint16)), f16_to_f64(z.view(np.uint16)))
            c, s, z = Q.quantize_v(bf16_to_f64(vbits[b, h]))
            v_ref[b, h] = Q.dequantize_v(c, f16_to_f64(s.view(np.uint16)), f16_to_f64(z.view(np.uint16)))
    ml = np.array([[256, 200], [37, 256]], np.int32)
    out = vc.draft_attn(to_dev_bf16(qbits), cache["k_codes"], cache["v_codes"], to_dev(ml), fmt=vc.VC_KV_INT4,
                        k_scale=cache["k_scale"], k_zero=cache["k_zero"], v_scale=cache["v_scale"],
                        v_zero=cache["v_zero"])
    torch.cuda.synchronize()
    o_ref, _ = A.draft_attn(bf16_to_f64(qbits), k_ref, v_ref, ml)
    assert_close(bf16_dev_to_f64(out), o_ref, TOL["bf16"], "draft over the device-quantized cache")


def test_quantize_packed_matches_separate_arrays():
    # vc_quantize_int4_packed writes exactly the six arrays' bytes, interleaved per block, and leaves
    # blocks outside the call untouched
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hkv, src_cap, cap, n = 2, 3, 160, 256, 3
    kbits = S.f32_to_bf16_bits(S.normal_f32((B, Hkv, src_cap, D), 44, S.TID["k"], std=1.5))
    vbits = S.f32_to_bf16_bits(S.normal_f32((B, Hkv, src_cap, D), 44, S.TID["v"], std=0.7))
    src = [[0, 7, 64], [31, 0, 64]]
    dst = [[0, 96, 160], [64, 160, 32]]
    sep, _ = _run(kbits, vbits, src, dst, n, cap)
    packed = torch.full((B, Hkv, cap // 32, 5120), SENT8, dtype=torch.uint8, device="cuda")
    vc.quantize_int4_packed(to_dev_bf16(kbits), to_dev_bf16(np.ascontiguousarray(np.swapaxes(vbits, -1, -2))),
                            to_dev(np.asarray(src, np.int32)), n, to_dev(np.asarray(dst, np.int32)), packed)
    torch.cuda.synchronize()
    got = packed.cpu().numpy()
    ref = S.pack_int4_blocks(sep["k_codes"], sep["v_codes"], sep["k_scale"].view(np.uint16),
                             sep["k_zero"].view(np.uint16), sep["v_scale"].view(np.uint16),
                             sep["v_zero"].view(np.uint16))
    for b in range(B):
        for h in range(Hkv):
            blk = slice(dst[b][h] // 32, dst[b][h] // 32 + n)
            np.testing.assert_array_equal(got[b, h, blk], ref[b, h, blk])
            untouched = np.ones(cap // 32, bool)
            untouched[blk] = False
            assert np.all(got[b, h, untouched] == SENT8)


def test_full_size_sampled_slices_bit_exact():
    # The launch configuration of the 128K int4 cache build: 32 requests x 8
    # KV heads, 131072 tokens each (4096 groups per slice).  Three sampled
    # slices are compared with the oracle bit for bit.
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hkv, n = 32, 8, 131072
    dev = "cuda"
    K = S.torch_normal((B, Hkv, n, D), 71, dev, torch.bfloat16, 1.5)
    Vt = S.torch_normal((B, Hkv, D, n), 72, dev, torch.bfloat16, 0.7)   # channel-major
    out = _alloc(B, Hkv, n)
    zeros = torch.zeros((B, Hkv), dtype=torch.int32, device=dev)
    vc.quantize_int4(K, Vt, zeros, n // 32, zeros, **out)
    torch.cuda.synchronize()
    host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    for b, h in [(0, 0), (17, 3), (31, 7)]:
        kb, vb = host(K[b, h]), host(Vt[b, h].t())
        kc, ks, kz = Q.quantize_k(bf16_to_f64(kb))
        vc_, vs, vz = Q.quantize_v(bf16_to_f64(vb))
        np.testing.assert_array_equal(unpack_int4(out["k_codes"][b, h].cpu().numpy()), kc)
        np.testing.assert_array_equal(host(out["k_scale"][b, h]), ks.view(np.uint16))
        np.testing.assert_array_equal(host(out["k_zero"][b, h]), kz.view(np.uint16))
        got_vc = unpack_int4(out["v_codes"][b, h].cpu().numpy()).transpose(0, 2, 1).reshape(-1, D)
        np.testing.assert_array_equal(got_vc, vc_)
        np.testing.assert_array_equal(host(out["v_scale"][b, h]).transpose(0, 2, 1).reshape(-1, D // 32),
                                      vs.view(np.uint16))
        np.testing.assert_array_equal(host(out["v_zero"][b, h]).transpose(0, 2, 1).reshape(-1, D // 32),
                                      vz.view(np.uint16))
