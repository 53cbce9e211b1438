"""GPU parity of vc_csm_round (one Chunked Soft Matching round) against the
oracle: on key sets with planted near-duplicates (every merge decision far
from a tie) the survivor count and order, the degrees (exactly), the unmerged
tokens (bit-exactly) and the centroids (bf16 tolerance) match; r = 0 copies;
on plain random keys the degree and degree-weighted-sum invariants hold and
every round is one of the valid results (matches and merged set within the
fp32 cosine error of the exact ones, tests/csm_check.py); and
the merged cache with its degrees feeds vc_draft_attn (attention over the
oracle's merged cache with the log-degree term)."""
import numpy as np
import pytest

import synthetic as S
from oracle import attention as A
from oracle import csm as C
from oracle.formats import bf16_to_f64

from .helpers import TOL, assert_close, bf16_dev_to_f64, blocked32, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
D = 128


def _plant(r):
    return lambda L: int(np.floor(r * ((L + 1) // 2)))


def _run(kbits, vbits, deg, n_in, sink, recent, chunk, r, cap_out):
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hkv, cap_in = kbits.shape[:3]
    dev = "cuda"
    out_k = torch.zeros((B, Hkv, cap_out, D), dtype=torch.bfloat16, device=dev)
    out_v = torch.zeros((B, Hkv, cap_out // 32, D, 32), dtype=torch.bfloat16, device=dev)
    out_deg = torch.zeros((B, Hkv, cap_out), dtype=torch.float32, device=dev)
    n_out = vc.csm_round(to_dev_bf16(kbits), to_dev_bf16(blocked32(vbits)), n_in, sink, recent, chunk, r, out_k, out_v,
                         out_deg, in_deg=None if deg is None else to_dev(deg.astype(np.float32)))
    torch.cuda.synchronize()
    ok = out_k.view(torch.int16).cpu().numpy().view(np.uint16)
    ov = out_v.view(torch.int16).cpu().numpy().view(np.uint16)
    ov = ov.transpose(0, 1, 2, 4, 3).reshape(B, Hkv, cap_out, D)   # back to token-major
    return n_out, ok, ov, out_deg.cpu().numpy(), (out_k, out_v, out_deg)


def _case(B, Hkv, n_in, sink, recent, chunk, r, seed, with_deg=True):
    cap_in = ((n_in + 31) // 32) * 32
    k, v, _ = S.csm_planted(B, Hkv, n_in, D, sink, recent, chunk, _plant(r), seed)
    kb = np.zeros((B, Hkv, cap_in, D), np.uint16)
    vb = np.zeros((B, Hkv, cap_in, D), np.uint16)
    kb[:, :, :n_in] = S.f32_to_bf16_bits(k)
    vb[:, :, :n_in] = S.f32_to_bf16_bits(v)
    deg = None
    if with_deg:
        deg = np.ones((B, Hkv, cap_in), np.float32)
        deg[:, :, :n_in] = S.degrees((B, Hkv, n_in), seed)
    return kb, vb, deg, cap_in


@pytest.mark.parametrize("n_in,sink,recent,chunk,r", [(4 + 5 * 64 + 23 + 16, 4, 16, 64, 1.0),
                                                      (300, 0, 32, 64, 0.5), (260, 8, 8, 128, 0.75),
                                                      (200, 4, 4, 16, 0.25),
                                                      # ratios a float32 would round below the exact count:
                                                      # floor(0.7 * 10) = 7, floor(0.9 * 20) = 18
                                                      (4 + 6 * 20 + 11 + 8, 4, 8, 20, 0.7),
                                                      (4 + 3 * 40 + 8, 4, 8, 40, 0.9)])
def test_planted_round_matches_oracle(n_in, sink, recent, chunk, r):
    B, Hkv = 2, 2
    kb, vb, deg, cap_in = _case(B, Hkv, n_in, sink, recent, chunk, r, seed=51)
    cap_out = cap_in
    n_out, ok, ov, od, _ = _run(kb, vb, deg, n_in, sink, recent, chunk, r, cap_out)
    rr = r   # the caller's ratio, unrounded: the merge count is floor(r * |A|) in double
    assert n_out == C.survivors(n_in, sink, recent, chunk, rr)
    for b in range(B):
        for h in range(Hkv):
            kx, vx = bf16_to_f64(kb[b, h, :n_in]), bf16_to_f64(vb[b, h, :n_in])
            k2, v2, d2, info = C.csm_round(kx, vx, deg[b, h, :n_in], sink, recent, chunk, rr)
            assert len(k2) == n_out
            np.testing.assert_array_equal(od[b, h, :n_out], d2.astype(np.float32))
            # survivors that absorbed nothing are copied bit-exactly
            pos = _survivor_positions(info, n_in)
            unmerged = np.array([_absorbed(info, p) == 0 for p in pos])
            np.testing.assert_array_equal(ok[b, h, :n_out][unmerged], kb[b, h, pos[unmerged]])
            np.testing.assert_array_equal(ov[b, h, :n_out][unmerged], vb[b, h, pos[unmerged]])
            assert_close(bf16_to_f64(ok[b, h, :n_out]), k2, 1e-2, "centroid keys")
            assert_close(bf16_to_f64(ov[b, h, :n_out]), v2, 1e-2, "centroid values")


def _survivor_positions(info, n):
    gone = set()
    for c in info:
        for i in np.nonzero(c["merged"])[0]:
            gone.add(c["start"] + 2 * int(i))
    return np.array([p for p in range(n) if p not in gone])


def _absorbed(info, p):
    for c in info:
        if c["start"] <= p < c["end"] and (p - c["start"]) % 2 == 1:
            j = (p - c["start"]) // 2
            return int(np.sum(c["merged"] & (c["match"] == j)))
    return 0


def test_r_zero_copies():
    kb, vb, deg, cap_in = _case(1, 2, 150, 4, 8, 32, 0.0, seed=52)
    n_out, ok, ov, od, _ = _run(kb, vb, deg, 150, 4, 8, 32, 0.0, cap_in)
    assert n_out == 150
    np.testing.assert_array_equal(ok[:, :, :150], kb[:, :, :150])
    np.testing.assert_array_equal(ov[:, :, :150], vb[:, :, :150])
    np.testing.assert_array_equal(od[:, :, :150], deg[:, :, :150])


def test_random_keys_conserve_degree_and_weighted_sums():
    B, Hkv, n_in, chunk = 2, 2, 500, 64
    k = S.normal_f32((B, Hkv, 512, D), 53, S.TID["k"])
    v = S.normal_f32((B, Hkv, 512, D), 53, S.TID["v"])
    kb, vb = S.f32_to_bf16_bits(k), S.f32_to_bf16_bits(v)
    deg = S.degrees((B, Hkv, 512), 53)
    n_out, ok, ov, od, _ = _run(kb, vb, deg, n_in, 4, 16, chunk, 0.5, 512)
    assert n_out == C.survivors(n_in, 4, 16, chunk, 0.5)
    for b in range(B):
        for h in range(Hkv):
            assert od[b, h, :n_out].sum() == deg[b, h, :n_in].sum()
            ws_in = (deg[b, h, :n_in, None] * bf16_to_f64(kb[b, h, :n_in])).sum(0)
            ws_out = (od[b, h, :n_out, None] * bf16_to_f64(ok[b, h, :n_out])).sum(0)
            np.testing.assert_allclose(ws_out, ws_in, rtol=0, atol=0.05 * np.abs(deg[b, h, :n_in]).sum() ** 0.5)


@pytest.mark.parametrize("r,chunk", [(0.25, 64), (0.5, 64), (1.0, 37), (0.7, 20)])
def test_random_keys_round_is_a_valid_round(r, chunk):
    # generic keys: near-equal cosines may be ordered differently by the
    # kernel's fp32 arithmetic, so the outputs are checked for being one of
    # the correct results (tests/csm_check.py) rather than the oracle's
    from .csm_check import check_round
    B, Hkv, n_in = 2, 2, 600
    k = S.normal_f32((B, Hkv, 608, D), 55, S.TID["k"])
    v = S.normal_f32((B, Hkv, 608, D), 55, S.TID["v"])
    kb, vb = S.f32_to_bf16_bits(k), S.f32_to_bf16_bits(v)
    deg = S.degrees((B, Hkv, 608), 55)
    n_out, ok, ov, od, _ = _run(kb, vb, deg, n_in, 4, 64, chunk, r, 608)
    for b in range(B):
        for h in range(Hkv):
            check_round(kb[b, h, :n_in], vb[b, h, :n_in], deg[b, h, :n_in], 4, 64, chunk, r,
                        ok[b, h, :n_out], ov[b, h, :n_out], od[b, h, :n_out])


def test_merged_cache_feeds_draft_attention():
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hq, Hkv, n_in, chunk, r = 2, 8, 2, 400, 64, 1.0
    kb, vb, deg, cap_in = _case(B, Hkv, n_in, 4, 16, chunk, r, seed=54)
    n_out, ok, ov, od, (tk, tv, tdeg) = _run(kb, vb, deg, n_in, 4, 16, chunk, r, 448)   # the drafter takes cap % 64 == 0
    qbits = S.f32_to_bf16_bits(S.normal_f32((B, Hq, D), 54, S.TID["q"], std=2.0, slice_dims=1))
    ml = np.full((B, Hkv), n_out, np.int32)
    out = vc.draft_attn(to_dev_bf16(qbits), tk, tv, to_dev(ml), degree=tdeg)
    torch.cuda.synchronize()
    k_ref = np.zeros((B, Hkv, n_out, D))
    v_ref = np.zeros((B, Hkv, n_out, D))
    d_ref = np.zeros((B, Hkv, n_out))
    for b in range(B):
        for h in range(Hkv):
            k_ref[b, h], v_ref[b, h], d_ref[b, h], _ = C.csm_round(bf16_to_f64(kb[b, h, :n_in]), bf16_to_f64(vb[b, h, :n_in]),
                                                                   deg[b, h, :n_in], 4, 16, chunk, r)
    o_ref, _ = A.draft_attn(bf16_to_f64(qbits), k_ref, v_ref, ml, degree=d_ref)
    assert_close(bf16_dev_to_f64(out), o_ref, TOL["bf16"], "draft over the merged cache")


def _survivors_and_unmerged(info, n):
    """Vectorised form of the two helpers above for long sequences: the
    surviving positions and, for each, whether it absorbed no token."""
    gone = np.zeros(n, bool)
    absorbed = np.zeros(n, np.int64)
    for c in info:
        m = np.asarray(c["merged"], bool)
        if not m.any():
            continue
        gone[c["start"] + 2 * np.nonzero(m)[0]] = True
        cnt = np.bincount(np.asarray(c["match"])[m], minlength=(c["end"] - c["start"]) // 2)
        absorbed[c["start"] + 2 * np.arange(len(cnt)) + 1] += cnt
    pos = np.nonzero(~gone)[0]
    return pos, absorbed[pos] == 0


def test_full_size_round_sampled_slices():
    # The launch configuration of the 128K cohort round: 16 requests x 8 KV
    # heads, 131072 tokens, 4 sinks, 1024 recent tokens, chunks of 64, r = 1,
    # no input degrees.  Two slices hold planted keys and are checked against
    # the oracle; every slice keeps the same number of tokens and its degrees
    # (token counts) add up to the input length.
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hkv, n, sink, recent, chunk, r = 16, 8, 131072, 4, 1024, 64, 1.0
    cap_out = n // 2 + 1024
    dev = "cuda"
    K = S.torch_normal((B, Hkv, n, D), 61, dev, torch.bfloat16, 1.0)
    V = S.torch_normal((B, Hkv, n // 32, D, 32), 62, dev, torch.bfloat16, 1.0)
    samples = [(0, 0), (11, 5)]
    planted = {}
    for i, (b, h) in enumerate(samples):
        k, v, _ = S.csm_planted(1, 1, n, D, sink, recent, chunk, _plant(r), 63 + i)
        kb, vb = S.f32_to_bf16_bits(k[0, 0]), S.f32_to_bf16_bits(v[0, 0])
        planted[(b, h)] = (kb, vb)
        K[b, h] = to_dev_bf16(kb)
        V[b, h] = to_dev_bf16(blocked32(vb))
    ok = torch.zeros((B, Hkv, cap_out, D), dtype=torch.bfloat16, device=dev)
    ov = torch.zeros((B, Hkv, cap_out // 32, D, 32), dtype=torch.bfloat16, device=dev)
    od = torch.zeros((B, Hkv, cap_out), dtype=torch.float32, device=dev)
    n_out = vc.csm_round(K, V, n, sink, recent, chunk, r, ok, ov, od)
    torch.cuda.synchronize()
    del K, V
    assert n_out == C.survivors(n, sink, recent, chunk, r)
    deg_all = od[:, :, :n_out].double().sum(-1).cpu().numpy()
    np.testing.assert_array_equal(deg_all, np.full((B, Hkv), float(n)))
    for (b, h), (kb, vb) in planted.items():
        k2, v2, d2, info = C.csm_round(bf16_to_f64(kb), bf16_to_f64(vb), np.ones(n), sink, recent, chunk, r)
        assert len(k2) == n_out
        got_d = od[b, h, :n_out].cpu().numpy()
        np.testing.assert_array_equal(got_d, d2.astype(np.float32))
        got_k = ok[b, h, :n_out].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        got_v = (ov[b, h].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                 .transpose(0, 2, 1).reshape(cap_out, D)[:n_out])
        pos, unmerged = _survivors_and_unmerged(info, n)
        np.testing.assert_array_equal(got_k[unmerged], kb[pos[unmerged]])
        np.testing.assert_array_equal(got_v[unmerged], vb[pos[unmerged]])
        assert_close(bf16_to_f64(got_k), k2, 1e-2, "centroid keys")
        assert_close(bf16_to_f64(got_v), v2, 1e-2, "centroid values")
