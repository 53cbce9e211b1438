"""GPU checks of the support entry points around the attention kernels:
drafter argmax with an output stride, the commit of verified rows, and the staggered PCIe streamer (data integrity and
independence of results from the schedule)."""
import numpy as np
import pytest

import synthetic as S
from oracle import attention as A
from oracle.accept import greedy_argmax
from oracle.formats import bf16_to_f64

from .helpers import TOL, assert_close, bf16_dev_to_f64, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def test_argmax_strided_output():
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, k, V = 6, 5, 3000
    y, d, n = S.planted_accept(B, k - 1, V, cfg_seed=8, n_lo=0, n_hi=k - 1)
    logits = S.planted_logits(y, V, cfg_seed=8, ties=2)     # [B][k][V]
    drafts = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    for i in range(k):
        vc.argmax(to_dev(np.ascontiguousarray(logits[:, i])), out=drafts.view(-1)[i:], out_stride=k)
    torch.cuda.synchronize()
    ref = np.array([[greedy_argmax(logits[b, i]) for i in range(k)] for b in range(B)])
    np.testing.assert_array_equal(drafts.cpu().numpy(), ref)


@pytest.mark.parametrize("dtype,v_blocked", [("bf16", False), ("fp32", False), ("bf16", True), ("fp32", True)])
def test_commit_rows(dtype, v_blocked):
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, Hkv, M, D, cap = 3, 2, 9, 64, 128
    rng = np.random.default_rng(0)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    bk = torch.randn((B, Hkv, M, D), device="cuda").to(tdt)
    bv = torch.randn((B, Hkv, D, M), device="cuda").to(tdt)
    K = torch.randn((B, Hkv, cap, D), device="cuda").to(tdt)
    Vt = torch.randn((B, Hkv, D, cap), device="cuda").to(tdt)
    if v_blocked:   # [cap/32][D][32]; Vt stays the channel-major view of the same values
        Vdst = Vt.reshape(B, Hkv, D, cap // 32, 32).permute(0, 1, 3, 2, 4).contiguous()
    else:
        Vdst = Vt
    deg = torch.full((B, 1, cap), 3.0, device="cuda")
    L0 = np.array([[10, 10], [120, 120], [0, 0]], np.int32)
    n_out = np.array([4, 9, 1], np.int32)
    length = to_dev(L0)
    K0, V0, D0 = K.cpu().clone(), Vt.cpu().clone(), deg.cpu().clone()
    vc.commit_rows(bk, bv, to_dev(n_out), K, Vdst, length, degree=deg, v_blocked=v_blocked)
    torch.cuda.synchronize()
    if v_blocked:
        Vt = Vdst.permute(0, 1, 3, 2, 4).reshape(B, Hkv, D, cap)
    exp_len = np.minimum(L0 + n_out[:, None], cap)
    np.testing.assert_array_equal(length.cpu().numpy(), exp_len)
    Kh, Vh, Dh = K.cpu(), Vt.cpu(), deg.cpu()
    bkh, bvh = bk.cpu(), bv.cpu()
    for b in range(B):
        for h in range(Hkv):
            L, n = L0[b, h], exp_len[b, h] - L0[b, h]
            assert torch.equal(Kh[b, h, L:L + n], bkh[b, h, :n])
            assert torch.equal(Vh[b, h, :, L:L + n], bvh[b, h, :, :n])
            assert torch.equal(Kh[b, h, :L], K0[b, h, :L]) and torch.equal(Kh[b, h, L + n:], K0[b, h, L + n:])
            assert torch.equal(Vh[b, h, :, :L], V0[b, h, :, :L])
        assert torch.all(Dh[b, 0, L0[b, 0]:exp_len[b, 0]] == 1.0)
        assert torch.equal(Dh[b, 0, exp_len[b, 0]:], D0[b, 0, exp_len[b, 0]:])


def test_stagger_streams_layers_and_matches_direct_verify():
    """Each layer's full cache is streamed host -> slot ring; verify reading
    the slot equals verify reading a resident copy (schedule-independent)."""
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, M, Hq, Hkv, D, N, L = 2, 9, 8, 2, 128, 1024, 5
    half = B * Hkv * N * D * 2
    host = [torch.empty(2 * half, dtype=torch.uint8, pin_memory=True) for _ in range(L)]
    res = []
    for l in range(L):
        k = S.normal_bf16((B, Hkv, N, D), 100 + l, 2)
        v = S.normal_bf16((B, Hkv, D, N), 100 + l, 3)
        host[l][:half].copy_(torch.from_numpy(k.view(np.uint8).reshape(-1)))
        host[l][half:].copy_(torch.from_numpy(v.view(np.uint8).reshape(-1)))
        res.append((to_dev_bf16(k), to_dev_bf16(v)))
    q = to_dev_bf16(S.normal_bf16((B, M, Hq, D), 7, 1, std=3.0, slice_dims=1))
    bk = to_dev_bf16(S.normal_bf16((B, Hkv, M, D), 7, 6))
    bv = to_dev_bf16(S.normal_bf16((B, Hkv, D, M), 7, 7))
    cl = to_dev(np.array([N, N - 100], np.int32))
    slots = [torch.empty(2 * half, dtype=torch.uint8, device="cuda") for _ in range(2)]
    stg = vc.Stagger(slots, 2 * half, L)
    vs = torch.cuda.Stream()
    outs = [torch.empty((B, M, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    stg.stream_layer(0, host[0], 2 * half)
    stg.stream_layer(1, host[1], 2 * half)
    for l in range(L):
        ptr = stg.acquire(l, vs)
        base = slots[0] if ptr == slots[0].data_ptr() else slots[1]
        kk = base[:half].view(torch.bfloat16).view(B, Hkv, N, D)
        vv = base[half:].view(torch.bfloat16).view(B, Hkv, D, N)
        vc.verify_attn(q, kk, vv, cl, bk, bv, out=outs[l], stream=vs)
        stg.release(l, vs)
        if l + 2 < L:
            stg.stream_layer(l + 2, host[l + 2], 2 * half)
    torch.cuda.synchronize()
    stg.sync()
    assert stg.copy_ms(L - 1) > 0
    for l in range(L):
        direct = vc.verify_attn(q, res[l][0], res[l][1], cl, bk, bv)
        torch.cuda.synchronize()
        assert torch.equal(outs[l], direct), l
    stg.close()


@pytest.mark.parametrize("delayed", [(0, 2), (1, 3, 4), (0, 1, 2, 3, 4)])
def test_stagger_slot_reuse_under_forced_delays(delayed):
    """The two-slot ring under forced reorderings: the verify stream stalls
    (a bounded spin kernel) before the chosen layers, so the copy engine is
    ready to run ahead.  A copy into a slot must still wait for the release of
    the layer that last read it: every layer's output stays bit-identical to
    verify over a resident copy of that layer."""
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    B, M, Hq, Hkv, D, N, L = 1, 9, 8, 2, 128, 4096, 5
    half = B * Hkv * N * D * 2
    host = [torch.empty(2 * half, dtype=torch.uint8, pin_memory=True) for _ in range(L)]
    res = []
    for l in range(L):
        k = S.normal_bf16((B, Hkv, N, D), 200 + l, 2)
        v = S.normal_bf16((B, Hkv, D, N), 200 + l, 3)
        host[l][:half].copy_(torch.from_numpy(k.view(np.uint8).reshape(-1)))
        host[l][half:].copy_(torch.from_numpy(v.view(np.uint8).reshape(-1)))
        res.append((to_dev_bf16(k), to_dev_bf16(v)))
    q = to_dev_bf16(S.normal_bf16((B, M, Hq, D), 8, 1, std=3.0, slice_dims=1))
    bk = to_dev_bf16(S.normal_bf16((B, Hkv, M, D), 8, 6))
    bv = to_dev_bf16(S.normal_bf16((B, Hkv, D, M), 8, 7))
    cl = to_dev(np.array([N], np.int32))
    slots = [torch.empty(2 * half, dtype=torch.uint8, device="cuda") for _ in range(2)]
    stg = vc.Stagger(slots, 2 * half, L)
    vs = torch.cuda.Stream()
    outs = [torch.empty((B, M, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in range(L)]
    stg.stream_layer(0, host[0], 2 * half)
    stg.stream_layer(1, host[1], 2 * half)
    for l in range(L):
        ptr = stg.acquire(l, vs)
        if l in delayed:
            with torch.cuda.stream(vs):
                torch.cuda._sleep(20_000_000)   # a few milliseconds of spinning, then it exits
        base = slots[0] if ptr == slots[0].data_ptr() else slots[1]
        kk = base[:half].view(torch.bfloat16).view(B, Hkv, N, D)
        vv = base[half:].view(torch.bfloat16).view(B, Hkv, D, N)
        vc.verify_attn(q, kk, vv, cl, bk, bv, out=outs[l], stream=vs)
        stg.release(l, vs)
        if l + 2 < L:
            stg.stream_layer(l + 2, host[l + 2], 2 * half)
    torch.cuda.synchronize()
    stg.sync()
    for l in range(L):
        direct = vc.verify_attn(q, res[l][0], res[l][1], cl, bk, bv)
        torch.cuda.synchronize()
        assert torch.equal(outs[l], direct), l
    stg.close()


def test_stagger_after_and_writeback_wait_for_the_compute_stream():
    # The compute stream spins for a few milliseconds and then writes; the
    # copy streams are told to wait for it.  The host-to-device copy into the
    # slot must land after that write (the slot ends with the host bytes), and
    # the write-back must read the buffer after it (the host gets the written
    # bytes).  Without the waits the copies would run first.
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    n = 1 << 20
    slot = torch.zeros(n, dtype=torch.uint8, device="cuda")
    src = torch.full((n,), 7, dtype=torch.uint8, pin_memory=True)
    dev_buf = torch.zeros(n, dtype=torch.uint8, device="cuda")
    back = torch.zeros(n, dtype=torch.uint8, pin_memory=True)
    stg = vc.Stagger([slot], n, 1)
    try:
        comp = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(comp):
            torch.cuda._sleep(20_000_000)   # a few milliseconds of spinning, then it exits
            slot.fill_(3)
            dev_buf.fill_(9)
        stg.after(comp)
        stg.stream_layer(0, src, n)
        stg.writeback(back, dev_buf, n, comp)
        stg.sync()
        torch.cuda.synchronize()
        assert bool((slot == 7).all()), "the copy into the slot ran before the compute stream's write"
        assert bool((back == 9).all()), "the write-back read the buffer before the compute stream wrote it"
    finally:
        stg.close()
