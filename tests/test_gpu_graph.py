"""The hot-path entry points enqueue only kernels on the caller's stream (no
allocation, memset or synchronization inside), so a round's steps can be
captured into a HIP graph: one draft step (vc_draft_attn, then
vc_lm_head_argmax writing the next draft column) and one verify step
(vc_verify_attn, then vc_lm_head_accept), captured once and replayed several
times with eager work and synchronizations between the replays, give the
eager result bit for bit on every replay."""
import numpy as np
import pytest

import synthetic as S

pytestmark = pytest.mark.gpu


def test_round_steps_replay_from_a_graph():
    import torch
    import lossless_speculative_decoding_vc_amd as vc
    dev = "cuda"
    B, Hq, Hkv, D, cap, ccap, M, Dm, V = 4, 16, 4, 128, 2048, 1024, 9, 256, 1000
    bf = torch.bfloat16
    rnd = lambda shape, seed, std=1.0: S.torch_normal(shape, seed, dev, bf, std)
    q_d = rnd((B, Hq, D), 1, 2.0)
    K, Vb = rnd((B, Hkv, cap, D), 2), rnd((B, Hkv, cap // 32, D, 32), 3)
    ml = torch.tensor([[2048, 1999, 1000, 64]] * Hkv, dtype=torch.int32, device=dev).t().contiguous()
    deg = S.torch_randint((B, 1, cap), 1, 5, 4, dev, torch.int32).float()
    q_v = rnd((B, M, Hq, D), 5, 2.0)
    ck, cv = rnd((B, Hkv, ccap, D), 6), rnd((B, Hkv, D, ccap), 7)
    cl = torch.tensor([1024, 700, 3, 0], dtype=torch.int32, device=dev)
    bk, bv = rnd((B, Hkv, M, D), 8), rnd((B, Hkv, D, M), 9)
    W = rnd((V, Dm), 10, 0.05)
    h_d, h_v = rnd((B, Dm), 11), rnd((B, M, Dm), 12)
    # outputs and workspaces, allocated before capture
    o_d = torch.empty((B, Hq, D), dtype=bf, device=dev)
    o_v = torch.empty((B, M, Hq, D), dtype=bf, device=dev)
    drafts = torch.zeros((B, M - 1), dtype=torch.int32, device=dev)
    am = torch.empty((B, M), dtype=torch.int32, device=dev)
    al = torch.empty(B, dtype=torch.int32, device=dev)
    toks = torch.empty((B, M), dtype=torch.int32, device=dev)
    nout = torch.empty(B, dtype=torch.int32, device=dev)
    ws = vc.new_workspace(1 << 24, dev)
    ws_lm_d = vc.lm_head_argmax_workspace(B, V, dev)
    ws_lm_v = vc.lm_head_argmax_workspace(B * M, V, dev)

    def steps():
        vc.draft_attn(q_d, K, Vb, ml, degree=deg, out=o_d, workspace=ws)
        vc.lm_head_argmax(h_d, W, out=drafts.view(-1)[3:], out_stride=M - 1, workspace=ws_lm_d)   # draft column 3
        vc.verify_attn(q_v, ck, cv, cl, bk, bv, out=o_v, workspace=ws)
        vc.lm_head_accept(h_v, W, drafts, argmax=am, accept_len=al, out_tokens=toks, n_out=nout,
                          workspace=ws_lm_v)

    outs = (o_d, drafts, o_v, am, al, toks, nout)
    steps()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        steps()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:                    # eager work between replays: clear every output
            if t is not drafts:
                t.fill_(-1 if t.dtype == torch.int32 else float("nan"))
        drafts.zero_()                    # an input as well: back to its state before the first call
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("draft out", "drafts", "verify out", "argmax", "accept_len", "tokens", "n_out"),
                                   outs, ref):
            assert torch.equal(got.view(torch.int16) if got.dtype == bf else got,
                               want.view(torch.int16) if want.dtype == bf else want), (rep, name)
