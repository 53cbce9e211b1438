"""CPU checks of the C ABI: the library loads and exports every function the
public header declares, the ctypes structs match the C layout (compiled with
gcc from include/vc.h), and argument validation rejects bad calls before
any GPU work."""
import ctypes
import os
import subprocess
import tempfile

import pytest

import lossless_speculative_decoding_vc_amd as vcb
from lossless_speculative_decoding_vc_amd import build as vbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(vbuild.LIB):
        vbuild.build()
    return vcb.lib()


def test_exports_every_declared_symbol(L):
    names = vcb.declared_symbols()
    assert {"vc_draft_attn", "vc_verify_attn", "vc_accept"} <= set(names)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def _c_layout(struct, fields):
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"vc_tiny.h\"\n#include \"vc.h\"\nint main(void){\n"
    src += f'printf("%zu\\n", sizeof({struct}));\n'
    for f in fields:
        src += f'printf("%zu\\n", offsetof({struct}, {f}));\n'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "l.c")
        exe = os.path.join(d, "l")
        with open(c, "w") as fh:
            fh.write(src)
        subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split()
    return [int(x) for x in out]


@pytest.mark.parametrize("cls,cname", [(vcb.DraftArgs, "vc_draft_args"),
                                       (vcb.VerifyArgs, "vc_verify_args"),
                                       (vcb.AcceptArgs, "vc_accept_args"),
                                       (vcb.RoundCommit, "vc_round_commit"),
                                       (vcb.RoundDesc, "vc_round_desc"),
                                       (vcb.RoundFetch, "vc_round_fetch"),
                                       ("TinyModelArgs", "vc_tiny_model"),
                                       ("TinyAttnArgs", "vc_tiny_attn")])
def test_struct_layout_matches_header(cls, cname):
    if isinstance(cls, str):
        import lossless_speculative_decoding_vc_amd.tiny_loop as tl
        cls = getattr(tl, cls)
    fields = [f[0] for f in cls._fields_]
    got = [ctypes.sizeof(cls)] + [getattr(cls, f).offset for f in fields]
    assert got == _c_layout(cname, fields)


def _draft(**kw):
    a = vcb.DraftArgs()
    a.B, a.Hq, a.Hkv, a.D, a.dtype, a.fmt, a.scale, a.cap = 2, 8, 2, 128, 0, 0, 0.088, 1024
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_validation_rejects_before_launch(L):
    # every one of these fails host-side validation; nothing reaches the GPU
    cases = [_draft(Hq=7), _draft(D=96), _draft(cap=1000), _draft(scale=0.0), _draft(dtype=5)]
    codes = [L.vc_draft_attn(ctypes.byref(a), None) for a in cases]
    assert codes == [vcb.VC_EINVAL, vcb.VC_ENOTSUP, vcb.VC_EINVAL, vcb.VC_EINVAL, vcb.VC_EINVAL]
    # missing pointers with a non-empty batch
    assert L.vc_draft_attn(ctypes.byref(_draft()), None) == vcb.VC_EINVAL
    assert b"required" in L.vc_last_error()
    v = vcb.VerifyArgs()
    v.B, v.Hq, v.Hkv, v.D, v.M, v.scale, v.ccap = 1, 64, 8, 128, 0, 0.088, 64
    assert L.vc_verify_attn(ctypes.byref(v), None) == vcb.VC_EINVAL
    acc = vcb.AcceptArgs()
    acc.B, acc.M, acc.V = 1, 0, 10
    assert L.vc_accept(ctypes.byref(acc), None) == vcb.VC_EINVAL
    assert L.vc_status_string(2) == b"VC_ENOTSUP"
    # token indices inside the kernels are 32-bit: capacities are bounded
    assert L.vc_draft_attn(ctypes.byref(_draft(cap=1 << 30, tcap=64)), None) == vcb.VC_EINVAL
    assert b"2^30" in L.vc_last_error()
    v2 = vcb.VerifyArgs()
    v2.B, v2.Hq, v2.Hkv, v2.D, v2.M, v2.scale, v2.ccap = 1, 16, 1, 128, 33, 0.088, (1 << 30) + 64
    assert L.vc_verify_attn(ctypes.byref(v2), None) == vcb.VC_EINVAL
    v2.ccap, v2.M = 64, 65535 * 4 + 1   # 16 * M packed rows need more than 65535 row groups of 64
    assert L.vc_verify_attn(ctypes.byref(v2), None) == vcb.VC_EINVAL
    assert b"65535 * 64" in L.vc_last_error()
    # (request, KV head) slices index a grid dimension capped at 65535
    assert L.vc_draft_attn(ctypes.byref(_draft(B=40000, Hq=4, Hkv=2)), None) == vcb.VC_EINVAL
    assert b"65535" in L.vc_last_error()
    # packed int4: bf16 queries and head_dim 128 only; the cache lives in k alone
    assert L.vc_draft_attn(ctypes.byref(_draft(fmt=2, dtype=1)), None) == vcb.VC_ENOTSUP
    assert L.vc_draft_attn(ctypes.byref(_draft(fmt=2, D=64)), None) == vcb.VC_ENOTSUP
    assert L.vc_draft_attn(ctypes.byref(_draft(fmt=3)), None) == vcb.VC_EINVAL
    fake = 1 << 20
    a = _draft(fmt=2, q=fake, out=fake, main_len=fake, k=fake, v=fake)
    assert L.vc_draft_attn(ctypes.byref(a), None) == vcb.VC_EINVAL
    assert b"NULL" in L.vc_last_error()


def test_workspace_plan_is_host_only(L):
    # c3 draft shape: 32 x 8 KV heads, 32768 compressed tokens -> split partials
    a = _draft(B=32, Hq=32, Hkv=8, cap=32768)
    ws = L.vc_draft_workspace_size(ctypes.byref(a))
    # one partial row (D values and a log-sum-exp) per split and query head
    assert ws > 0 and ws % (32 * 32 * 129 * 4) == 0
    # fp32 mode runs unsplit
    assert L.vc_draft_workspace_size(ctypes.byref(_draft(dtype=1))) == 0


def test_lm_head_argmax_validation_is_host_only(L):
    # the fused LM head + argmax: bad shapes, null pointers and a short
    # workspace are rejected before any GPU work
    fake = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced on these paths
    ws_need = L.vc_lm_head_argmax_workspace_size(528, 32768)
    # one (max, index) pair per row and 256-entry (128-entry for drafting rows) vocabulary tile
    assert ws_need == 528 * 128 * 8
    assert L.vc_lm_head_argmax_workspace_size(16, 32768) == 16 * 256 * 8
    assert L.vc_lm_head_argmax(4, 48, 100, fake, fake, fake, 1, fake, 1 << 20, None) == vcb.VC_ENOTSUP
    assert L.vc_lm_head_argmax(4, 64, 100, fake, fake, fake, 1, fake, 8, None) == vcb.VC_EINVAL
    assert b"workspace" in L.vc_last_error()
    assert L.vc_lm_head_argmax(4, 64, 100, None, fake, fake, 1, fake, 1 << 20, None) == vcb.VC_EINVAL
    assert L.vc_lm_head_argmax(4, 64, 100, fake, fake, fake, 0, fake, 1 << 20, None) == vcb.VC_EINVAL
    assert L.vc_lm_head_argmax(0, 64, 100, None, None, None, 1, None, 0, None) == vcb.VC_OK
    assert L.vc_lm_head_accept(2, 3, 64, 100, fake, fake, None, fake, fake, fake, fake, fake, 1 << 20,
                               None) == vcb.VC_EINVAL   # M > 1 needs drafts
    assert L.vc_lm_head_accept(0, 3, 64, 100, None, None, None, None, None, None, None, None, 0,
                               None) == vcb.VC_OK


def test_compact_kv_validation_is_host_only(L):
    fake = ctypes.c_void_p(1 << 20)
    args = lambda **kw: [kw.get(k, d) for k, d in (("B", 2), ("Hkv", 2), ("D", 128), ("dtype", 0), ("sk", fake),
                                                    ("sv", fake), ("src_cap", 256), ("idx", fake), ("stride", 64),
                                                    ("n", fake), ("dk", fake), ("dv", fake), ("cap", 64),
                                                    ("dl", None), ("s", None))]
    assert L.vc_compact_kv(*args(dtype=5)) == vcb.VC_EINVAL
    assert L.vc_compact_kv(*args(D=96)) == vcb.VC_ENOTSUP
    assert L.vc_compact_kv(*args(cap=40)) == vcb.VC_EINVAL
    assert L.vc_compact_kv(*args(idx=None)) == vcb.VC_EINVAL
    assert L.vc_compact_kv(*args(stride=0)) == vcb.VC_EINVAL
    assert L.vc_compact_kv(*args(B=0, sk=None)) == vcb.VC_OK


def test_empty_batches_return_before_any_gpu_call(L):
    # an empty batch (B = 0, R = 0 or no groups) is a valid call that enqueues
    # nothing: NULL tensors are accepted and no HIP call is made, which is why
    # these succeed on a machine without a GPU
    d = _draft(B=0)
    assert L.vc_draft_attn(ctypes.byref(d), None) == vcb.VC_OK
    assert L.vc_draft_workspace_size(ctypes.byref(d)) == 0
    v = vcb.VerifyArgs()
    v.B, v.Hq, v.Hkv, v.D, v.M, v.scale, v.ccap = 0, 40, 8, 128, 33, 0.088, 131072
    assert L.vc_verify_attn(ctypes.byref(v), None) == vcb.VC_OK
    acc = vcb.AcceptArgs()
    acc.B, acc.M, acc.V = 0, 33, 32768
    assert L.vc_accept(ctypes.byref(acc), None) == vcb.VC_OK
    assert L.vc_argmax(0, 32768, 1, None, None, 1, None) == vcb.VC_OK
    assert L.vc_commit_rows(0, 8, 128, 33, 0, 1024, 0, None, None, None, None, None, None, None, 0,
                            None) == vcb.VC_OK
    assert L.vc_quantize_int4(0, 8, 128, None, None, 64, None, 1, 64, None, None, None, None, None, None, None,
                              None) == vcb.VC_OK
    assert L.vc_quantize_int4_packed(2, 8, 128, None, None, 64, None, 0, 64, None, None, None) == vcb.VC_OK
    # a non-empty call with the same NULL tensors is rejected
    assert L.vc_argmax(4, 32768, 1, None, None, 1, None) == vcb.VC_EINVAL
    assert L.vc_quantize_int4_packed(2, 8, 128, None, None, 64, None, 1, 64, None, None, None) == vcb.VC_EINVAL


def test_stagger_create_failure_leaves_nothing_behind(L):
    # without a usable device the first stream creation fails: the call
    # reports that HIP error (not one from the cleanup), frees the partly
    # built object and leaves the output handle untouched
    h = ctypes.c_void_p(0)
    slots = (ctypes.c_void_p * 2)(1 << 20, 2 << 20)
    r = L.vc_stagger_create(ctypes.byref(h), slots, 2, 1024, 4)
    if r == vcb.VC_OK:
        assert L.vc_stagger_destroy(h) == vcb.VC_OK
        pytest.skip("a GPU is present: creation succeeded")
    assert r == vcb.VC_EHIP
    assert b"hipStreamCreateWithFlags" in L.vc_last_error()
    assert h.value is None
    # argument errors come before any HIP call
    assert L.vc_stagger_create(ctypes.byref(h), slots, 0, 1024, 4) == vcb.VC_EINVAL
    assert L.vc_stagger_destroy(None) == vcb.VC_OK


def test_csm_and_commit_validation_is_host_only(L):
    from oracle import csm as C
    fake = ctypes.c_void_p(1 << 20)
    n = ctypes.c_int32(-1)
    base = dict(B=2, Hkv=2, D=128, n_in=300, sink=4, recent=16, chunk=64, r=1.0, ik=fake, iv=fake, ideg=None,
                cap_in=320, ok=fake, ov=fake, odeg=fake, cap_out=320)

    def csm(**kw):
        a = {**base, **kw}
        return L.vc_csm_round(a["B"], a["Hkv"], a["D"], a["n_in"], a["sink"], a["recent"], a["chunk"], a["r"],
                              a["ik"], a["iv"], a["ideg"], a["cap_in"], a["ok"], a["ov"], a["odeg"], a["cap_out"],
                              ctypes.byref(n), None, None)
    assert csm(D=64) == vcb.VC_ENOTSUP
    assert csm(chunk=1) == vcb.VC_EINVAL
    assert csm(r=1.5) == vcb.VC_EINVAL
    assert csm(sink=200, recent=200) == vcb.VC_EINVAL
    assert csm(cap_out=64) == vcb.VC_EINVAL       # the round keeps more tokens than that
    assert csm(ik=None) == vcb.VC_EINVAL
    # an empty batch still reports how many tokens the round keeps, as the oracle counts them
    assert csm(B=0, ik=None, iv=None, ok=None, ov=None, odeg=None) == vcb.VC_OK
    assert n.value == C.survivors(300, 4, 16, 64, 1.0)

    def commit(**kw):
        a = dict(B=2, Hkv=2, D=128, M=9, dtype=0, cap=1024, blocked=0, bk=fake, bv=fake, no=fake, dk=fake, dv=fake,
                 ln=fake, deg=None, dhs=0)
        a.update(kw)
        return L.vc_commit_rows(a["B"], a["Hkv"], a["D"], a["M"], a["dtype"], a["cap"], a["blocked"], a["bk"],
                                a["bv"], a["no"], a["dk"], a["dv"], a["ln"], a["deg"], a["dhs"], None)
    assert commit(dtype=7) == vcb.VC_EINVAL
    assert commit(blocked=1, cap=1000) == vcb.VC_EINVAL
    assert commit(deg=fake, dhs=5) == vcb.VC_EINVAL
    assert commit(ln=None) == vcb.VC_EINVAL
    assert commit(B=0, bk=None, bv=None, no=None, dk=None, dv=None, ln=None) == vcb.VC_OK


def test_csm_survivor_count_matches_oracle_on_many_shapes(L):
    # the library's survivor count (host integer arithmetic, reported even for
    # an empty batch) equals the oracle's over a seeded sweep of shapes,
    # including r at 0 and 1, chunks of 2 and 128, and no middle segment
    import numpy as np
    from oracle import csm as C
    rng = np.random.default_rng(5)
    n = ctypes.c_int32(-1)
    cases = [(40, 20, 20, 2, 1.0), (40, 0, 0, 128, 0.0), (1, 0, 0, 64, 1.0), (131072, 4, 1024, 64, 1.0),
             # ratios of a decaying schedule that float32 would round down: floor(0.7 * 10) = 7 needs r in double
             (4 + 6 * 20 + 8, 4, 8, 20, 0.7), (4 + 3 * 40 + 8, 4, 8, 40, 0.9), (100, 0, 0, 20, 0.7),
             (1000, 4, 64, 64, 1.0 - 3 * 0.1)]
    for _ in range(200):
        n_in = int(rng.integers(1, 5000))
        sink = int(rng.integers(0, 40))
        recent = int(rng.integers(0, 200))
        if sink + recent > n_in:
            continue
        cases.append((n_in, sink, recent, int(rng.integers(2, 129)), float(rng.random())))
    for n_in, sink, recent, chunk, r in cases:
        cap = (n_in + 31) // 32 * 32
        st = L.vc_csm_round(0, 2, 128, n_in, sink, recent, chunk, r, None, None, None, cap, None, None, None, cap,
                            ctypes.byref(n), None, None)
        assert st == vcb.VC_OK, (n_in, sink, recent, chunk, r, L.vc_last_error())
        assert n.value == C.survivors(n_in, sink, recent, chunk, r), (n_in, sink, recent, chunk, r)


def test_centroid_schedule_functions_match_the_oracle(L):
    # the library's CentroidKV schedule (when a round runs, with which ratio)
    # drives the same sequence of rounds as the oracle's pipeline, on the
    # hand-derived golden and on a longer run
    import json
    import numpy as np
    from oracle import csm as C
    for j in range(12):
        for r_init, dr in ((1.0, 0.1), (0.75, 0.25), (0.5, 0.0), (1.2, 0.3)):
            assert L.vc_csm_schedule_ratio(r_init, dr, j) == C.schedule_ratio(j, r_init, dr)
    assert L.vc_csm_round_due(10, 5, 3, 0) == -1 and L.vc_csm_round_due(10, 5, -1, 4) == -1
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "centroid_schedule.json")))
    for cfg, steps, n0 in ((g["config"], g["config"]["decode_steps"], g["config"]["n_prefill"]),
                           (dict(n_sink=4, n_recent=32, chunk=32, budget=250, every=32, r_init=0.75, delta_r=0.125),
                            160, 400)):
        rng = np.random.default_rng(3)
        k0, v0 = rng.standard_normal((n0, 8)), rng.standard_normal((n0, 8))
        kn, vn = rng.standard_normal((steps, 8)), rng.standard_normal((steps, 8))
        _, _, _, rounds = C.centroid_run(k0, v0, kn, vn, cfg["budget"], cfg["every"], cfg["r_init"], cfg["delta_r"],
                                         cfg["n_sink"], cfg["n_recent"], cfg["chunk"])
        # replay the schedule with the library's decisions and survivor counts
        n, j, lib_rounds = n0, 0, []
        for step in range(steps + 1):
            if step > 0:
                n += 1
            if L.vc_csm_round_due(n, cfg["budget"], step, cfg["every"]) == 1:
                r = L.vc_csm_schedule_ratio(cfg["r_init"], cfg["delta_r"], j)
                cnt = ctypes.c_int32(-1)
                cap = (n + 31) // 32 * 32
                assert L.vc_csm_round(0, 1, 128, n, cfg["n_sink"], cfg["n_recent"], cfg["chunk"], r, None, None, None,
                                      cap, None, None, None, cap, ctypes.byref(cnt), None, None) == vcb.VC_OK
                lib_rounds.append((step, j, r, n, cnt.value))
                n, j = cnt.value, j + 1
        assert lib_rounds == [(rd["step"], rd["j"], rd["r"], rd["n_in"], rd["n_out"]) for rd in rounds]
