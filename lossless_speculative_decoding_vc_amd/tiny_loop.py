"""The draft-then-verify loop on the GPU for the small fp32 decoder of
``include/vc_tiny.h``.

"Riepilogo Tecnico: VeriCache", section "Algoritmo Principale": the model
drafts k tokens over its compressed cache, one forward pass over the full
cache verifies them, tokens are accepted up to the first mismatch (plus the
bonus token on a full match) and decoding resumes from the last accepted
token.  Every step runs in libvc kernels: the compacted cache
(vc_gather_evict), forward passes (vc_tiny_forward), drafter argmax
(vc_argmax), acceptance (vc_accept), commit of the verified rows
(vc_commit_rows) and the next round's first input (vc_next_input).

A round's state lives on the device -- the committed length (which also
gives the positions and the kept set of the compressor), the drafted and
emitted tokens -- so the round is enqueued the same way every time: it is
captured into a HIP graph once, after the prefill, and every round replays
it.  The host reads one small
record per round (drafts, predictions, accept length, emitted tokens).

The eviction compressor keeps the attention sinks, the most recent tokens
and every ``stride``-th older token (sinks and recent tokens are preserved as
in "Riassunto Tecnico: CentroidKV", "Componenti Chiave", item 2); its kept
positions are a pure function of the committed length and are computed on
the device.
"""
import ctypes

import numpy as np
import torch

from . import (_check, _p, _i32, _i64, _stream, accept, argmax, commit_rows, lib, next_input)

MAXL = 16


class TinyModelArgs(ctypes.Structure):
    _fields_ = [("n_layers", _i32), ("d_model", _i32), ("n_q_heads", _i32), ("n_kv_heads", _i32),
                ("head_dim", _i32), ("ffn", _i32), ("vocab", _i32), ("eps", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("emb", _p),
                ("wq", _p * MAXL), ("wk", _p * MAXL), ("wv", _p * MAXL), ("wo", _p * MAXL),
                ("wg", _p * MAXL), ("wu", _p * MAXL), ("wd", _p * MAXL), ("w_lm", _p),
                ("rope_cos", _p), ("rope_sin", _p), ("rope_rows", _i32)]


class TinyAttnArgs(ctypes.Structure):
    _fields_ = [("mode", _i32), ("cap", _i64), ("k", _p * MAXL), ("v", _p * MAXL), ("len", _p),
                ("blk_k", _p * MAXL), ("blk_v", _p * MAXL), ("tcap", _i64), ("tail_pos", _i32),
                ("tail_len", _p), ("pos_base", _p)]


def _setup_lib():
    L = lib()
    if not getattr(L, "_tiny_ready", False):
        L.vc_tiny_rope_table.argtypes = [_i32, _i32, ctypes.c_float, _p, _p]
        L.vc_tiny_rope_table.restype = ctypes.c_int
        L.vc_tiny_workspace_size.argtypes = [ctypes.POINTER(TinyModelArgs), _i32]
        L.vc_tiny_workspace_size.restype = ctypes.c_size_t
        L.vc_tiny_forward.argtypes = [ctypes.POINTER(TinyModelArgs), _i32, _p, _i32, ctypes.POINTER(TinyAttnArgs),
                                      _p, _p, ctypes.c_size_t, _p]
        L.vc_tiny_forward.restype = ctypes.c_int
        L.vc_gather_rows.argtypes = [_i32, _i32, _i32, _p, _p, _p, _i64, _p, _p, _i64, _p, _p]
        L.vc_gather_rows.restype = ctypes.c_int
        L.vc_evict_kept_count.argtypes = [_i32, _i32, _i32, _i32]
        L.vc_evict_kept_count.restype = _i32
        L.vc_gather_evict.argtypes = [_i32, _i32, _p, _i32, _i32, _i32, _p, _p, _i64, _p, _p, _i64, _p, _p]
        L.vc_gather_evict.restype = ctypes.c_int
        L._tiny_ready = True
    return L


def _ceil64(x):
    return (x + 63) // 64 * 64


def evict_kept_count(T, sinks, recent, stride):
    """Positions the eviction rule keeps of T committed tokens (``vc_evict_kept_count``)."""
    n = _setup_lib().vc_evict_kept_count(T, sinks, recent, stride)
    if n < 0:
        raise ValueError("bad eviction rule")
    return n


def gather_evict(src_len, sinks, recent, stride, src_k, src_v, dst_k, dst_v, dst_len, stream=None):
    """Compacted cache of the eviction rule at T = ``src_len[0]`` (device), per
    KV head (``vc_gather_evict``): ``src_k [Hkv][cap][D]``, ``src_v
    [Hkv][D][cap]``, ``dst_k [Hkv][ccap][D]``, ``dst_v [Hkv][ccap/32][D][32]``
    fp32, ``dst_len`` int32 ``[Hkv]``."""
    Hkv, cap, D = src_k.shape[-3:]
    ccap = dst_k.shape[-2]
    for t, shape in ((src_v, (Hkv, D, cap)), (dst_k, (Hkv, ccap, D)), (dst_v, (Hkv, ccap // 32, D, 32))):
        if tuple(t.shape[-len(shape):]) != shape or t.numel() != int(np.prod(shape)) or t.dtype != torch.float32:
            raise ValueError(f"expected an fp32 tensor of shape {list(shape)}, got {list(t.shape)}")
    if dst_len.numel() < Hkv or src_len.numel() < 1:
        raise ValueError("src_len needs 1 entry and dst_len Hkv entries")
    for t in (src_k, src_v, dst_k, dst_v, src_len, dst_len):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("all tensors must be contiguous GPU tensors")
    _check(_setup_lib().vc_gather_evict(Hkv, D, src_len.data_ptr(), sinks, recent, stride, src_k.data_ptr(),
                                        src_v.data_ptr(), cap, dst_k.data_ptr(), dst_v.data_ptr(), ccap,
                                        dst_len.data_ptr(), _stream(stream)))


class TinyDecoder:
    """Weights on the GPU plus the model descriptor (``vc_tiny_model``)."""

    def __init__(self, arrays, n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=1024,
                 vocab=512, eps=1e-5, rope_base=10000.0, max_pos=4096):
        L = _setup_lib()
        dev = "cuda"
        self.spec = dict(n_layers=n_layers, d_model=d_model, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                         head_dim=head_dim, ffn=ffn, vocab=vocab)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        self._keep = {k: t(v) for k, v in arrays.items()}
        cos = np.empty((max_pos, head_dim // 2), np.float32)
        sin = np.empty((max_pos, head_dim // 2), np.float32)
        _check(L.vc_tiny_rope_table(max_pos, head_dim, rope_base, cos.ctypes.data, sin.ctypes.data))
        self._keep["rope_cos"], self._keep["rope_sin"] = t(cos), t(sin)
        m = TinyModelArgs()
        m.n_layers, m.d_model, m.n_q_heads, m.n_kv_heads = n_layers, d_model, n_q_heads, n_kv_heads
        m.head_dim, m.ffn, m.vocab, m.eps, m.rope_base = head_dim, ffn, vocab, eps, rope_base
        m.emb = self._keep["emb"].data_ptr()
        for l in range(n_layers):
            for name in ("wq", "wk", "wv", "wo", "wg", "wu", "wd"):
                getattr(m, name)[l] = self._keep[f"l{l}.{name}"].data_ptr()
        m.w_lm = self._keep["w_lm"].data_ptr()
        m.rope_cos, m.rope_sin = self._keep["rope_cos"].data_ptr(), self._keep["rope_sin"].data_ptr()
        m.rope_rows = max_pos
        self.m = m
        self.L = L

    def workspace(self, R):
        n = self.L.vc_tiny_workspace_size(ctypes.byref(self.m), R)
        return torch.empty(n, dtype=torch.uint8, device="cuda")

    def forward(self, R, tokens, pos0, attn, logits, ws, stream=None):
        _check(self.L.vc_tiny_forward(ctypes.byref(self.m), R, tokens.data_ptr(), pos0, ctypes.byref(attn),
                                      logits.data_ptr(), ws.data_ptr(), ws.numel(), _stream(stream)))


class TinyVeriCache:
    """GPU VeriCache loop (batch 1) over a :class:`TinyDecoder`.

    ``compressor``: ``"evict"`` (sinks/recent/stride rule) or ``"identity"``
    (the compressed cache is the full cache).  ``graph``: capture the round
    into a HIP graph after the prefill and replay it (else enqueue each round).
    """

    def __init__(self, model, max_tokens, k, compressor="evict", sinks=4, recent=128, stride=8, graph=True):
        sp = model.spec
        self.model, self.k = model, k
        self.Hkv, self.D, self.V = sp["n_kv_heads"], sp["head_dim"], sp["vocab"]
        self.nl = sp["n_layers"]
        self.rule = (0, 0, 1) if compressor == "identity" else (sinks, recent, stride)
        self.compressor = compressor
        self.use_graph = graph
        self.graph = None
        dev = "cuda"
        self.cap = _ceil64(max_tokens + k + 1)
        z = lambda *s: torch.zeros(s, dtype=torch.float32, device=dev)
        Hkv, D = self.Hkv, self.D
        self.full_k = [z(1, Hkv, self.cap, D) for _ in range(self.nl)]
        self.full_v = [z(1, Hkv, D, self.cap) for _ in range(self.nl)]
        # committed length per layer (each commit advances its own layer's
        # length); layer 0's [0][0] is the verify context length and the base
        # of every position of the round
        self.full_len = [torch.zeros((1, Hkv), dtype=torch.int32, device=dev) for _ in range(self.nl)]
        self.ccap = _ceil64(evict_kept_count(self.cap, *self.rule))
        self.comp_k = [z(1, Hkv, self.ccap, D) for _ in range(self.nl)]
        self.comp_v = [z(1, Hkv, self.ccap // 32, D, 32) for _ in range(self.nl)]   # 32-token blocks
        self.comp_len = torch.zeros((1, Hkv), dtype=torch.int32, device=dev)
        self.tail_k = [z(1, Hkv, max(k, 1), D) for _ in range(self.nl)]
        self.tail_v = [z(1, Hkv, D, max(k, 1)) for _ in range(self.nl)]
        self.tail_len = torch.zeros(1, dtype=torch.int32, device=dev)
        self.blk_k = [z(1, Hkv, k + 1, D) for _ in range(self.nl)]
        self.blk_v = [z(1, Hkv, D, k + 1) for _ in range(self.nl)]
        # the round's record: inputs x0, d_1..d_k | predictions [k+1] |
        # accept length | emitted tokens [k+1] | emitted count
        M = k + 1
        self.rec = torch.zeros(3 * M + 2, dtype=torch.int32, device=dev)
        self.tokens = self.rec[0:M]
        self.am = self.rec[M:2 * M]
        self.acc = self.rec[2 * M:2 * M + 1]
        self.toks = self.rec[2 * M + 1:3 * M + 1]
        self.nout = self.rec[3 * M + 1:3 * M + 2]
        self.logits_d = z(1, self.V)
        self.logits_v = z(M, self.V)
        self.ws1 = model.workspace(1)
        self.wsk = model.workspace(M)
        self._va = self._verify_attn(self.blk_k, self.blk_v, self.full_len[0])
        self._da = [self._draft_attn(i) for i in range(k)]

    def _verify_attn(self, blk_k, blk_v, pos_base=None):
        a = TinyAttnArgs()
        a.mode, a.cap = 0, self.cap
        for l in range(self.nl):
            a.k[l], a.v[l] = self.full_k[l].data_ptr(), self.full_v[l].data_ptr()
            a.blk_k[l], a.blk_v[l] = blk_k[l].data_ptr(), blk_v[l].data_ptr()
        a.len = self.full_len[0].data_ptr()
        a.pos_base = None if pos_base is None else pos_base.data_ptr()
        return a

    def _draft_attn(self, i):
        a = TinyAttnArgs()
        a.mode, a.cap, a.tcap, a.tail_pos = 1, self.ccap, max(self.k, 1), i
        for l in range(self.nl):
            a.k[l], a.v[l] = self.comp_k[l].data_ptr(), self.comp_v[l].data_ptr()
            a.blk_k[l], a.blk_v[l] = self.tail_k[l].data_ptr(), self.tail_v[l].data_ptr()
        a.len = self.comp_len.data_ptr()
        a.tail_len = self.tail_len.data_ptr()
        a.pos_base = self.full_len[0].data_ptr()
        return a

    def prefill(self, prompt):
        """Causal prefill of the prompt; returns the first generated token."""
        P = len(prompt)
        dev = "cuda"
        z = lambda *s: torch.zeros(s, dtype=torch.float32, device=dev)
        bk = [z(1, self.Hkv, P, self.D) for _ in range(self.nl)]
        bv = [z(1, self.Hkv, self.D, P) for _ in range(self.nl)]
        toks = torch.from_numpy(np.asarray(prompt, dtype=np.int32)).to(dev)
        logits = z(P, self.V)
        for fl in self.full_len:
            fl.zero_()
        self.model.forward(P, toks, 0, self._verify_attn(bk, bv), logits, self.model.workspace(P))
        n_all = torch.full((1,), P, dtype=torch.int32, device=dev)
        for l in range(self.nl):
            commit_rows(bk[l], bv[l], n_all, self.full_k[l], self.full_v[l], self.full_len[l])
        argmax(logits[P - 1:P].contiguous(), out=self.tokens[0:1])
        self.T = P
        first = int(self.tokens[0].item())
        if self.use_graph and self.graph is None:
            # capture records the round without running it; every round replays it
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._enqueue_round()
            self.graph = g
        return first

    def _enqueue_round(self):
        """One round on the current stream, with no host data: the kept set,
        the positions and the next input all come from device state."""
        k, M, L, s = self.k, self.k + 1, self.model.L, _stream(None)
        sinks, recent, stride = self.rule
        for l in range(self.nl):
            _check(L.vc_gather_evict(self.Hkv, self.D, self.full_len[0].data_ptr(), sinks, recent, stride,
                                     self.full_k[l].data_ptr(), self.full_v[l].data_ptr(), self.cap,
                                     self.comp_k[l].data_ptr(), self.comp_v[l].data_ptr(), self.ccap,
                                     self.comp_len.data_ptr(), s))
        for i in range(k):
            self.model.forward(1, self.tokens[i:i + 1], i, self._da[i], self.logits_d, self.ws1)
            argmax(self.logits_d, out=self.tokens[i + 1:i + 2])
        self.model.forward(M, self.tokens, 0, self._va, self.logits_v, self.wsk)
        accept(self.logits_v.view(1, M, self.V), self.tokens[1:].view(1, k), argmax=self.am, accept_len=self.acc,
               out_tokens=self.toks, n_out=self.nout)
        for l in range(self.nl):
            commit_rows(self.blk_k[l], self.blk_v[l], self.nout, self.full_k[l], self.full_v[l], self.full_len[l])
        next_input(self.toks.view(1, M), self.nout, self.tokens[0:1])

    def round(self):
        """One draft / verify / accept / commit round.  Returns
        ``(drafts, predictions, n, emitted)`` (host lists)."""
        k = self.k
        if self.T + k + 1 > self.cap or self.T + k + 1 > self.model.m.rope_rows:
            raise ValueError("the round would exceed the cache capacity or the RoPE table")
        if self.use_graph:
            self.graph.replay()
        else:
            self._enqueue_round()
        r = self.rec.cpu().numpy()         # the one host read per round
        M = k + 1
        n = int(r[2 * M])
        res = (r[1:M].tolist(), r[M:2 * M].tolist(), n, r[2 * M + 1:2 * M + 2 + n].tolist())
        self.T += n + 1
        return res

    def generate(self, prompt, n_new):
        first = self.prefill(prompt)
        out, rounds = [first], []
        while len(out) < n_new:
            r = self.round()
            rounds.append(r)
            out.extend(r[3])
        return out[:n_new], rounds
