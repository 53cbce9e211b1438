"""The draft-then-verify loop on the GPU for the small fp32 decoder of
``include/vc_tiny.h``.

"Riepilogo Tecnico: VeriCache", section "Algoritmo Principale": the model
drafts k tokens over its compressed cache, one forward pass over the full
cache verifies them, tokens are accepted up to the first mismatch (plus the
bonus token on a full match) and decoding resumes from the last accepted
token.  Every step runs in libvc kernels: forward passes (vc_tiny_forward),
drafter argmax (vc_argmax), acceptance (vc_accept), commit of the verified
rows (vc_commit_rows) and the compacted cache (vc_gather_rows).  The host
reads the acceptance result once per round.

The eviction compressor keeps the attention sinks, the most recent tokens
and every ``stride``-th older token (sinks and recent tokens are preserved as
in "Riassunto Tecnico: CentroidKV", "Componenti Chiave", item 2); its kept
positions are a pure function of the committed length.
"""
import ctypes

import numpy as np
import torch

from . import (VC_BF16, VC_FP32, _check, _p, _i32, _i64, _stream, accept, argmax, commit_rows, lib)

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
                ("tail_len", _p)]


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
        L._tiny_ready = True
    return L


def _ceil64(x):
    return (x + 63) // 64 * 64


def kept_positions(T, sinks=4, recent=128, stride=8):
    """Eviction rule: sinks, the last ``recent`` tokens, and positions
    divisible by ``stride`` in between (ascending)."""
    if T <= sinks + recent:
        return np.arange(T, dtype=np.int32)
    mid = np.arange(sinks, T - recent)
    mid = mid[mid % stride == 0]
    return np.concatenate([np.arange(sinks), mid, np.arange(T - recent, T)]).astype(np.int32)


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
    (the compressed cache is the full cache).
    """

    def __init__(self, model, max_tokens, k, compressor="evict", sinks=4, recent=128, stride=8):
        sp = model.spec
        self.model, self.k = model, k
        self.Hkv, self.D, self.V = sp["n_kv_heads"], sp["head_dim"], sp["vocab"]
        self.nl = sp["n_layers"]
        self.rule = (sinks, recent, stride)
        self.compressor = compressor
        dev = "cuda"
        self.cap = _ceil64(max_tokens + k + 1)
        z = lambda *s: torch.zeros(s, dtype=torch.float32, device=dev)
        Hkv, D = self.Hkv, self.D
        self.full_k = [z(1, Hkv, self.cap, D) for _ in range(self.nl)]
        self.full_v = [z(1, Hkv, D, self.cap) for _ in range(self.nl)]
        # committed length per layer (each commit advances its own layer's
        # length); layer 0's [0][0] doubles as the verify context length
        self.full_len = [torch.zeros((1, Hkv), dtype=torch.int32, device=dev) for _ in range(self.nl)]
        self.ccap = self.cap if compressor == "identity" else _ceil64(sinks + recent + max_tokens // stride + 1)
        self.comp_k = [z(1, Hkv, self.ccap, D) for _ in range(self.nl)]
        self.comp_v = [z(1, Hkv, self.ccap // 32, D, 32) for _ in range(self.nl)]   # 32-token blocks
        self.comp_len = torch.zeros((1, Hkv), dtype=torch.int32, device=dev)
        self.tail_k = [z(1, Hkv, max(k, 1), D) for _ in range(self.nl)]
        self.tail_v = [z(1, Hkv, D, max(k, 1)) for _ in range(self.nl)]
        self.tail_len = torch.zeros(1, dtype=torch.int32, device=dev)
        self.blk_k = [z(1, Hkv, k + 1, D) for _ in range(self.nl)]
        self.blk_v = [z(1, Hkv, D, k + 1) for _ in range(self.nl)]
        self.tokens = torch.zeros(k + 1, dtype=torch.int32, device=dev)
        self.logits_d = z(1, self.V)
        self.logits_v = z(k + 1, self.V)
        self.ws1 = model.workspace(1)
        self.wsk = model.workspace(k + 1)
        self.idx = torch.zeros(self.ccap, dtype=torch.int32, device=dev)
        self.n_out = torch.zeros(1, dtype=torch.int32, device=dev)

    def _verify_attn(self, blk_k, blk_v):
        a = TinyAttnArgs()
        a.mode, a.cap = 0, self.cap
        for l in range(self.nl):
            a.k[l], a.v[l] = self.full_k[l].data_ptr(), self.full_v[l].data_ptr()
            a.blk_k[l], a.blk_v[l] = blk_k[l].data_ptr(), blk_v[l].data_ptr()
        a.len = self.full_len[0].data_ptr()
        return a

    def _draft_attn(self, i):
        a = TinyAttnArgs()
        a.mode, a.cap, a.tcap, a.tail_pos = 1, self.ccap, max(self.k, 1), i
        for l in range(self.nl):
            a.k[l], a.v[l] = self.comp_k[l].data_ptr(), self.comp_v[l].data_ptr()
            a.blk_k[l], a.blk_v[l] = self.tail_k[l].data_ptr(), self.tail_v[l].data_ptr()
        a.len = self.comp_len.data_ptr()
        a.tail_len = self.tail_len.data_ptr()
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
        first = argmax(logits[P - 1:P].contiguous())
        self.T = P
        self.tokens[0:1].copy_(first)
        return int(first.item())

    def _compress(self):
        if self.compressor == "identity":
            kept = np.arange(self.T, dtype=np.int32)
        else:
            kept = kept_positions(self.T, *self.rule)
        n = len(kept)
        self.idx[:n].copy_(torch.from_numpy(kept))
        for l in range(self.nl):
            _check(self.model.L.vc_gather_rows(self.Hkv, self.D, n, self.idx.data_ptr(), self.full_k[l].data_ptr(),
                                               self.full_v[l].data_ptr(), self.cap, self.comp_k[l].data_ptr(),
                                               self.comp_v[l].data_ptr(), self.ccap, self.comp_len.data_ptr(),
                                               _stream(None)))

    def round(self):
        """One draft / verify / accept / commit round.  Returns
        ``(drafts, predictions, n, emitted)`` (host lists)."""
        k, T = self.k, self.T
        self._compress()
        for i in range(k):
            self.model.forward(1, self.tokens[i:i + 1], T + i, self._draft_attn(i), self.logits_d, self.ws1)
            argmax(self.logits_d, out=self.tokens[i + 1:i + 2])
        self.model.forward(k + 1, self.tokens, T, self._verify_attn(self.blk_k, self.blk_v), self.logits_v, self.wsk)
        drafts = self.tokens[1:].contiguous().view(1, k)
        am, n_acc, toks, n_out = accept(self.logits_v.view(1, k + 1, self.V), drafts)
        for l in range(self.nl):
            commit_rows(self.blk_k[l], self.blk_v[l], n_out, self.full_k[l], self.full_v[l], self.full_len[l])
        n = int(n_acc.item())                         # the one host sync per round
        emitted = toks[0, :n + 1].cpu().tolist()
        res = (drafts[0].cpu().tolist(), am[0].cpu().tolist(), n, emitted)
        self.T += n + 1
        self.tokens[0:1].copy_(toks[0, n:n + 1])
        return res

    def generate(self, prompt, n_new):
        first = self.prefill(prompt)
        out, rounds = [first], []
        while len(out) < n_new:
            r = self.round()
            rounds.append(r)
            out.extend(r[3])
        return out[:n_new], rounds
