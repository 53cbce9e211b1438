"""Tiny random-weight decoder, full-KV greedy decoding and the VeriCache loop.

Test infrastructure only (see :mod:`oracle`).

The pages fix no model.  The decoder is the plainest Llama-family reading
of a 2-layer, d_model 256, 4 query / 2 KV heads, head_dim 64, vocab 512,
RMSNorm + RoPE model (the summaries evaluate Llama/Mistral/Qwen models,
"Riepilogo Tecnico: VeriCache", section "Risultati Sperimentali"):

* pre-norm residual blocks, no biases, RMSNorm ``x / sqrt(mean(x^2) + 1e-5)``
  with unit gain;
* attention: ``q = a Wq``, ``k = a Wk``, ``v = a Wv``, RoPE on q and k
  (rotate-half pairs ``(i, i + D/2)``, ``theta_i = 10000^(-2i/D)``), GQA with
  query head h reading KV head ``h // 2``, scale ``1/sqrt(D)``, ``h += o Wo``;
* MLP: ``h += (SiLU(m Wg) * (m Wu)) Wd`` with ``m = RMSNorm(h)``, width 1024;
* ``logits = RMSNorm(h) W_lm`` (untied).

Every token is computed by one routine (:func:`token_step`) whose result
depends only on the token, its position and the key/value rows it attends to,
in a fixed order.  A causal verify block is therefore, bit for bit, the same as
that many single-token greedy steps -- the property the loop's losslessness
rests on ("Riepilogo Tecnico: VeriCache", sections "Algoritmo Principale" and
"Risultati Sperimentali").

Loop ("Algoritmo Principale"): draft k tokens with the compressed cache plus a
draft tail, verify ``[x0, d_1..d_k]`` in one full-cache pass, accept up to
the first mismatch and emit the full-cache prediction after it (the bonus
token when all k match); commit the verified K/V rows of the accepted block
prefix, discard the draft tail, continue from the last emitted token.

Parity: the loop output is pinned to full-KV greedy decoding (identical
tokens), the identity compressor to full acceptance with the bonus every
round, k = 0 to plain greedy steps, RoPE to the complex-rotation closed form
and RMSNorm to unit RMS.  The absolute token values of this model are
"parity unpinned" beyond those properties: the model is defined by this spec.
"""
from dataclasses import dataclass, field

import numpy as np

from .accept import accept, greedy_argmax
from .attention import attend


@dataclass(frozen=True)
class TinySpec:
    n_layers: int = 2
    d_model: int = 256
    n_q_heads: int = 4
    n_kv_heads: int = 2
    head_dim: int = 64
    ffn: int = 1024
    vocab: int = 512
    eps: float = 1e-5
    rope_base: float = 10000.0


def rmsnorm(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x) + eps)


def rope(x, pos, base):
    """Rotate-half RoPE on ``x [H][D]`` at absolute position ``pos``."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    theta = base ** (-2.0 * np.arange(half) / D)
    ang = pos * theta
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


@dataclass
class TinyWeights:
    """float64 copies of the model parameters (row-vector convention x @ W)."""
    spec: TinySpec
    emb: np.ndarray                      # [V][d]
    layers: list = field(default_factory=list)   # dicts wq wk wv wo wg wu wd
    w_lm: np.ndarray = None              # [d][V]

    @classmethod
    def from_arrays(cls, spec, arrays):
        """``arrays``: dict with ``emb``, ``w_lm`` and per-layer keys
        ``l{i}.wq`` ... ``l{i}.wd`` (any float dtype)."""
        f = lambda a: np.asarray(a, dtype=np.float64)
        layers = []
        for i in range(spec.n_layers):
            layers.append({n: f(arrays[f"l{i}.{n}"]) for n in
                           ("wq", "wk", "wv", "wo", "wg", "wu", "wd")})
        return cls(spec, f(arrays["emb"]), layers, f(arrays["w_lm"]))


def token_step(W, token, pos, layer_ctx):
    """One token through the model.

    ``layer_ctx[l] = (K [Hkv][T][D], V [Hkv][T][D], bias [T] or None)`` are the
    rows this token attends to besides itself (its own row is appended last,
    bias 0).  Returns ``(logits [V], [(k [Hkv][D], v [Hkv][D]) per layer])``
    with k already rotated.
    """
    sp = W.spec
    Hq, Hkv, D = sp.n_q_heads, sp.n_kv_heads, sp.head_dim
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D)
    h = W.emb[token].copy()
    new_kv = []
    for l, P in enumerate(W.layers):
        a = rmsnorm(h, sp.eps)
        q = rope((a @ P["wq"]).reshape(Hq, D), pos, sp.rope_base)
        k = rope((a @ P["wk"]).reshape(Hkv, D), pos, sp.rope_base)
        v = (a @ P["wv"]).reshape(Hkv, D)
        Kc, Vc, bc = layer_ctx[l]
        o = np.empty((Hq, D))
        for hq in range(Hq):
            g = hq // G
            keys = np.concatenate([Kc[g], k[g][None]])
            vals = np.concatenate([Vc[g], v[g][None]])
            bias = None if bc is None else np.concatenate([bc, [0.0]])
            o[hq], _ = attend(q[hq], keys, vals, scale, bias)
        h = h + o.reshape(-1) @ P["wo"]
        m = rmsnorm(h, sp.eps)
        h = h + (silu(m @ P["wg"]) * (m @ P["wu"])) @ P["wd"]
        new_kv.append((k, v))
    logits = rmsnorm(h, sp.eps) @ W.w_lm
    return logits, new_kv


class KVCache:
    """Per-layer full cache ``K/V [Hkv][T][D]`` (rows at absolute positions)."""

    def __init__(self, spec):
        self.spec = spec
        z = np.zeros((spec.n_kv_heads, 0, spec.head_dim))
        self.k = [z.copy() for _ in range(spec.n_layers)]
        self.v = [z.copy() for _ in range(spec.n_layers)]

    @property
    def length(self):
        return self.k[0].shape[1]

    def append(self, kv_rows):
        """``kv_rows``: per layer ``(k [Hkv][D], v [Hkv][D])`` of one token."""
        for l, (k, v) in enumerate(kv_rows):
            self.k[l] = np.concatenate([self.k[l], k[:, None, :]], axis=1)
            self.v[l] = np.concatenate([self.v[l], v[:, None, :]], axis=1)

    def ctx(self, positions=None, extra=None):
        """Context rows per layer: cached rows (all, or ``positions``) then the
        ``extra`` per-layer row lists (draft tail or earlier block rows)."""
        out = []
        for l in range(self.spec.n_layers):
            K, V = self.k[l], self.v[l]
            if positions is not None:
                K, V = K[:, positions], V[:, positions]
            if extra:
                K = np.concatenate([K] + [e[l][0][:, None] for e in extra], axis=1)
                V = np.concatenate([V] + [e[l][1][:, None] for e in extra], axis=1)
            out.append((K, V, None))
        return out


def prefill(W, prompt):
    """Run the prompt token by token with the full cache; returns the cache
    (post-RoPE rows for every prompt position) and the last row's logits."""
    cache = KVCache(W.spec)
    logits = None
    for p, tok in enumerate(prompt):
        logits, kv = token_step(W, int(tok), p, cache.ctx())
        cache.append(kv)
    return cache, logits


def greedy_decode(W, prompt, n_new):
    """Full-KV greedy decoding: the lossless reference.  Returns the first
    ``n_new`` generated token ids (the first comes from the prompt's last
    logits)."""
    cache, logits = prefill(W, prompt)
    out = [greedy_argmax(logits)]
    while len(out) < n_new:
        logits, kv = token_step(W, out[-1], cache.length, cache.ctx())
        cache.append(kv)
        out.append(greedy_argmax(logits))
    return out


def kept_positions(T, sinks=4, recent=128, stride=8):
    """Eviction compressor of the tiny loop: attention sinks, the most recent
    tokens, and older tokens at absolute positions divisible by ``stride``
    (sinks and recent tokens are preserved as in "Riassunto Tecnico:
    CentroidKV", "Componenti Chiave", item 2).  Ascending positions < T."""
    keep = set(range(min(sinks, T)))
    keep |= set(range(max(T - recent, 0), T))
    keep |= {p for p in range(sinks, max(T - recent, sinks)) if p % stride == 0}
    return np.array(sorted(keep), dtype=np.int64)


def all_positions(T):
    """Identity compressor: keeps every token."""
    return np.arange(T, dtype=np.int64)


@dataclass
class RoundRecord:
    T: int              # committed length before the round (position of x0)
    x0: int
    drafts: list
    predictions: list   # y_1 .. y_{k+1}
    n: int              # accepted drafts
    emitted: list       # d_1..d_n, y_{n+1}
    draft_margin: float = np.inf    # min top-2 logit gap over the draft steps
    verify_margin: float = np.inf   # min top-2 logit gap over the verify rows


def _margin(logits):
    top = np.sort(np.asarray(logits, dtype=np.float64))[-2:]
    return float(top[1] - top[0])


def vericache_decode(W, prompt, n_new, k, compressor=kept_positions):
    """The draft-then-verify loop run step by step.

    Returns ``(tokens, rounds)``: the first ``n_new`` emitted tokens and one
    :class:`RoundRecord` per round.  ``compressor(T)`` gives the kept
    positions of the compressed cache for a committed length ``T``.
    """
    cache, logits = prefill(W, prompt)
    T = cache.length
    x0 = greedy_argmax(logits)
    emitted = [x0]
    rounds = []
    while len(emitted) < n_new:
        kept = compressor(T)
        # Draft: k single-token steps over the compressed cache + draft tail.
        tail, drafts, dmargin = [], [], np.inf
        tok = x0
        for i in range(k):
            lg, kv = token_step(W, tok, T + i, cache.ctx(kept, tail))
            tail.append(kv)
            dmargin = min(dmargin, _margin(lg))
            tok = greedy_argmax(lg)
            drafts.append(tok)
        # Verify: block rows x0, d_1..d_k against the full cache, causal.
        block = [x0] + drafts
        blk, vlogits = [], []
        for i, tok in enumerate(block):
            lg, kv = token_step(W, tok, T + i, cache.ctx(None, blk))
            blk.append(kv)
            vlogits.append(lg)
        y, n, out = accept(np.array(vlogits), drafts)
        rounds.append(RoundRecord(T, x0, drafts, y, n, out, dmargin,
                                  min(_margin(r) for r in vlogits)))
        # Commit the verified rows of x0, d_1..d_n; drop the draft tail.
        for kv in blk[:n + 1]:
            cache.append(kv)
        T += n + 1
        emitted.extend(out)
        x0 = out[-1]
    return emitted[:n_new], rounds
