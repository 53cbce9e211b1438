"""Seeded input generators (numpy PCG64), one stream per tensor slice.

Every tensor slice is drawn from ``PCG64(SeedSequence([cfg_seed, tensor_id,
*index]))`` so any slice can be regenerated alone.  bfloat16 tensors are
produced as uint16 bit patterns by round-to-nearest-even from float32; int4
tensors as packed bytes (eight codes per little-endian 32-bit word, the even
codes of the word in its low half) with binary16 scales/zeros as uint16 bit
patterns.

Workload recipes (shapes follow the configurations the library is measured
on; the value distributions are stated per function).
"""
import numpy as np

__all__ = [
    "rng", "f32_to_bf16_bits", "normal_bf16", "normal_f32", "tiny_weights",
    "tiny_prompt", "kept_random", "degrees", "int4_grid", "pack_codes",
    "planted_accept", "planted_logits", "csm_planted", "lm_planted", "pack_int4_blocks", "TINY_WEIGHT_ORDER", "TID", "torch_normal",
    "torch_randint",
]

# Tensor ids used in SeedSequence keys.
TID = dict(q=1, k=2, v=3, tail_k=4, tail_v=5, blk_k=6, blk_v=7, kept=8,
           degree=9, kcode=10, vcode=11, kscale=12, vscale=13, logits=14,
           accept=15, hidden=16, lm=17, csm=18, lm_head=19)


def rng(cfg_seed, tensor_id, *index):
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(cfg_seed), int(tensor_id)] + [int(i) for i in index])))


def f32_to_bf16_bits(x):
    """float32 values -> uint16 bfloat16 bit patterns, round to nearest even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def normal_f32(shape, cfg_seed, tensor_id, std=1.0, slice_dims=2):
    """float32 N(0, std^2) of ``shape``; the first ``slice_dims`` axes index
    independent streams (e.g. (b, kv head))."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    lead = shape[:slice_dims]
    for idx in np.ndindex(*lead):
        g = rng(cfg_seed, tensor_id, *idx)
        out[idx] = (g.standard_normal(shape[slice_dims:], dtype=np.float32) * np.float32(std))
    return out


def normal_bf16(shape, cfg_seed, tensor_id, std=1.0, slice_dims=2):
    """bf16 bit patterns of :func:`normal_f32` draws."""
    return f32_to_bf16_bits(normal_f32(shape, cfg_seed, tensor_id, std, slice_dims))


# --------------------------------------------------------------------------
# Tiny decoder (2 layers, d_model 256, 4 q heads / 2 KV heads, head_dim 64,
# MLP width 1024, vocab 512): float32 weights N(0, 0.02^2) drawn in this
# order from one PCG64(seed) stream.
TINY_WEIGHT_ORDER = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def tiny_weights(seed=0, n_layers=2, d_model=256, n_q_heads=4, n_kv_heads=2,
                 head_dim=64, ffn=1024, vocab=512, std=0.02):
    g = np.random.Generator(np.random.PCG64(seed))
    draw = lambda *s: (g.standard_normal(s, dtype=np.float64) * std).astype(np.float32)
    w = {"emb": draw(vocab, d_model)}
    shapes = {"wq": (d_model, n_q_heads * head_dim), "wk": (d_model, n_kv_heads * head_dim),
              "wv": (d_model, n_kv_heads * head_dim), "wo": (n_q_heads * head_dim, d_model),
              "wg": (d_model, ffn), "wu": (d_model, ffn), "wd": (ffn, d_model)}
    for l in range(n_layers):
        for name in TINY_WEIGHT_ORDER:
            w[f"l{l}.{name}"] = draw(*shapes[name])
    w["w_lm"] = draw(d_model, vocab)
    return w


def tiny_prompt(seed=1, length=1024, vocab=512):
    return np.random.Generator(np.random.PCG64(seed)).integers(0, vocab, length).astype(np.int32)


# --------------------------------------------------------------------------
# Compressed-cache metadata (variant A: kept token subset with degrees).
def kept_random(n_ctx, n_keep, cfg_seed, b, sinks=4, recent=1024):
    """Ascending kept positions: sinks, the last ``recent`` tokens, and the
    rest drawn uniformly without replacement from the range between them."""
    rest = n_keep - sinks - recent
    if rest < 0 or rest > n_ctx - sinks - recent:
        raise ValueError("kept budget does not fit the context")
    g = rng(cfg_seed, TID["kept"], b)
    mid = g.choice(np.arange(sinks, n_ctx - recent), size=rest, replace=False)
    return np.sort(np.concatenate([np.arange(sinks), mid,
                                   np.arange(n_ctx - recent, n_ctx)])).astype(np.int32)


def degrees(shape, cfg_seed, lo=1, hi=4):
    """float32 merge degrees n_t drawn uniformly from {lo..hi}; the first axis
    (batch) indexes independent streams."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    for b in range(shape[0]):
        out[b] = rng(cfg_seed, TID["degree"], b).integers(lo, hi + 1, shape[1:]).astype(np.float32)
    return out


# --------------------------------------------------------------------------
# Int4 compressed cache (variant B), drawn directly on the quantization grid.
def pack_codes(codes):
    """int codes 0..15 ``[..., N]`` (N a multiple of 8) -> uint8 ``[..., N/2]``.

    Each group of eight consecutive codes c0..c7 becomes one little-endian
    32-bit word with c_2j in bits 4j..4j+3 and c_2j+1 in bits 16+4j..16+4j+3.
    """
    c = np.asarray(codes).astype(np.uint32)
    n = c.shape[-1]
    assert n % 8 == 0
    c = c.reshape(c.shape[:-1] + (n // 8, 8))
    w = np.zeros(c.shape[:-1], np.uint32)
    for j in range(4):
        w |= c[..., 2 * j] << np.uint32(4 * j)
        w |= c[..., 2 * j + 1] << np.uint32(16 + 4 * j)
    return np.ascontiguousarray(w.astype("<u4")).view(np.uint8).reshape(c.shape[:-2] + (n // 2,))


def pack_int4_blocks(k_codes, v_codes, k_scale, k_zero, v_scale, v_zero):
    """The six int4 arrays of :func:`int4_grid` (library layouts) interleaved
    per 32-token block: uint8 ``[B][Hkv][cap/32][5120]`` holding K codes
    (2048 B), V codes (2048 B), K scales, K zeros, V scales, V zeros (256 B
    each, little-endian binary16).  Storage layout only."""
    k_codes, v_codes = np.asarray(k_codes), np.asarray(v_codes)
    B, Hkv, cap = k_codes.shape[:3]
    nb = cap // 32
    parts = [k_codes.reshape(B, Hkv, nb, 2048), v_codes.reshape(B, Hkv, nb, 2048)]
    for a in (k_scale, k_zero, v_scale, v_zero):
        parts.append(np.ascontiguousarray(np.asarray(a).astype("<u2")).view(np.uint8).reshape(B, Hkv, nb, 256))
    return np.ascontiguousarray(np.concatenate(parts, axis=-1))


def int4_grid(B, Hkv, cap, D, cfg_seed, smin=0.3, smax=0.5):
    """Codes uniform on 0..15 and binary16 scales ``s ~ U[smin, smax]``,
    zeros ``z = -7.5 s`` (so reconstructions span about +-3.75).

    Library layouts (uint8 codes, uint16 binary16 bits), all in 32-token
    blocks:
      ``k_codes [B][Hkv][cap][D/2]`` (a token's codes in channel order, packed
      as :func:`pack_codes` does),
      ``k_scale/k_zero [B][Hkv][cap/32][D]``,
      ``v_codes [B][Hkv][cap/32][D][16]`` (per block, channel d's 32 codes in
      token order, packed as :func:`pack_codes` does),
      ``v_scale/v_zero [B][Hkv][cap/32][D/32][32]``.
    Also the token-major forms for the oracle side: unpacked codes
    ``k_c/v_c [B][Hkv][cap][D]`` and ``v_scale_td/v_zero_td [B][Hkv][cap][D/32]``.
    """
    assert cap % 32 == 0 and D % 32 == 0
    nb, ng = cap // 32, D // 32
    res = {"k_c": np.empty((B, Hkv, cap, D), np.uint8), "v_c": np.empty((B, Hkv, cap, D), np.uint8),
           "k_scale": np.empty((B, Hkv, nb, D), np.uint16),
           "k_zero": np.empty((B, Hkv, nb, D), np.uint16),
           "v_scale_td": np.empty((B, Hkv, cap, ng), np.uint16),
           "v_zero_td": np.empty((B, Hkv, cap, ng), np.uint16)}
    for b in range(B):
        for h in range(Hkv):
            res["k_c"][b, h] = rng(cfg_seed, TID["kcode"], b, h).integers(0, 16, (cap, D))
            res["v_c"][b, h] = rng(cfg_seed, TID["vcode"], b, h).integers(0, 16, (cap, D))
            ks = rng(cfg_seed, TID["kscale"], b, h).uniform(smin, smax, (nb, D)).astype(np.float16)
            res["k_scale"][b, h] = ks.view(np.uint16)
            res["k_zero"][b, h] = (ks.astype(np.float32) * np.float32(-7.5)).astype(np.float16).view(np.uint16)
            vs = rng(cfg_seed, TID["vscale"], b, h).uniform(smin, smax, (cap, ng)).astype(np.float16)
            res["v_scale_td"][b, h] = vs.view(np.uint16)
            res["v_zero_td"][b, h] = (vs.astype(np.float32) * np.float32(-7.5)).astype(np.float16).view(np.uint16)
    res["k_codes"] = pack_codes(res["k_c"])
    # [cap][D] -> [cap/32][32][D] -> [cap/32][D][32] -> pack each channel's 32 tokens -> [cap/32][D][16]
    vblk = res["v_c"].reshape(B, Hkv, nb, 32, D).transpose(0, 1, 2, 4, 3)
    res["v_codes"] = pack_codes(np.ascontiguousarray(vblk))
    for key in ("v_scale", "v_zero"):
        td = res[key + "_td"].reshape(B, Hkv, nb, 32, ng).transpose(0, 1, 2, 4, 3)
        res[key] = np.ascontiguousarray(td)
    return res


# --------------------------------------------------------------------------
# Key sets with planted near-duplicates for the chunked clustering round.
def csm_planted(B, Hkv, n, D, n_sink, n_recent, chunk, n_plant, cfg_seed, noise=0.02):
    """float32 ``k, v [B][Hkv][n][D]``, N(0,1), where in every chunk of the
    middle segment ``[n_sink, n - n_recent)`` (cut every ``chunk`` tokens,
    positions counted from the chunk start) ``n_plant(L)`` of the even
    positions are copies of a randomly chosen odd position of the same chunk
    plus ``noise`` times N(0,1) (``L`` = chunk length); several may copy the
    same odd position.  Returns ``(k, v, planted)`` with ``planted`` a list of
    ``(b, h, even position, odd position)``.
    """
    k = np.empty((B, Hkv, n, D), np.float32)
    v = np.empty((B, Hkv, n, D), np.float32)
    planted = []
    for b in range(B):
        for h in range(Hkv):
            g = rng(cfg_seed, TID["csm"], b, h)
            k[b, h] = g.standard_normal((n, D), dtype=np.float32)
            v[b, h] = g.standard_normal((n, D), dtype=np.float32)
            for s in range(n_sink, n - n_recent, chunk):
                L = min(chunk, n - n_recent - s)
                n_even, n_odd = (L + 1) // 2, L // 2
                if n_odd == 0:
                    continue
                for i in g.choice(n_even, size=min(n_plant(L), n_even), replace=False):
                    j = int(g.integers(0, n_odd))
                    k[b, h, s + 2 * i] = k[b, h, s + 2 * j + 1] + noise * g.standard_normal(D, dtype=np.float32)
                    planted.append((b, h, s + 2 * int(i), s + 2 * j + 1))
    return k, v, planted


# --------------------------------------------------------------------------
# Acceptance patterns for workloads without a trained model.
def planted_accept(B, k, vocab, cfg_seed, n_lo, n_hi, force=()):
    """Per request a target sequence ``y_1..y_{k+1}`` and drafts ``d_1..d_k``
    that copy ``y`` for the first ``n`` positions and then differ, with
    ``n ~ U{n_lo..n_hi}``; ``force`` maps request index -> fixed n.

    Returns ``(y [B][k+1], d [B][k], n [B])`` int32.
    """
    y = np.empty((B, k + 1), np.int32)
    d = np.empty((B, k), np.int32)
    n = np.empty(B, np.int32)
    force = dict(force)
    for b in range(B):
        g = rng(cfg_seed, TID["accept"], b)
        n[b] = force.get(b, g.integers(n_lo, n_hi + 1))
        y[b] = g.integers(0, vocab, k + 1)
        d[b] = g.integers(0, vocab, k)
        d[b, :n[b]] = y[b, :n[b]]
        if n[b] < k and d[b, n[b]] == y[b, n[b]]:
            d[b, n[b]] = (y[b, n[b]] + 1) % vocab
    return y, d, n


def planted_logits(y, vocab, cfg_seed, margin=4.0, ties=0):
    """float32 logits ``[B][M][V]`` N(0,1) whose row argmax is ``y`` (the
    planted entry is the row maximum plus ``margin``).  ``ties > 0`` plants
    that many extra copies of the maximum at higher indices than ``y``."""
    B, M = y.shape
    out = np.empty((B, M, vocab), np.float32)
    for b in range(B):
        g = rng(cfg_seed, TID["logits"], b)
        out[b] = g.standard_normal((M, vocab), dtype=np.float32)
        for j in range(M):
            top = out[b, j].max() + np.float32(margin)
            out[b, j, y[b, j]] = top
            if ties:
                higher = np.arange(y[b, j] + 1, vocab)
                if higher.size:
                    for t in g.choice(higher, size=min(ties, higher.size), replace=False):
                        out[b, j, t] = top
    return out


# --------------------------------------------------------------------------
# Bulk device-side draws for the full-size workloads (torch's seeded Philox
# generator on the GPU; only random numbers, no method arithmetic).
def lm_planted(V, Dm, targets, cfg_seed, scale_exp=-4):
    """A vocab-major LM head ``w [V][Dm]`` of random +-2^scale_exp entries
    (distinct rows, all of the same norm) and hidden rows ``h = w[targets]``,
    as bf16 bit patterns ``(h [R][Dm], w [V][Dm])``."""
    g = rng(cfg_seed, TID["lm_head"], 0)
    while True:
        signs = g.integers(0, 2, size=(V, Dm), dtype=np.int8)
        if len(np.unique(signs, axis=0)) == V:
            break
    w = np.where(signs == 1, 1.0, -1.0).astype(np.float32) * np.float32(2.0 ** scale_exp)
    wb = f32_to_bf16_bits(w)
    return wb[np.asarray(targets).reshape(-1)], wb


def torch_normal(shape, seed, device, dtype, std=1.0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.empty(tuple(shape), dtype=dtype, device=device)
    t.normal_(0.0, std, generator=g)
    return t


def torch_randint(shape, lo, hi, seed, device, dtype):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randint(lo, hi, tuple(shape), generator=g, device=device, dtype=dtype)
