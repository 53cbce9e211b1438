"""Draft and verify attention, written as the softmax definition (fp64).

Test infrastructure only (see :mod:`oracle`).

* Draft step ("Riepilogo Tecnico: VeriCache", section "Algoritmo
  Principale", step 1): the target model decodes one token per call over the
  compressed cache.  The compressed cache is a kept/merged token subset; when
  tokens were merged into centroids, each centroid's degree n_t enters the
  softmax as a logarithmic term ("Riassunto Tecnico: CentroidKV", section
  "Componenti Chiave", item 4 "Aggregazione").  The reading used here (the
  pages give no formula) is the additive score term ``ln n_t`` after the
  ``1/sqrt(D)`` scaling, which makes a centroid of degree n act exactly like n
  identical copies of itself.  A dense "tail" segment (this round's drafted
  tokens, degree 1) follows the compressed segment.
* Verify step (same page and section, step 2): one forward pass over the full
  cache for the whole drafted block; row i of the block sees every context
  key and the block keys 0..i.

Grouped-query attention: query head h reads KV head ``h // (Hq // Hkv)``.

Parity: pinned by tests against the textbook definition computed by another
route (torch ``scaled_dot_product_attention`` on CPU in float64), against the
duplicate-token identity for the log-degree term, and against permutation
invariance of the key set.
"""
import numpy as np


def attend(q, keys, values, scale, bias=None):
    """Softmax attention of one query over a key set.

    ``s_t = scale * (q . k_t) + bias_t``; returns ``(o, lse)`` with
    ``o = sum_t exp(s_t - m) v_t / sum_t exp(s_t - m)`` and
    ``lse = m + ln sum_t exp(s_t - m)``, ``m = max_t s_t``.
    An empty key set has no softmax and raises ``ValueError``.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if keys.shape[0] == 0:
        raise ValueError("softmax over an empty key set is undefined")
    s = (keys @ q) * scale
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)
    m = s.max()
    e = np.exp(s - m)
    z = e.sum()
    return (e @ values) / z, m + np.log(z)


def draft_attn_one(q_row, main_k, main_v, main_len, degree=None,
                   tail_k=None, tail_v=None, tail_len=0, scale=None):
    """One query head of the draft step.

    ``q_row [D]``; ``main_k/main_v [cap][D]`` (decoded values of the query's KV
    head); ``degree [cap]`` (n_t >= 1) or None; ``tail_k/tail_v [tcap][D]``.
    Keys: main tokens ``0..main_len-1`` with bias ``ln n_t`` (0 without
    degrees), then tail tokens ``0..tail_len-1`` with bias 0.
    """
    D = q_row.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    keys = [np.asarray(main_k[:main_len], dtype=np.float64)]
    vals = [np.asarray(main_v[:main_len], dtype=np.float64)]
    if degree is None:
        bias = [np.zeros(main_len)]
    else:
        bias = [np.log(np.asarray(degree[:main_len], dtype=np.float64))]
    if tail_len:
        keys.append(np.asarray(tail_k[:tail_len], dtype=np.float64))
        vals.append(np.asarray(tail_v[:tail_len], dtype=np.float64))
        bias.append(np.zeros(tail_len))
    return attend(q_row, np.concatenate(keys), np.concatenate(vals), scale,
                  np.concatenate(bias))


def draft_attn(q, main_k, main_v, main_len, degree=None, tail_k=None,
               tail_v=None, tail_len=None, scale=None, heads=None):
    """Draft attention for a batch.

    ``q [B][Hq][D]``; ``main_k/main_v [B][Hkv][cap][D]``; ``main_len [B][Hkv]``;
    ``degree [B][Hd][cap]`` with ``Hd`` 1 (shared by all KV heads) or ``Hkv``,
    or None; ``tail_k/tail_v [B][Hkv][tcap][D]``, ``tail_len [B]``.
    Returns ``out [B][Hq][D]`` and ``lse [B][Hq]`` (float64).  ``heads``
    optionally restricts the work to a list of ``(b, h)`` pairs; the other
    entries are left NaN.
    """
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv = main_k.shape[1]
    G = Hq // Hkv
    main_len = np.asarray(main_len).reshape(B, Hkv)
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        g = h // G
        deg = None
        if degree is not None:
            deg = degree[b, 0 if degree.shape[1] == 1 else g]
        tl = 0 if tail_len is None else int(tail_len[b])
        tk = None if tail_k is None else tail_k[b, g]
        tv = None if tail_v is None else tail_v[b, g]
        out[b, h], lse[b, h] = draft_attn_one(
            q[b, h], main_k[b, g], main_v[b, g], int(main_len[b, g]), deg,
            tk, tv, tl, scale)
    return out, lse


def verify_attn_row(q_row, ctx_k, ctx_v, ctx_len, blk_k, blk_v, i, scale=None):
    """One (row, head) of the verify step: keys are context ``0..ctx_len-1``
    followed by block keys ``0..i`` (causal inside the block)."""
    D = q_row.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    keys = np.concatenate([np.asarray(ctx_k[:ctx_len], dtype=np.float64),
                           np.asarray(blk_k[:i + 1], dtype=np.float64)])
    vals = np.concatenate([np.asarray(ctx_v[:ctx_len], dtype=np.float64),
                           np.asarray(blk_v[:i + 1], dtype=np.float64)])
    return attend(q_row, keys, vals, scale)


def verify_attn(q, ctx_k, ctx_v, ctx_len, blk_k, blk_v, scale=None, rows=None):
    """Verify attention for a batch.

    ``q [B][M][Hq][D]``; ``ctx_k/ctx_v [B][Hkv][ccap][D]``; ``ctx_len [B]``;
    ``blk_k/blk_v [B][Hkv][M][D]``.  Returns ``out [B][M][Hq][D]`` and
    ``lse [B][M][Hq]``.  ``rows`` optionally restricts the work to a list of
    ``(b, i, h)`` triples; other entries are left NaN.
    """
    q = np.asarray(q)
    B, M, Hq, D = q.shape
    Hkv = blk_k.shape[1]
    G = Hq // Hkv
    out = np.full((B, M, Hq, D), np.nan)
    lse = np.full((B, M, Hq), np.nan)
    trip = rows if rows is not None else [(b, i, h) for b in range(B)
                                          for i in range(M) for h in range(Hq)]
    for b, i, h in trip:
        g = h // G
        out[b, i, h], lse[b, i, h] = verify_attn_row(
            q[b, i, h], ctx_k[b, g], ctx_v[b, g], int(ctx_len[b]),
            blk_k[b, g], blk_v[b, g], i, scale)
    return out, lse
