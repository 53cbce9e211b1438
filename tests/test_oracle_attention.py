"""Pins of the oracle's attention against things outside the oracle.

* torch ``scaled_dot_product_attention`` (CPU, float64, ``enable_gqa``) is an
  independent implementation of the softmax-attention definition; an additive
  float mask carries the log-degree term and the block-causal pattern.
* The log-degree term ("Riassunto Tecnico: CentroidKV", "Componenti Chiave",
  item 4) must make a centroid of degree n equal to n identical tokens.
* Softmax attention is invariant under a permutation of its key set.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

from oracle import attention as A
from oracle.formats import bf16_to_f64

RNG = np.random.default_rng(1234)


def _sdpa(q, k, v, mask=None, scale=None):
    """q [Hq][Lq][D], k/v [Hkv][Lk][D] float64 -> [Hq][Lq][D]."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x))[None] for x in (q, k, v))
    m = None if mask is None else torch.from_numpy(mask)[None]
    return F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=scale,
                                          enable_gqa=True)[0].numpy()


@pytest.mark.parametrize("Hq,Hkv,D", [(4, 2, 64), (8, 8, 32), (10, 2, 128), (32, 8, 128)])
def test_draft_matches_sdpa_with_log_degree_mask(Hq, Hkv, D):
    B, cap, tcap = 2, 97, 5
    q = RNG.standard_normal((B, Hq, D)) * 2
    mk = RNG.standard_normal((B, Hkv, cap, D))
    mv = RNG.standard_normal((B, Hkv, cap, D))
    tk = RNG.standard_normal((B, Hkv, tcap, D))
    tv = RNG.standard_normal((B, Hkv, tcap, D))
    deg = RNG.integers(1, 5, (B, 1, cap)).astype(np.float64)
    main_len = np.array([[cap - 3] * Hkv, [40 + h for h in range(Hkv)]])
    tail_len = np.array([tcap, 2])
    out, lse = A.draft_attn(q, mk, mv, main_len, deg, tk, tv, tail_len)
    for b in range(B):
        for g in range(Hkv):
            L = main_len[b, g]
            keys = np.concatenate([mk[b, g, :L], tk[b, g, :tail_len[b]]])
            vals = np.concatenate([mv[b, g, :L], tv[b, g, :tail_len[b]]])
            bias = np.concatenate([np.log(deg[b, 0, :L]), np.zeros(tail_len[b])])
            G = Hq // Hkv
            qs = q[b, g * G:(g + 1) * G][:, None, :]
            ref = _sdpa(qs, keys[None], vals[None], bias[None, None, :].repeat(G, 0))
            np.testing.assert_allclose(out[b, g * G:(g + 1) * G], ref[:, 0], rtol=1e-12, atol=1e-12)
            s = qs[:, 0] @ keys.T / np.sqrt(D) + bias
            np.testing.assert_allclose(lse[b, g * G:(g + 1) * G], logsumexp(s, axis=1), rtol=1e-12)


def test_draft_gqa_head_mapping_against_sdpa_whole_batch():
    # One SDPA call over all heads: pins query head h -> KV head h // G.
    Hq, Hkv, D, L = 12, 3, 16, 33
    q = RNG.standard_normal((1, Hq, D))
    k = RNG.standard_normal((1, Hkv, L, D))
    v = RNG.standard_normal((1, Hkv, L, D))
    out, _ = A.draft_attn(q, k, v, np.full((1, Hkv), L))
    ref = _sdpa(q[0][:, None, :], k[0], v[0])[:, 0]
    np.testing.assert_allclose(out[0], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("M,N,G", [(1, 50, 2), (9, 31, 2), (33, 64, 5), (32, 0, 8)])
def test_verify_matches_sdpa_block_causal(M, N, G):
    Hkv, D = 2, 32
    Hq = Hkv * G
    q = RNG.standard_normal((1, M, Hq, D)) * 3
    ck = RNG.standard_normal((1, Hkv, N + 3, D))
    cv = RNG.standard_normal((1, Hkv, N + 3, D))
    bk = RNG.standard_normal((1, Hkv, M, D))
    bv = RNG.standard_normal((1, Hkv, M, D))
    out, lse = A.verify_attn(q, ck, cv, np.array([N]), bk, bv)
    keys = np.concatenate([ck[0, :, :N], bk[0]], axis=1)
    vals = np.concatenate([cv[0, :, :N], bv[0]], axis=1)
    visible = np.zeros((M, N + M), dtype=bool)
    visible[:, :N] = True
    visible[:, N:] = np.tril(np.ones((M, M), dtype=bool))
    mask = np.where(visible, 0.0, -np.inf)[None].repeat(Hq, 0)
    ref = _sdpa(q[0].transpose(1, 0, 2), keys, vals, mask)
    np.testing.assert_allclose(out[0], ref.transpose(1, 0, 2), rtol=1e-11, atol=1e-12)


def test_log_degree_equals_duplicated_tokens():
    # A centroid of degree n must act as n identical copies (closed form of
    # the log-degree softmax term).
    D, L = 64, 40
    q = RNG.standard_normal(D) * 3
    k = RNG.standard_normal((L, D))
    v = RNG.standard_normal((L, D))
    deg = RNG.integers(1, 6, L)
    o_bias, lse_bias = A.draft_attn_one(q, k, v, L, deg.astype(np.float64))
    kd = np.repeat(k, deg, axis=0)
    vd = np.repeat(v, deg, axis=0)
    o_dup, lse_dup = A.draft_attn_one(q, kd, vd, kd.shape[0])
    np.testing.assert_allclose(o_bias, o_dup, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_bias, lse_dup, rtol=1e-12)
    # and without the bias the two differ (the term is not vacuous)
    o_nob, _ = A.draft_attn_one(q, k, v, L)
    assert np.abs(o_nob - o_dup).max() > 1e-3


def test_permutation_invariance():
    D, L = 32, 57
    q = RNG.standard_normal(D) * 2
    k = RNG.standard_normal((L, D))
    v = RNG.standard_normal((L, D))
    deg = RNG.integers(1, 5, L).astype(np.float64)
    p = RNG.permutation(L)
    o1, l1 = A.draft_attn_one(q, k, v, L, deg)
    o2, l2 = A.draft_attn_one(q, k[p], v[p], L, deg[p])
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_special_cases():
    D = 8
    v = RNG.standard_normal((3, D))
    k = RNG.standard_normal((3, D))
    q = RNG.standard_normal(D)
    # one key: output is its value, lse is its score
    o, lse = A.draft_attn_one(q, k[:1], v[:1], 1)
    np.testing.assert_array_equal(o, v[0])
    assert lse == pytest.approx(q @ k[0] / np.sqrt(D), rel=1e-15)
    # two keys: logistic weights
    o, _ = A.draft_attn_one(q, k[:2], v[:2], 2)
    s = k[:2] @ q / np.sqrt(D)
    w0 = 1.0 / (1.0 + np.exp(s[1] - s[0]))
    np.testing.assert_allclose(o, w0 * v[0] + (1 - w0) * v[1], rtol=1e-13)
    # equal keys: plain average of the values
    o, _ = A.draft_attn_one(q, np.repeat(k[:1], 3, 0), v, 3)
    np.testing.assert_allclose(o, v.mean(0), rtol=1e-13, atol=1e-15)
    # empty set is an error
    with pytest.raises(ValueError):
        A.draft_attn_one(q, k, v, 0)


def test_verify_single_row_is_draft_over_context_plus_self():
    # M = 1 verify == draft over the context with the block key as tail.
    D, N = 64, 70
    q = RNG.standard_normal((1, 1, 2, D))
    ck = RNG.standard_normal((1, 1, N, D))
    cv = RNG.standard_normal((1, 1, N, D))
    bk = RNG.standard_normal((1, 1, 1, D))
    bv = RNG.standard_normal((1, 1, 1, D))
    vo, vl = A.verify_attn(q, ck, cv, np.array([N]), bk, bv)
    do, dl = A.draft_attn(q[:, 0], ck, cv, np.array([[N]]), None, bk, bv, np.array([1]))
    np.testing.assert_array_equal(vo[:, 0], do)
    np.testing.assert_array_equal(vl[:, 0], dl)


def test_bf16_decode_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F7F, 0x0001], dtype=np.uint16)
    vals = bf16_to_f64(bits)
    assert vals[0] == 1.0 and vals[1] == -1.0 and vals[2] == 0.0
    assert np.signbit(vals[3]) and vals[3] == 0.0
    assert vals[4] == 3.140625
    assert vals[5] == (2.0 - 2.0 ** -7) * 2.0 ** 127   # largest finite bf16
    assert vals[6] == 2.0 ** -133
