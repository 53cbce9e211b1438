"""Pins of the eviction compaction (oracle.compress) against the softmax
definition: attention over the compacted cache is attention over the full
cache with the evicted tokens masked out."""
import numpy as np

from oracle.attention import attend
from oracle.compress import compact_kv


def test_compaction_equals_masked_full_attention():
    rng = np.random.default_rng(3)
    N, D = 200, 16
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, D))
    q = rng.standard_normal(D) * 2
    keep = np.sort(rng.choice(N, 57, replace=False))
    kc, vc = compact_kv(k, v, keep)
    o_c, lse_c = attend(q, kc, vc, 0.25)
    mask = np.full(N, -np.inf)
    mask[keep] = 0.0
    o_f, lse_f = attend(q, k, v, 0.25, bias=mask)
    np.testing.assert_allclose(o_c, o_f, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse_c, lse_f, rtol=1e-12)


def test_identity_selection_and_out_of_range_rows():
    rng = np.random.default_rng(4)
    k = rng.standard_normal((2, 3, 40, 8))
    v = rng.standard_normal((2, 3, 40, 8))
    kc, vc = compact_kv(k, v, np.arange(40))
    assert np.array_equal(kc, k) and np.array_equal(vc, v)
    kc, vc = compact_kv(k, v, [5, -1, 40, 39])
    assert np.array_equal(kc[..., 0, :], k[..., 5, :]) and np.array_equal(vc[..., 3, :], v[..., 39, :])
    assert not kc[..., 1:3, :].any() and not vc[..., 1:3, :].any()


def test_duplicate_index_acts_as_degree_two():
    # a token kept twice enters the softmax twice: the same as one copy with ln 2 added to its score
    rng = np.random.default_rng(5)
    k = rng.standard_normal((30, 8))
    v = rng.standard_normal((30, 8))
    q = rng.standard_normal(8)
    kc, vc = compact_kv(k, v, [0, 3, 3, 7])
    o_dup, _ = attend(q, kc, vc, 0.5)
    kk, vv = compact_kv(k, v, [0, 3, 7])
    o_deg, _ = attend(q, kk, vv, 0.5, bias=np.log([1.0, 2.0, 1.0]))
    np.testing.assert_allclose(o_dup, o_deg, rtol=1e-12, atol=1e-12)
