"""Pins of the oracle's acceptance rule ("Riepilogo Tecnico: VeriCache",
"Algoritmo Principale", step 3): hand-derived golden cases, brute force over
every match/mismatch pattern, and numpy's first-occurrence argmax."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.accept import accept, accept_batch, fp32_sum_bound, greedy_argmax, lm_head_argmax, lm_head_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_cases.json")


def test_golden_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 8
    for c in cases:
        y, n, emitted = accept(np.array(c["logits"], dtype=np.float64), c["draft"])
        assert y == c["argmax"], c["name"]
        assert n == c["n"], c["name"]
        assert emitted == c["emitted"], c["name"]


@pytest.mark.parametrize("k", range(0, 9))
def test_brute_force_all_patterns(k):
    # For every pattern of matches, n is the first mismatch index (k if none),
    # never longer, and the round emits n + 1 tokens ending in the prediction.
    V = 11
    rng = np.random.default_rng(k)
    for pattern in itertools.product([True, False], repeat=k):
        y = rng.integers(0, V, k + 1)
        logits = rng.standard_normal((k + 1, V))
        for j in range(k + 1):
            logits[j, y[j]] = logits[j].max() + 1.0
        d = [int(y[j]) if pattern[j] else int((y[j] + 1 + rng.integers(0, V - 1)) % V)
             for j in range(k)]
        yy, n, emitted = accept(logits, d)
        first_miss = next((j for j, ok in enumerate(pattern) if not ok), k)
        assert yy == [int(t) for t in y]
        assert n == first_miss and n <= k
        assert emitted[:n] == d[:n] and emitted[-1] == y[n] and len(emitted) == n + 1
        if n == k:   # bonus token on a full match
            assert emitted[-1] == y[k]


def test_argmax_matches_numpy_first_occurrence_with_ties():
    rng = np.random.default_rng(7)
    for _ in range(200):
        row = rng.integers(-3, 4, rng.integers(1, 40)).astype(np.float64)
        assert greedy_argmax(row) == int(np.argmax(row))
    for _ in range(50):
        row = rng.standard_normal(1000).astype(np.float32)
        assert greedy_argmax(row) == int(np.argmax(row))


def test_rejects_non_finite():
    with pytest.raises(ValueError):
        greedy_argmax([0.0, np.nan])
    with pytest.raises(ValueError):
        greedy_argmax([0.0, np.inf])


def test_batch_layout():
    logits = np.zeros((2, 3, 4))
    logits[0, :, 1] = 1
    logits[1, 0, 2] = 1
    logits[1, 1:, 3] = 1
    am, n, toks, n_out = accept_batch(logits, np.array([[1, 1], [3, 3]]))
    assert am.tolist() == [[1, 1, 1], [2, 3, 3]]
    assert n.tolist() == [2, 0]
    assert toks.tolist() == [[1, 1, 1], [2, -1, -1]]
    assert n_out.tolist() == [3, 1]


# ---- LM head fused with the greedy choice -----------------------------------

def _int_bf16(x):
    """Small integers are exact in bf16: their bit pattern is the top half of fp32."""
    return (np.asarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_lm_head_logits_exact_on_integers():
    # Integer inputs: the logits follow from exact int64 arithmetic, a path
    # that shares nothing with the fp64 evaluation.
    rng = np.random.default_rng(11)
    for R, Dm, V in ((1, 32, 5), (7, 96, 300), (3, 64, 17)):
        hi = rng.integers(-8, 9, size=(R, Dm))
        wi = rng.integers(-8, 9, size=(V, Dm))
        ref = hi.astype(np.int64) @ wi.T.astype(np.int64)
        got = lm_head_logits(_int_bf16(hi), _int_bf16(wi))
        np.testing.assert_array_equal(got, ref.astype(np.float64))
        assert lm_head_argmax(_int_bf16(hi), _int_bf16(wi)).tolist() == [int(np.argmax(r)) for r in ref]


def test_lm_head_planted_rows_cauchy_schwarz():
    # Rows of equal norm: h = w[t] attains the unique maximum h.w[t] = |w|^2
    # over all distinct rows (Cauchy-Schwarz), so the argmax is t.
    import synthetic as S
    targets = np.array([0, 5, 511, 17, 17, 300])
    h, w = S.lm_planted(512, 64, targets, cfg_seed=3)
    assert lm_head_argmax(h, w).tolist() == targets.tolist()


def test_lm_head_duplicate_rows_pick_lowest_index():
    import synthetic as S
    h, w = S.lm_planted(64, 32, [40, 9], cfg_seed=5)
    w = w.copy()
    w[12] = w[40]           # an equal maximum at a lower index than the target
    w[50] = w[9]            # and one at a higher index
    assert lm_head_argmax(h, w).tolist() == [12, 9]


def test_fp32_sum_bound_covers_fp32_evaluation():
    rng = np.random.default_rng(2)
    import synthetic as S
    h = S.f32_to_bf16_bits(rng.standard_normal((4, 512), dtype=np.float32))
    w = S.f32_to_bf16_bits(rng.standard_normal((256, 512), dtype=np.float32) * np.float32(0.02))
    exact = lm_head_logits(h, w)
    from oracle.formats import bf16_to_f64
    h32 = bf16_to_f64(h).astype(np.float32)
    w32 = bf16_to_f64(w).astype(np.float32)
    # fp32 sums in two different orders stay within the bound
    fwd = np.zeros_like(exact, dtype=np.float32)
    for k in range(512):
        fwd += np.outer(h32[:, k], w32[:, k]).astype(np.float32)
    bound = fp32_sum_bound(h, w)[:, None]
    assert np.all(np.abs(fwd - exact) <= bound)
    assert np.all(np.abs((h32 @ w32.T).astype(np.float64) - exact) <= bound)
    assert np.all(bound > 0)
