"""Pins of the oracle's acceptance rule ("Riepilogo Tecnico: VeriCache",
"Algoritmo Principale", step 3): hand-derived golden cases, brute force over
every match/mismatch pattern, and numpy's first-occurrence argmax."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.accept import accept, accept_batch, greedy_argmax

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
