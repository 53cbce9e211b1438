"""Pins of the oracle's Chunked Soft Matching round (CentroidKV, "Componenti
Chiave" items 2-4): identity at r = 0, conservation of total degree and of the
degree-weighted key/value sums, the survivor count, preserved sinks and recent
tokens, matches that are the most similar B token (checked by an explicit loop
over the chunk), a merged set that is a top-m set by similarity, and the
duplicate-token identity of the log-degree term (merging exact duplicates
leaves draft attention unchanged)."""
import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import csm as C

RNG = np.random.default_rng(7)


def _kv(n, D=16, scale=1.0):
    return RNG.standard_normal((n, D)) * scale, RNG.standard_normal((n, D))


def test_r_zero_is_identity():
    k, v = _kv(70)
    deg = RNG.integers(1, 5, 70).astype(float)
    k2, v2, d2, _ = C.csm_round(k, v, deg, 4, 8, 16, 0.0)
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(v2, v)
    np.testing.assert_array_equal(d2, deg)


@pytest.mark.parametrize("n,sink,recent,chunk,r", [(100, 4, 16, 16, 0.5), (131, 0, 0, 32, 1.0),
                                                   (64, 4, 4, 7, 0.75), (9, 2, 2, 4, 1.0)])
def test_conservation_and_counts(n, sink, recent, chunk, r):
    k, v = _kv(n)
    deg = RNG.integers(1, 6, n).astype(float)
    k2, v2, d2, info = C.csm_round(k, v, deg, sink, recent, chunk, r)
    assert math.isclose(d2.sum(), deg.sum())
    np.testing.assert_allclose((d2[:, None] * k2).sum(0), (deg[:, None] * k).sum(0), rtol=1e-12, atol=1e-10)
    np.testing.assert_allclose((d2[:, None] * v2).sum(0), (deg[:, None] * v).sum(0), rtol=1e-12, atol=1e-10)
    assert len(k2) == C.survivors(n, sink, recent, chunk, r)
    merged = sum(int(c["merged"].sum()) for c in info)
    assert len(k2) == n - merged
    # sinks and recent tokens pass through unchanged
    np.testing.assert_array_equal(k2[:sink], k[:sink])
    np.testing.assert_array_equal(d2[:sink], deg[:sink])
    if recent:
        np.testing.assert_array_equal(k2[len(k2) - recent:], k[n - recent:])


def test_matches_and_top_m_by_explicit_loops():
    k, v = _kv(96, D=8)
    _, _, _, info = C.csm_round(k, v, None, 0, 0, 24, 0.5)
    for c in info:
        keys = k[c["start"]:c["end"]]
        a_pos, b_pos = list(range(0, len(keys), 2)), list(range(1, len(keys), 2))
        for i, a in enumerate(a_pos):
            best, best_j = -2.0, -1
            for j, b in enumerate(b_pos):
                dot = sum(keys[a][d] * keys[b][d] for d in range(keys.shape[1]))
                cs = dot / (math.sqrt(sum(x * x for x in keys[a])) * math.sqrt(sum(x * x for x in keys[b])))
                if cs > best + 1e-15:
                    best, best_j = cs, j
            assert c["match"][i] == best_j
            assert math.isclose(c["score"][i], best, rel_tol=1e-12)
        m = int(np.floor(0.5 * len(a_pos)))
        assert c["merged"].sum() == m
        if 0 < m < len(a_pos):
            assert c["score"][c["merged"]].min() >= c["score"][~c["merged"]].max()


def test_merging_duplicates_keeps_attention():
    # token 2i+1 duplicates token 2i inside every chunk: r = 1 merges each A
    # token into its duplicate, and with ln(degree) in the scores the
    # attention over the compressed cache equals the original one
    D, n = 32, 4 + 6 * 16 + 8
    k, v = _kv(n, D, scale=2.0)
    for s in range(4, n - 8, 16):
        for p in range(s, s + 16, 2):
            k[p + 1], v[p + 1] = k[p], v[p]
    k2, v2, d2, info = C.csm_round(k, v, None, 4, 8, 16, 1.0)
    assert len(k2) == 4 + 6 * 8 + 8
    assert all(c["merged"].all() for c in info)
    q = RNG.standard_normal((1, 4, D))
    o1, l1 = A.draft_attn(q, k[None, None], v[None, None], np.array([[n]]))
    o2, l2 = A.draft_attn(q, k2[None, None], v2[None, None], np.array([[len(k2)]]), degree=d2[None, None])
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------------------
# The pipeline over several rounds ("Pipeline di Inferenza", "Scheduling
# Progressivo"): a round after the prefill when over the budget, one every
# `every` decode steps while over the budget, r_j = r_init - j * delta_r.
def test_schedule_matches_the_hand_derived_golden():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "centroid_schedule.json")))
    c = g["config"]
    D = 8
    k0, v0 = _kv(c["n_prefill"], D)
    kn, vn = _kv(c["decode_steps"], D)
    k, v, deg, rounds = C.centroid_run(k0, v0, kn, vn, c["budget"], c["every"], c["r_init"], c["delta_r"],
                                       c["n_sink"], c["n_recent"], c["chunk"])
    got = [{key: rd[key] for key in ("step", "j", "r", "n_in", "n_out")} for rd in rounds]
    assert got == g["rounds"]
    assert len(k) == g["final_tokens"] and deg.sum() == g["total_degree"]


def test_schedule_ratio_decays_and_clamps():
    assert [C.schedule_ratio(j, 0.75, 0.25) for j in range(5)] == [0.75, 0.5, 0.25, 0.0, 0.0]
    assert C.schedule_ratio(0, 1.5, 0.1) == 1.0
    # the decaying ratio of a schedule step that a float32 would round down
    assert int(np.floor(C.schedule_ratio(3, 1.0, 0.1) * 10)) == 7


def test_pipeline_conserves_degree_and_weighted_sums_over_rounds():
    D, n0, steps = 16, 400, 160
    k0, v0 = _kv(n0, D)
    kn, vn = _kv(steps, D)
    k, v, deg, rounds = C.centroid_run(k0, v0, kn, vn, budget=250, every=32, r_init=0.75, delta_r=0.125,
                                       n_sink=4, n_recent=32, chunk=32)
    assert len(rounds) >= 4
    kall, vall = np.concatenate([k0, kn]), np.concatenate([v0, vn])
    assert deg.sum() == n0 + steps                       # every token counted exactly once
    np.testing.assert_allclose((deg[:, None] * k).sum(0), kall.sum(0), rtol=1e-10, atol=1e-9)
    np.testing.assert_allclose((deg[:, None] * v).sum(0), vall.sum(0), rtol=1e-10, atol=1e-9)
    for i, rd in enumerate(rounds):
        assert rd["j"] == i and rd["r"] == C.schedule_ratio(i, 0.75, 0.125)
        assert rd["n_out"] == C.survivors(rd["n_in"], 4, 32, 32, rd["r"])
        # a round removes at most half of its middle segment (only A tokens merge away)
        mid = rd["n_in"] - 4 - 32
        assert rd["n_in"] - rd["n_out"] <= (mid + 1) // 2
        # rounds run only after the prefill or on a multiple of `every`, and only over the budget
        assert rd["step"] % 32 == 0 and rd["n_in"] > 250
    # recent tokens are the last decode tokens, untouched
    np.testing.assert_array_equal(k[-32:], kn[-32:])


def test_pipeline_of_duplicate_runs_keeps_attention_exactly():
    # Every token appears in a run of 8 identical copies (prefill and decode
    # alike).  Merges that join identical tokens leave the log-degree
    # attention unchanged, so after several rounds the compressed cache must
    # attend exactly like the full sequence -- which needs the degrees carried
    # over from round to round (a reset degree would change the weights).
    D, run = 32, 8
    base_k, base_v = _kv(100, D, scale=3.0)
    seq_k = np.repeat(base_k, run, axis=0)
    seq_v = np.repeat(base_v, run, axis=0)
    n0 = 4 + 64 * 6
    k0, v0, kn, vn = seq_k[:n0], seq_v[:n0], seq_k[n0:n0 + 256], seq_v[n0:n0 + 256]
    k, v, deg, rounds = C.centroid_run(k0, v0, kn, vn, budget=200, every=64, r_init=0.5, delta_r=0.125,
                                       n_sink=4, n_recent=16, chunk=32)
    assert len(rounds) >= 3
    for rd in rounds:   # the premise: every merge in every round joined identical tokens
        for c in rd["info"]:
            if c["merged"].any():
                np.testing.assert_allclose(c["score"][c["merged"]], 1.0, rtol=0, atol=1e-12)
    assert sum(int(c["merged"].sum()) for rd in rounds for c in rd["info"]) > 0
    q = RNG.standard_normal((1, 4, D))
    full_k, full_v = np.concatenate([k0, kn]), np.concatenate([v0, vn])
    o1, l1 = A.draft_attn(q, full_k[None, None], full_v[None, None], np.array([[len(full_k)]]))
    o2, l2 = A.draft_attn(q, k[None, None], v[None, None], np.array([[len(k)]]), degree=deg[None, None])
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-10, atol=1e-12)
