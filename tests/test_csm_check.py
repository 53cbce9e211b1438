"""CPU pins of the CSM validity check (tests/csm_check.py) used on the GPU's
random-key rounds: a round emulated from the oracle's decisions (centroids
rounded to bf16 as a fp32 kernel would) passes, and each plausible mistake a
kernel could make fails it -- merging the bottom-m instead of the top-m A
tokens, merging into the second-best B token, summing counts instead of
degrees, weighting the mean by counts, or one merge too few."""
import numpy as np
import pytest

import synthetic as S
from oracle import csm as C
from oracle.formats import bf16_to_f64

from .csm_check import check_round

D = 128


def _inputs(n, seed):
    g = np.random.default_rng(seed)
    kb = S.f32_to_bf16_bits(g.standard_normal((n, D), dtype=np.float32))
    vb = S.f32_to_bf16_bits(g.standard_normal((n, D), dtype=np.float32))
    deg = g.integers(1, 5, n).astype(np.float32)
    return kb, vb, deg


def _emulate(kb, vb, deg, sink, recent, chunk, r, mutate=None):
    """The round's outputs from the oracle's per-chunk decisions, optionally
    with one mistake planted; clusters are fp32 weighted means rounded to bf16."""
    k, v = bf16_to_f64(kb), bf16_to_f64(vb)
    n = len(kb)
    ok, ov, od = list(kb[:sink]), list(vb[:sink]), list(deg[:sink])
    for (s, e) in C.chunk_plan(n, sink, recent, chunk):
        a_idx, b_idx, match, score, merged = C.chunk_decisions(k[s:e], r)
        if len(b_idx) and merged.sum():
            m = int(merged.sum())
            if mutate == "rank":            # bottom-m instead of top-m
                order = sorted(range(len(a_idx)), key=lambda i: (score[i], i))
                merged = np.zeros_like(merged)
                merged[order[:m]] = True
            if mutate == "one_less":
                merged[np.nonzero(merged)[0][-1]] = False
            if mutate == "match" and len(b_idx) > 1:   # second-best B token
                sim = C.cosine_matrix(k[s + a_idx], k[s + b_idx])
                match = np.argsort(-sim, axis=1, kind="stable")[:, 1]
        members = {int(b): [int(b)] for b in b_idx}
        for i in np.nonzero(merged)[0]:
            members[int(b_idx[match[i]])].append(int(a_idx[i]))
        for off in range(e - s):
            p = s + off
            if off % 2 == 0 and merged[off // 2] if len(b_idx) else False:
                continue
            mem = [s + x for x in members.get(off, [off])]
            if len(mem) == 1:
                ok.append(kb[p]); ov.append(vb[p]); od.append(deg[p])
                continue
            w = deg[mem].astype(np.float32)
            if mutate == "count_weights":
                w = np.ones_like(w)
            kc = (w[:, None] * k[mem].astype(np.float32)).sum(0) / w.sum()
            vc = (w[:, None] * v[mem].astype(np.float32)).sum(0) / w.sum()
            ok.append(S.f32_to_bf16_bits(kc.astype(np.float32)))
            ov.append(S.f32_to_bf16_bits(vc.astype(np.float32)))
            od.append(float(len(mem)) if mutate == "count_degree" else float(deg[mem].sum()))
    ok += list(kb[n - recent:]); ov += list(vb[n - recent:]); od += list(deg[n - recent:])
    return np.array(ok), np.array(ov), np.array(od, np.float32)


CASES = [(600, 4, 64, 64, 0.25), (600, 4, 64, 64, 0.5), (500, 0, 16, 37, 0.75), (300, 8, 8, 128, 1.0)]


@pytest.mark.parametrize("n,sink,recent,chunk,r", CASES)
def test_emulated_round_passes(n, sink, recent, chunk, r):
    kb, vb, deg = _inputs(n, n + chunk)
    check_round(kb, vb, deg, sink, recent, chunk, r, *_emulate(kb, vb, deg, sink, recent, chunk, r))


@pytest.mark.parametrize("mutate", ["rank", "match", "count_degree", "count_weights", "one_less"])
@pytest.mark.parametrize("n,sink,recent,chunk,r", CASES[:2])
def test_each_planted_mistake_fails(mutate, n, sink, recent, chunk, r):
    kb, vb, deg = _inputs(n, n + chunk)
    out = _emulate(kb, vb, deg, sink, recent, chunk, r, mutate)
    with pytest.raises(AssertionError):
        check_round(kb, vb, deg, sink, recent, chunk, r, *out)
