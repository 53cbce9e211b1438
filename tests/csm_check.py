"""Validity check of one Chunked Soft Matching round's outputs on generic keys.

"Riassunto Tecnico: CentroidKV", "Componenti Chiave" items 3-4: in each
chunk every A token (even position) points at its most similar B token (odd
position) by key cosine, the floor(r |A|) best-matched A tokens merge into
their matches, and a cluster is the degree-weighted mean of its members with
the summed degree.  On random keys two cosines may lie closer than the GPU's
fp32 arithmetic resolves, so more than one result is correct; this check
accepts exactly the results that follow the rules within ``eps`` of the exact
(fp64) cosines:

* the survivor count and the pass-through of sinks and recent tokens;
* in each chunk, the unmerged A tokens and every B token survive in position
  order, unmerged tokens bit-exactly, and exactly floor(r |A|) A tokens are
  gone;
* the merged A set is a top-m set: no unmerged A token's best cosine exceeds
  a merged one's by more than ``eps``;
* every merged A token went to a B token whose cosine is within ``eps`` of
  its best, such that each B token's degree grew by exactly the degrees it
  absorbed and its key and value are the degree-weighted means of its
  members (bf16 tolerance); a B token that absorbed nothing is unchanged.

The inputs are those the round actually read (bf16 bits); the oracle's cosine
routine provides the exact similarities.
"""
import itertools

import numpy as np

from oracle import csm as C
from oracle.formats import bf16_to_f64

from .helpers import assert_close


def _eq(a, b, what):
    np.testing.assert_array_equal(np.asarray(a), np.asarray(b), err_msg=what)


def check_round(kb, vb, deg, sink, recent, chunk, r, ok, ov, od, eps=1e-4):
    """``kb, vb`` bf16 bits ``[n][D]`` (token-major) and ``deg [n]``: the
    round's inputs; ``ok, ov`` bits ``[n_out][D]`` and ``od [n_out]``: its
    outputs.  Raises AssertionError unless the outputs are a valid result."""
    kb, vb = np.asarray(kb), np.asarray(vb)
    deg = np.asarray(deg, np.float64)
    ok, ov, od = np.asarray(ok), np.asarray(ov), np.asarray(od, np.float64)
    n, n_out = len(kb), len(ok)
    assert n_out == C.survivors(n, sink, recent, chunk, r), "survivor count"
    k = bf16_to_f64(kb)
    v = bf16_to_f64(vb)
    _eq(ok[:sink], kb[:sink], "sink keys")
    _eq(ov[:sink], vb[:sink], "sink values")
    _eq(od[:sink], deg[:sink], "sink degrees")
    if recent:
        _eq(ok[n_out - recent:], kb[n - recent:], "recent keys")
        _eq(ov[n_out - recent:], vb[n - recent:], "recent values")
        _eq(od[n_out - recent:], deg[n - recent:], "recent degrees")
    pos = sink
    for (s, e) in C.chunk_plan(n, sink, recent, chunk):
        L = e - s
        n_a, n_b = (L + 1) // 2, L // 2
        m = int(np.floor(r * n_a)) if n_b else 0
        ns = L - m
        # walk the chunk: B tokens always survive; an A token survives when the
        # next output row is its row, bit for bit
        slot_of, gone, i = {}, [], 0
        for off in range(L):
            p = s + off
            if off % 2 == 1:
                assert i < ns, f"chunk at {s}: outputs exhausted before B token {p}"
                slot_of[p] = pos + i
                i += 1
            elif (i < ns and np.array_equal(ok[pos + i], kb[p]) and np.array_equal(ov[pos + i], vb[p])
                  and od[pos + i] == deg[p]):
                slot_of[p] = pos + i
                i += 1
            else:
                gone.append(off // 2)
        assert i == ns, f"chunk at {s}: {i} survivors identified, {ns} expected"
        assert len(gone) == m, f"chunk at {s}: {len(gone)} A tokens merged, floor(r |A|) = {m}"
        if m:
            a_pos = s + 2 * np.arange(n_a)
            b_pos = s + 2 * np.arange(n_b) + 1
            cos = C.cosine_matrix(k[a_pos], k[b_pos])
            best = cos.max(axis=1)
            merged = np.zeros(n_a, bool)
            merged[gone] = True
            if m < n_a:
                assert best[merged].min() >= best[~merged].max() - eps, \
                    f"chunk at {s}: the merged set is not a top-{m} set by similarity"
            absorbed = {int(b): od[slot_of[int(b)]] - deg[int(b)] for b in b_pos}
            cands = [np.nonzero(cos[a] >= best[a] - eps)[0] for a in gone]
            choices = [list(b_pos[c]) for c in cands]
            n_comb = int(np.prod([len(c) for c in choices]))
            assert n_comb <= 4096, f"chunk at {s}: too many near-tied matches to enumerate"
            ok_assign = None
            for assign in itertools.product(*choices):
                got = {int(b): 0.0 for b in b_pos}
                for a, b in zip(gone, assign):
                    got[int(b)] += deg[s + 2 * a]
                if all(got[b] == absorbed[b] for b in got):
                    ok_assign = assign
                    break
            assert ok_assign is not None, f"chunk at {s}: no assignment to near-best matches gives the degrees"
            members = {int(b): [int(b)] for b in b_pos}
            for a, b in zip(gone, ok_assign):
                members[int(b)].append(s + 2 * a)
            for b, mem in members.items():
                sl = slot_of[b]
                if len(mem) == 1:
                    _eq(ok[sl], kb[b], f"unmerged B token {b} key")
                    _eq(ov[sl], vb[b], f"unmerged B token {b} value")
                    continue
                w = deg[mem]
                assert od[sl] == w.sum(), f"cluster at {b}: degree"
                assert_close(bf16_to_f64(ok[sl]), (w[:, None] * k[mem]).sum(0) / w.sum(), 1e-2, f"cluster {b} key")
                assert_close(bf16_to_f64(ov[sl]), (w[:, None] * v[mem]).sum(0) / w.sum(), 1e-2, f"cluster {b} value")
        else:
            for off in range(L):
                _eq(ok[pos + off], kb[s + off], f"chunk at {s}: token {s + off} key")
                _eq(ov[pos + off], vb[s + off], f"chunk at {s}: token {s + off} value")
        pos += ns
    assert pos == n_out - recent, "chunk outputs do not end where the recent tokens start"
