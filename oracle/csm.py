"""One clustering round of Chunked Soft Matching (CentroidKV), float64.

Test infrastructure only (see :mod:`oracle`).

"Riassunto Tecnico: CentroidKV", section "Metodologia: CentroidKV",
"Componenti Chiave":

* item 2 "Pipeline di Inferenza": attention sinks and recent tokens are kept
  out of the partition;
* item 3 "Chunked Soft Matching (CSM)": the sequence is cut into chunks;
  inside a chunk the tokens are split alternately into two sets A and B; like
  bipartite soft matching, each token is paired with a highly similar token of
  the other set; the candidate pairs are ranked by similarity and only the top
  fraction, set by the compression ratio r, is merged; r decays linearly over
  rounds (``r = r_init - j * delta_r``);
* item 1 "Osservazioni": the similarity that drives the grouping is the
  cosine similarity of the key states;
* item 4 "Aggregazione": a cluster's key and value are the degree-weighted
  mean of its members, and its degree n_t is their summed degree.

Readings where the page is silent (each is a choice, listed in the design
notes):

* A = even positions inside the chunk, B = odd positions; each A token points
  at its most similar B token of the same chunk (lowest B index on equal
  similarity); the ``floor(r * |A|)`` A tokens with the highest similarity
  (lower A index first on equal similarity) merge into the token they point
  at, chunk by chunk;
* similarity = cosine of the key vectors as cached;
* one round per call with a given r; a last chunk shorter than ``chunk`` is
  processed the same way;
* survivors (unmerged A tokens and every B token) keep ascending position.

The rounds compose into the inference pipeline of item 2 and the progressive
schedule of item 3 (:func:`schedule_ratio`, :func:`centroid_run`), read as:

* after the prefill, one round when the cache holds more tokens than the
  budget; during decoding the cache grows by one token (degree 1) per step
  and every ``every``-th step one round runs when it is over the budget;
* round j (counting the rounds run so far, prefill round included) merges
  with ``r_j = r_init - j * delta_r``, kept within [0, 1]; a round reduces
  its middle segment by at most half, since only A tokens (every other token
  of a chunk) can merge away ("Limitazioni": at most half per step);
* degrees carry over from round to round (a centroid's degree counts every
  token it ever absorbed).

Parity: pinned by invariants a wrong index, weight or sign would break --
conservation of total degree and of the degree-weighted key and value sums,
the survivor count, the top-m property of the merged set, r = 0 as the
identity -- and by the duplicate-token identity: merging exact duplicates
leaves attention with the log-degree term unchanged.
"""
import numpy as np


def cosine_matrix(ka, kb):
    """Cosine similarity of every row of ``ka`` with every row of ``kb``."""
    na = np.linalg.norm(ka, axis=1)
    nb = np.linalg.norm(kb, axis=1)
    return (ka @ kb.T) / np.outer(na, nb)


def chunk_plan(n, n_sink, n_recent, chunk):
    """Start/end of every chunk of the clustered middle ``[n_sink, n - n_recent)``."""
    lo, hi = n_sink, max(n_sink, n - n_recent)
    return [(s, min(s + chunk, hi)) for s in range(lo, hi, chunk)]


def chunk_decisions(keys, r):
    """Decisions of one chunk: ``match[i]`` (B index, chunk-local) of each A
    token i, its similarity ``score[i]`` and the boolean ``merged[i]``."""
    a_idx = np.arange(0, len(keys), 2)
    b_idx = np.arange(1, len(keys), 2)
    n_a = len(a_idx)
    if len(b_idx) == 0:
        return a_idx, b_idx, np.zeros(n_a, np.int64), np.zeros(n_a), np.zeros(n_a, bool)
    sim = cosine_matrix(keys[a_idx], keys[b_idx])
    match = np.argmax(sim, axis=1)                    # first maximum = lowest B index
    score = sim[np.arange(n_a), match]
    m = int(np.floor(r * n_a))
    order = sorted(range(n_a), key=lambda i: (-score[i], i))
    merged = np.zeros(n_a, bool)
    merged[order[:m]] = True
    return a_idx, b_idx, match, score, merged


def csm_round(k, v, deg, n_sink, n_recent, chunk, r):
    """One CSM round over one KV head.

    ``k, v [n][D]`` float64, ``deg [n]`` (None = all 1).  Returns
    ``(k_out, v_out, deg_out, info)`` with the survivors in ascending position
    and ``info`` the per-chunk decisions.
    """
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n = len(k)
    deg = np.ones(n) if deg is None else np.asarray(deg, np.float64)
    members = {}                      # B token -> the A tokens merged into it
    merged_away = np.zeros(n, bool)
    info = []
    for (s, e) in chunk_plan(n, n_sink, n_recent, chunk):
        a_idx, b_idx, match, score, merged = chunk_decisions(k[s:e], r)
        for i in np.nonzero(merged)[0]:
            members.setdefault(s + b_idx[match[i]], []).append(s + a_idx[i])
            merged_away[s + a_idx[i]] = True
        info.append(dict(start=s, end=e, match=match, score=score, merged=merged))
    k_out, v_out, d_out = k.copy(), v.copy(), deg.copy()
    for dst, srcs in members.items():
        idx = [dst] + srcs
        w = deg[idx]
        d_out[dst] = w.sum()
        k_out[dst] = (w[:, None] * k[idx]).sum(0) / w.sum()
        v_out[dst] = (w[:, None] * v[idx]).sum(0) / w.sum()
    keep = ~merged_away
    return k_out[keep], v_out[keep], d_out[keep], info


def survivors(n, n_sink, n_recent, chunk, r):
    """Survivor count of one round (it depends only on the sizes)."""
    out = n
    for (s, e) in chunk_plan(n, n_sink, n_recent, chunk):
        out -= int(np.floor(r * ((e - s + 1) // 2))) if e - s > 1 else 0
    return out


def schedule_ratio(j, r_init, delta_r):
    """Ratio of clustering round ``j`` (0-based): ``r_init - j * delta_r``
    ("Scheduling Progressivo"), kept within [0, 1]."""
    return min(1.0, max(0.0, r_init - j * delta_r))


def centroid_run(k0, v0, k_new, v_new, budget, every, r_init, delta_r, n_sink, n_recent, chunk):
    """The CentroidKV pipeline over one KV head ("Pipeline di Inferenza",
    "Scheduling Progressivo"): the prefill cache ``k0, v0 [n0][D]`` (degree
    1), a round after the prefill if ``n0 > budget``, then one decode token
    per step (``k_new, v_new [steps][D]``, degree 1) and a round after every
    ``every``-th step while the cache holds more than ``budget`` tokens.

    Returns ``(k, v, deg, rounds)``; ``rounds`` lists per round a dict with
    the decode step it ran after (0 = prefill), its index ``j``, ratio ``r``,
    token counts ``n_in`` / ``n_out`` and the round's per-chunk decisions.
    """
    if every < 1:
        raise ValueError("every must be >= 1")
    k = np.asarray(k0, np.float64).copy()
    v = np.asarray(v0, np.float64).copy()
    deg = np.ones(len(k))
    rounds = []

    def cluster(step):
        nonlocal k, v, deg
        j = len(rounds)
        r = schedule_ratio(j, r_init, delta_r)
        n_in = len(k)
        k, v, deg, info = csm_round(k, v, deg, n_sink, n_recent, chunk, r)
        rounds.append(dict(step=step, j=j, r=r, n_in=n_in, n_out=len(k), info=info))

    if len(k) > budget:
        cluster(0)
    for t in range(len(k_new)):
        k = np.concatenate([k, np.asarray(k_new[t], np.float64)[None]])
        v = np.concatenate([v, np.asarray(v_new[t], np.float64)[None]])
        deg = np.concatenate([deg, [1.0]])
        if (t + 1) % every == 0 and len(k) > budget:
            cluster(t + 1)
    return k, v, deg, rounds
