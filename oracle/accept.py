"""Greedy token choice and the acceptance rule.

Test infrastructure only (see :mod:`oracle`).

"Riepilogo Tecnico: VeriCache", section "Algoritmo Principale", step 3
("Accettazione"): drafted tokens are accepted up to the first position where
they disagree with the full-cache prediction; when every drafted token agrees,
one extra "bonus" token (the full-cache prediction after the last draft) is
accepted too; decoding then resumes from the last accepted token.  Section
"Risultati Sperimentali" states the output equals full-cache greedy decoding,
so the prediction is the greedy argmax.

Readings where the pages are silent:
* On a mismatch at position n+1 the full-cache prediction ``y_{n+1}`` is
  emitted as well (the correction), so every round emits ``n + 1`` tokens and
  the bonus is the special case ``n = k``.  Without it a round with ``n = 0``
  would leave the state unchanged and repeat forever.
* Ties in the argmax go to the lowest vocabulary index; comparisons are on
  values (so -0.0 equals +0.0); non-finite logits are rejected.

Parity: pinned by brute force over every match/mismatch pattern for small k,
by hand-derived cases under ``tests/golden/`` and by ``numpy.argmax``'s
first-occurrence rule.  The LM-head argmax (:func:`lm_head_argmax`) is pinned
by exact integer arithmetic on integer-valued inputs and by the
Cauchy-Schwarz maximum of planted equal-norm rows.
"""
import numpy as np

from .formats import bf16_to_f64


def greedy_argmax(row):
    """Lowest index attaining the maximum value of a finite vector."""
    row = np.asarray(row, dtype=np.float64)
    if row.size == 0:
        raise ValueError("argmax of an empty row")
    if not np.all(np.isfinite(row)):
        raise ValueError("logits must be finite")
    best = row.max()
    return int(np.flatnonzero(row == best)[0])


def accept(logits, draft):
    """Acceptance for one request.

    ``logits [M][V]`` are the full-cache logits of the verify block rows
    ``x0, d_1, ..., d_k`` (``M = k + 1``); ``draft [k]`` holds ``d_1..d_k``.
    Row ``j`` predicts ``y_{j+1} = argmax(logits[j])``.
    Returns ``(y, n, emitted)``: the M predictions, the number ``n`` of
    leading drafts equal to their prediction, and the emitted tokens
    ``d_1..d_n, y_{n+1}``.
    """
    logits = np.asarray(logits)
    M = logits.shape[0]
    k = M - 1
    draft = [int(t) for t in draft]
    if len(draft) != k:
        raise ValueError("draft length must be M - 1")
    y = [greedy_argmax(logits[j]) for j in range(M)]
    n = 0
    while n < k and draft[n] == y[n]:
        n += 1
    return y, n, draft[:n] + [y[n]]


def accept_batch(logits, drafts):
    """Batched :func:`accept`: ``logits [B][M][V]``, ``drafts [B][M-1]``.

    Returns int32 arrays ``argmax [B][M]``, ``accept_len [B]``,
    ``out_tokens [B][M]`` (emitted tokens then -1 padding) and ``n_out [B]``.
    """
    logits = np.asarray(logits)
    B, M, _ = logits.shape
    am = np.zeros((B, M), dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    toks = np.full((B, M), -1, dtype=np.int32)
    n_out = np.zeros(B, dtype=np.int32)
    for b in range(B):
        y, n, emitted = accept(logits[b], np.asarray(drafts[b]).reshape(-1)[:M - 1])
        am[b] = y
        n_acc[b] = n
        toks[b, :len(emitted)] = emitted
        n_out[b] = len(emitted)
    return am, n_acc, toks, n_out


def lm_head_logits(h_bits, w_bits):
    """Logits of bf16 hidden rows through a vocab-major bf16 LM head:
    ``logit[r][v] = sum_k h[r][k] * w[v][k]`` with ``h [R][Dm]`` and
    ``w [V][Dm]`` given as bf16 bit patterns.  Products of bf16 values are
    exact in fp64 and the sum is accumulated in fp64."""
    h = bf16_to_f64(np.asarray(h_bits))
    w = bf16_to_f64(np.asarray(w_bits))
    return h @ w.T


def lm_head_argmax(h_bits, w_bits):
    """Greedy token of each hidden row ("Algoritmo Principale", steps 1 and
    3): :func:`greedy_argmax` of every row of :func:`lm_head_logits`."""
    return np.array([greedy_argmax(r) for r in lm_head_logits(h_bits, w_bits)], dtype=np.int32)


def fp32_sum_bound(h_bits, w_bits):
    """Per-row bound on how far any fp32 evaluation of a logit (exact
    products, fp32 additions in any order) can lie from the exact value:
    ``gamma_Dm * max_v sum_k |h[r][k] w[v][k]|`` with ``gamma_n = n u / (1 - n u)``
    and ``u = 2^-24`` (the standard bound for recursive summation).
    Returns ``[R]``."""
    h = np.abs(bf16_to_f64(np.asarray(h_bits)))
    w = np.abs(bf16_to_f64(np.asarray(w_bits)))
    n = h.shape[1]
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    return gamma * (h @ w.T).max(axis=1)
