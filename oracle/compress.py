"""Token-eviction compaction of a KV cache.

Test infrastructure only (see :mod:`oracle`).

"Riepilogo Tecnico: VeriCache", section "Supporto Architetturale": an
eviction policy is one of the compressors behind the drafter's uniform
interface; it keeps a subset of the tokens, and the drafter attends over the
full cache restricted to them.  The kept set is per token, shared by the KV
heads of a request; keys stay where the full cache put them (after RoPE).

Parity: pinned by the masked-attention identity (attention over the compacted
cache equals attention over the full cache with the evicted tokens' scores
sent to minus infinity), by the identity selection and by the duplicate-index
case (a token kept twice counts twice, like a degree of 2).
"""
import numpy as np


def compact_kv(k, v, idx):
    """Rows ``idx`` of a cache.

    ``k, v [..., N, D]`` (both token-major), ``idx`` integer ``[n]``.  Returns
    ``(k_c, v_c) [..., n, D]`` with row j equal to row ``idx[j]`` of the source;
    an index outside ``[0, N)`` gives a zero row.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    idx = np.asarray(idx, dtype=np.int64)
    N = k.shape[-2]
    ok = (idx >= 0) & (idx < N)
    safe = np.where(ok, idx, 0)
    k_c = np.where(ok[:, None], np.take(k, safe, axis=-2), 0)
    v_c = np.where(ok[:, None], np.take(v, safe, axis=-2), 0)
    return k_c.astype(k.dtype), v_c.astype(v.dtype)
