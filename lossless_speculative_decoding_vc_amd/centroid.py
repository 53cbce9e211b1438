"""CentroidKV on the GPU: a compressed cache kept within a token budget by
Chunked Soft Matching rounds on the method's schedule.

"Riassunto Tecnico: CentroidKV", "Componenti Chiave": after the prefill a
first clustering round runs when the cache exceeds the budget; during
decoding the cache grows by one token per step and a round runs every ``g``
steps to keep it within the budget, sinks and recent tokens preserved (item
2); each round merges the top fraction ``r`` of the chunk matches, with ``r``
decaying linearly over rounds (item 3); centroids carry their degree across
rounds and enter the drafter's softmax with its logarithm (item 4).

Every step runs in libvc: rows enter the cache through ``vc_commit_rows``
(degree 1), rounds through ``vc_csm_round`` (into the other of two buffers,
degrees carried, the new length written on the device), and the decisions of
the schedule -- whether a round is due and its ratio -- come from
``vc_csm_round_due`` / ``vc_csm_schedule_ratio``.  The host keeps only the
token count, the same for every request and KV head (each decode step
appends one token to every request).
"""
import torch

from . import commit_rows, csm_round, csm_round_due, csm_schedule_ratio


class CentroidCache:
    """Two ping-pong caches in the drafter's dense layout (K ``[B][Hkv][cap][D]``,
    V ``[B][Hkv][cap/32][D][32]`` bf16, per-head degrees ``[B][Hkv][cap]``
    fp32) and the schedule state.  :meth:`draft_view` gives what
    ``draft_attn`` reads."""

    def __init__(self, B, Hkv, cap, budget, every, r_init, delta_r, n_sink, n_recent, chunk, D=128, device="cuda"):
        if cap % 64:
            raise ValueError("cap must be a multiple of 64 (the drafter's block)")
        self.B, self.Hkv, self.cap, self.D = B, Hkv, cap, D
        self.budget, self.every, self.r_init, self.delta_r = budget, every, r_init, delta_r
        self.n_sink, self.n_recent, self.chunk = n_sink, n_recent, chunk
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        self.k = [z((B, Hkv, cap, D), torch.bfloat16) for _ in range(2)]
        self.v = [z((B, Hkv, cap // 32, D, 32), torch.bfloat16) for _ in range(2)]
        self.deg = [z((B, Hkv, cap), torch.float32) for _ in range(2)]
        self.length = z((B, Hkv), torch.int32)        # device copy of the token count (the drafter's main_len)
        self._one = torch.ones(B, dtype=torch.int32, device=device)
        self.cur = 0
        self.n = 0        # tokens in the cache
        self.step = 0     # decode steps so far (0: after the prefill)
        self.rounds = []  # per round: decode step, index j, ratio r, n_in, n_out

    def draft_view(self):
        """``(k, v, main_len, degree)`` of the current cache."""
        return self.k[self.cur], self.v[self.cur], self.length, self.deg[self.cur]

    def prefill(self, k_rows, v_rows, stream=None):
        """Enter the prompt's rows (``k_rows [B][Hkv][n][D]``, ``v_rows
        [B][Hkv][D][n]`` bf16); the first round follows with
        :meth:`cluster_if_due` (:meth:`prefill_step` does both)."""
        n = k_rows.shape[2]
        if self.n or n > self.cap:
            raise ValueError("prefill once, into an empty cache of sufficient capacity")
        n_all = torch.full((self.B,), n, dtype=torch.int32, device=k_rows.device)
        commit_rows(k_rows, v_rows, n_all, self.k[self.cur], self.v[self.cur], self.length, degree=self.deg[self.cur],
                    v_blocked=True, stream=stream)
        self.n = n

    def prefill_step(self, k_rows, v_rows, stream=None):
        """:meth:`prefill` then :meth:`cluster_if_due`."""
        self.prefill(k_rows, v_rows, stream)
        return self.cluster_if_due(stream)

    def append(self, k_row, v_row, stream=None):
        """One decode token per request (``[B][Hkv][1][D]``, ``[B][Hkv][D][1]``);
        no round yet (see :meth:`cluster_if_due`)."""
        if self.n >= self.cap:
            raise ValueError("the cache is full")
        commit_rows(k_row, v_row, self._one, self.k[self.cur], self.v[self.cur], self.length,
                    degree=self.deg[self.cur], v_blocked=True, stream=stream)
        self.n += 1
        self.step += 1

    def cluster_if_due(self, stream=None):
        """Run a round if the schedule calls for one now; returns its record or None."""
        if not csm_round_due(self.n, self.budget, self.step, self.every):
            return None
        j = len(self.rounds)
        r = csm_schedule_ratio(self.r_init, self.delta_r, j)
        nxt = 1 - self.cur
        n_out = csm_round(self.k[self.cur], self.v[self.cur], self.n, self.n_sink, self.n_recent, self.chunk, r,
                          self.k[nxt], self.v[nxt], self.deg[nxt], in_deg=self.deg[self.cur], out_len=self.length,
                          stream=stream)
        rec = dict(step=self.step, j=j, r=r, n_in=self.n, n_out=n_out)
        self.rounds.append(rec)
        self.cur, self.n = nxt, n_out
        return rec

    def decode_step(self, k_row, v_row, stream=None):
        """:meth:`append` then :meth:`cluster_if_due`."""
        self.append(k_row, v_row, stream)
        return self.cluster_if_due(stream)
