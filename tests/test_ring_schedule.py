"""The verify kernels' LDS ring protocols, checked on a model.

In both verify kernels the two wave groups of a workgroup (waves 0-3 and
4-7) run the same cluster sequence one cluster apart, a workgroup barrier
after every cluster.  Each wave issues its own share of every K/V tile's
direct global->LDS loads into a ring of LDS stages and waits for its own
loads with `s_waitcnt vmcnt(n)` (loads complete in order).  This model
lists, per group, the clusters of the main loop as pp_rows writes them
(issues, waits, LDS reads of a tile) and checks, for every tile count, that:

  * both groups pass the same number of barriers;
  * every tile is issued by both groups in the same phase;
  * no tile is read before every wave has waited for its own loads of it in
    an earlier phase (the barrier between publishes the data);
  * no stage is refilled while the tile it held may still be read (all reads
    of the tile a ring length earlier lie in phases before the issue);
  * every `vmcnt` allowance leaves exactly the tiles issued after the one
    waited for, so the wait is neither short nor draining the ring.

The token split (verify_ts) has five stages and two clusters per tile; the
row split (verify_pp) four stages and four clusters per tile (two 32-token
halves, each an MFMA and a VALU cluster).  A change to either kernel's
schedule must be mirrored here.
"""
import pytest

STAGES = 5        # token split
STAGES_ROW = 4    # row split


def group_clusters(g, T):
    """Clusters of wave group g over T full tiles; each cluster ends at a barrier.

    Actions: ('issue', u), ('wait', u, n) = wait until tile u has landed with
    n tiles allowed to stay in flight, ('read', u).
    """
    cl = []
    # prologue: tiles 0..2, wait for tile 0, __syncthreads
    cl.append([("issue", u) for u in range(min(3, T))] + [("wait", 0, min(T - 1, 2))])
    if g == 1:   # phase 0: group 1's cluster "V_-1"
        cl.append([("issue", 3)] if 3 < T else [])
    c = []   # M_0: K operands and S of tile 0
    if g == 0 and 3 < T:
        c.append(("issue", 3))
    c.append(("read", 0))
    if g == 1 and 1 < T:
        c.append(("wait", 1, min(2, T - 2)))
    cl.append(c)
    for t in range(T):
        c = []   # V_t: P of tile t
        if g == 1 and t + 4 < T:
            c.append(("issue", t + 4))
        if g == 0 and t + 1 < T:
            c.append(("wait", t + 1, min(2, T - 2 - t)))
        cl.append(c)
        c = []   # M_t+1: V operands and PV of tile t, K operands (and S) of tile t+1
        if g == 0 and t + 4 < T:
            c.append(("issue", t + 4))
        c.append(("read", t))
        c.append(("read", min(t + 1, T - 1)))
        if g == 1 and t + 2 < T:
            c.append(("wait", t + 2, min(2, T - 3 - t)))
        cl.append(c)
    if g == 0:
        cl.append([])
    return cl


def row_split_clusters(g, T):
    """Clusters of wave group g in verify_pp over T full tiles (same actions)."""
    cl = [[("issue", u) for u in range(min(3, T))] + [("wait", 0, min(T - 1, 2))]]
    if g == 1:   # group 1 reads tile 0's K operands, then its leading barrier
        cl.append([("read", 0)])
        first = []
    else:
        first = [("read", 0)]
    c = first   # M_0: V operands and S of half 0 of tile 0
    if g == 1 and 3 < T:
        c.append(("issue", 3))
    c.append(("read", 0))
    cl.append(c)
    for t in range(T):
        sn = min(t + 1, T - 1)
        c = []   # V_2t: P of half 0; K operands of half 1
        if g == 0 and t + 3 < T:
            c.append(("issue", t + 3))
        c.append(("read", t))
        if g == 1 and t + 1 < T:
            c.append(("wait", t + 1, min(2, T - 2 - t)))
        cl.append(c)
        c = [("read", t)]   # M_2t+1: PV of half 0; V operands and S of half 1
        if g == 0 and t + 1 < T:
            c.append(("wait", t + 1, min(2, T - 2 - t)))
        cl.append(c)
        cl.append([("read", sn)])   # V_2t+1: P of half 1; K operands of tile t+1
        c = []   # M_2t+2: PV of half 1; V operands and S of tile t+1
        if g == 1 and t + 4 < T:
            c.append(("issue", t + 4))
        c.append(("read", sn))
        cl.append(c)
    if g == 0:
        cl.append([])
    return cl


def check(T, model=None, stages=STAGES):
    model = model or group_clusters
    clusters = {g: model(g, T) for g in (0, 1)}
    assert len(clusters[0]) == len(clusters[1]), "barrier counts differ"
    issue_phase, reads, waited = {}, {}, {0: {}, 1: {}}
    for g in (0, 1):
        issued = []
        for phase, actions in enumerate(clusters[g]):
            for a in actions:
                if a[0] == "issue":
                    issued.append(a[1])
                    issue_phase.setdefault(a[1], set()).add(phase)
                elif a[0] == "read":
                    reads.setdefault(a[1], []).append(phase)
                else:
                    _, u, n = a
                    # exact allowance: the tiles issued after u are the ones left in flight
                    assert u in issued and len(issued) - 1 - issued.index(u) == n, (T, g, phase, u, n, issued)
                    for v in issued[:issued.index(u) + 1]:
                        waited[g].setdefault(v, phase)
    for u in range(T):
        assert len(issue_phase.get(u, ())) == 1, (T, u, issue_phase.get(u))
        p_issue = next(iter(issue_phase[u]))
        for p_read in reads.get(u, []):
            for g in (0, 1):
                assert u in waited[g] and waited[g][u] < p_read, (T, "read before wait", u, g, p_read)
        if u >= stages:
            assert max(reads[u - stages]) < p_issue, (T, "stage refilled while read", u)


@pytest.mark.parametrize("T", range(1, 40))
def test_token_split_ring(T):
    check(T)


@pytest.mark.parametrize("T", range(1, 40))
def test_row_split_ring(T):
    check(T, row_split_clusters, STAGES_ROW)


def test_a_short_ring_is_caught():
    # the same row-split schedule over three stages would refill a stage still being read
    with pytest.raises(AssertionError):
        check(12, row_split_clusters, 3)


def test_a_short_allowance_is_caught():
    # the check is not vacuous: allowing one tile too many in flight fails
    orig = group_clusters

    def wrong(g, T):
        cl = orig(g, T)
        return [[(a[0], a[1], a[2] + 1) if a[0] == "wait" and a[2] < 2 else a for a in c] for c in cl]

    globals()["group_clusters"] = wrong
    try:
        with pytest.raises(AssertionError):
            check(8)
    finally:
        globals()["group_clusters"] = orig
