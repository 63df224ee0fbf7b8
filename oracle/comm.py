"""CPU oracle for the congestion-free communication plan (test infrastructure).

TEST INFRASTRUCTURE ONLY: nothing on the product path imports or calls this module.

FCP paper Sec. 4.2, "Congestion-free solver": the block transfers among N workers form
a bipartite multigraph with send nodes S(i) and receive nodes R(j), one edge S(i)->R(j)
per block worker i must send to worker j. A sub-stage in which every worker sends at
most one block and receives at most one block is a matching of that graph (Lemma 1); a
worker of degree Delta needs at least Delta sub-stages (Lemma 2); the edges split into
Delta disjoint matchings, so Delta is the optimum. The pages defer the construction to
an appendix that is not reproduced; the colouring here is the textbook alternating-path
proof of that fact (Konig's edge-colouring theorem), which shares nothing with the
library's construction. Parity status: pinned (exhaustive search on tiny multigraphs,
the all-to-all closed form, planted invalid plans; see tests/test_comm_plan.py).
"""
from itertools import product

import numpy as np


def max_degree(n, src, dst):
    """Delta: the largest number of edges at any send or receive node."""
    src = np.asarray(src, dtype=np.int64)
    dst = np.asarray(dst, dtype=np.int64)
    if src.size == 0:
        return 0
    return int(max(np.bincount(src, minlength=n).max(), np.bincount(dst, minlength=n).max()))


def is_congestion_free(n, src, dst, stage, n_stages):
    """True when every edge has a stage in [0, n_stages) and, within each stage, no send
    node and no receive node has more than one edge (Lemma 1: each stage is a matching)."""
    src, dst, stage = (np.asarray(a, dtype=np.int64) for a in (src, dst, stage))
    if stage.shape != src.shape:
        return False
    if src.size and (stage.min() < 0 or stage.max() >= n_stages):
        return False
    seen_s, seen_r = set(), set()
    for i, j, c in zip(src.tolist(), dst.tolist(), stage.tolist()):
        if (c, i) in seen_s or (c, j) in seen_r:
            return False
        seen_s.add((c, i))
        seen_r.add((c, j))
    return True


def min_stages_brute_force(n, src, dst):
    """The fewest stages of any congestion-free plan, by trying every assignment of
    stages to edges with k = 0, 1, 2, ... stages (tiny graphs only: k ** |E| plans)."""
    e = len(src)
    if e == 0:
        return 0
    k = 1
    while True:
        for plan in product(range(k), repeat=e):
            if is_congestion_free(n, src, dst, plan, k):
                return k
        k += 1


def alternating_path_plan(n, src, dst):
    """A plan with Delta stages, edges coloured one at a time. For edge S(u)->R(v): pick
    a stage a free at S(u) and b free at R(v) (each node has fewer than Delta coloured
    edges, so both exist). If a is taken at R(v), swap a and b on the path that leaves
    R(v) by its a-edge and then alternates b, a, b, ... That path enters send nodes only
    through a-edges, and a is free at S(u), so it never reaches S(u); after the swap a
    is free at both ends of the new edge, which takes it."""
    delta = max_degree(n, src, dst)
    # at[node][c] = edge index of colour c at that node; send nodes 0..n-1, receive n..2n-1
    at = [dict() for _ in range(2 * n)]
    stage = [-1] * len(src)
    for e, (u, v) in enumerate(zip(src, dst)):
        su, rv = int(u), n + int(v)
        a = next(c for c in range(delta) if c not in at[su])
        b = next(c for c in range(delta) if c not in at[rv])
        if a in at[rv]:
            # Collect the alternating path from rv: colours a, b, a, ...
            path, node, c = [], rv, a
            while c in at[node]:
                f = at[node][c]
                path.append(f)
                other = n + int(dst[f]) if node < n else int(src[f])
                node = other
                c = b if c == a else a
            for f in path:
                fu, fv = int(src[f]), n + int(dst[f])
                del at[fu][stage[f]]
                del at[fv][stage[f]]
            for f in path:
                stage[f] = b if stage[f] == a else a
                at[int(src[f])][stage[f]] = f
                at[n + int(dst[f])][stage[f]] = f
        stage[e] = a
        at[su][a] = e
        at[rv][a] = e
    return np.asarray(stage, dtype=np.int32), delta
