"""Scalar brute-force attention for tiny inputs: the definition written as plain loops.

Independent of the oracle: it walks the workload's segment lists directly, enumerates
every (query, key) token pair, tests same-sequence and the causal condition on
in-sequence positions, and sums with math.fsum. No max-shift trick beyond what exact
float64 needs, no masking by -inf, no matrices.
"""
import math


def _tokens(blocks):
    """[(buffer row, seq, pos)] for every token of the given placed blocks."""
    out = []
    for blk in blocks:
        for s in blk:
            for t in range(s.length):
                out.append((s.row0 + t, s.seq, s.pos0 + t))
    return out


def attention(q, k, v, wl, scale=None):
    """Returns {(row, head): (O list, LSE)} for every owned query row and head.
    q, k, v are nested float arrays indexed [row][head][d] (numpy float64 works)."""
    d = wl.head_dim
    sc = scale if scale else 1.0 / math.sqrt(d)
    group = wl.num_q_heads // wl.num_kv_heads
    keys = _tokens(wl.kv_blocks)
    out = {}
    for (qr, qs, qp) in _tokens(wl.q_blocks):
        for h in range(wl.num_q_heads):
            g = h // group
            scores, vis = [], []
            for (kr, ks, kp) in keys:
                if ks != qs:
                    continue
                if wl.causal and kp > qp:
                    continue
                scores.append(math.fsum(float(q[qr][h][e]) * float(k[kr][g][e])
                                        for e in range(d)) * sc)
                vis.append(kr)
            if not scores:
                out[(qr, h)] = ([0.0] * d, -math.inf)
                continue
            top = max(scores)
            z = math.fsum(math.exp(s - top) for s in scores)
            lse = top + math.log(z)
            o = [math.fsum(math.exp(s - lse) * float(v[kr][g][e])
                           for s, kr in zip(scores, vis)) for e in range(d)]
            out[(qr, h)] = (o, lse)
    return out
