"""Float64 CPU oracle for one worker's block-level varlen attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this
module; only the tests, the smoke check and the bench's CPU-baseline leg do. It shares
no code with the HIP library or its Python binding and never reads a block-pair table:
it works per sequence from token positions.

What it computes (FCP paper Sec. 2.2; the equation is only legible on the review page,
section "核心公式与建模"): for every sequence, query head h and owned query at
in-sequence position i,

    S_ij = (q_i . k_j) * scale,       scale = 1/sqrt(D) unless given,
    LSE_i = ln sum_{j in V(i)} exp(S_ij),
    O_i = sum_{j in V(i)} exp(S_ij - LSE_i) v_j,

with V(i) = {0..i} for the causal mask and {0..L-1} otherwise, keys of the same sequence
only. Readings of the pages used here (the pages are silent or garbled on each):
  * the mask multiplies nothing: masked keys are left out of the softmax;
  * query head h reads KV head h // (Hq / Hkv) (contiguous groups);
  * LSE is a natural logarithm;
  * a query with no visible key has O = 0 and LSE = -inf;
  * partials over disjoint key subsets combine by the LSE-weighted sum (the pages state
    only that per-slice results reduce to the final output, FCP paper Sec. 2.2);
  * the backward is the exact gradient of sum_i <dO_i, O_i> over the owned rows (the
    paper says a backward exists, Sec. 2.2, but does not give it).

Inputs are the bf16 arrays the GPU receives, widened exactly to float64. Matrix
products over key chunks are the only library primitive used.
"""
import numpy as np


def _scale(d, scale):
    return float(scale) if scale else 1.0 / np.sqrt(d)


class SeqIndex:
    """Where each sequence's tokens sit: owned query rows with their positions, and the
    KV buffer row of every key position that is present (-1 where absent)."""

    def __init__(self, wl):
        self.causal = wl.causal
        self.seqlens = list(wl.seqlens)
        self.hq, self.hkv, self.d = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
        self.q_row_seq = np.full(wl.q_rows, -1, dtype=np.int64)
        self.q_row_pos = np.full(wl.q_rows, -1, dtype=np.int64)
        for s in wl.q_segments():
            self.q_row_seq[s.row0:s.row0 + s.length] = s.seq
            self.q_row_pos[s.row0:s.row0 + s.length] = np.arange(s.pos0, s.pos0 + s.length)
        self.kv_row_of_pos = {}
        for s in wl.kv_segments():
            m = self.kv_row_of_pos.setdefault(
                s.seq, np.full(self.seqlens[s.seq], -1, dtype=np.int64))
            m[s.pos0:s.pos0 + s.length] = np.arange(s.row0, s.row0 + s.length)

    def owned_rows(self):
        return np.nonzero(self.q_row_seq >= 0)[0]

    def visible_key_rows(self, seq, max_pos):
        """KV rows of key positions 0..max_pos (causal) or the whole sequence."""
        n = (max_pos + 1) if self.causal else self.seqlens[seq]
        rows = self.kv_row_of_pos[seq][:n]
        if (rows < 0).any():
            raise ValueError("sequence %d: a visible key is missing from the KV buffer" % seq)
        return rows


def _chunk(n_keys):
    return max(1, (1 << 22) // max(1, n_keys))


def forward(qf, kf, vf, idx, scale=None, rows=None, heads=None):
    """O [len(rows), len(heads), D] and LSE [len(rows), len(heads)] in float64."""
    rows = idx.owned_rows() if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(idx.hq)) if heads is None else list(heads)
    group = idx.hq // idx.hkv
    sc = _scale(idx.d, scale)
    out_o = np.zeros((len(rows), len(heads), idx.d))
    out_l = np.full((len(rows), len(heads)), -np.inf)
    seqs = idx.q_row_seq[rows]
    for s in np.unique(seqs):
        sel = np.nonzero(seqs == s)[0]
        pos = idx.q_row_pos[rows[sel]]
        krows = idx.visible_key_rows(s, pos.max())
        kpos = np.arange(len(krows))
        step = _chunk(len(krows))
        for a in range(0, len(sel), step):
            c = sel[a:a + step]
            qp = pos[a:a + step]
            mask = (kpos[None, :] <= qp[:, None]) if idx.causal else None
            for hi, h in enumerate(heads):
                g = h // group
                smat = (qf[rows[c], h] @ kf[krows, g].T) * sc
                if mask is not None:
                    smat = np.where(mask, smat, -np.inf)
                m = smat.max(axis=1, keepdims=True)
                lse = m[:, 0] + np.log(np.exp(smat - m).sum(axis=1))
                p = np.exp(smat - lse[:, None])
                out_o[c, hi] = p @ vf[krows, g]
                out_l[c, hi] = lse
    return out_o, out_l


def partial(qf, kf, vf, q_rows, q_pos, kv_rows, kv_pos, causal, hq, hkv, scale=None,
            heads=None):
    """One partial: the queries at ``q_rows`` (in-sequence positions ``q_pos``) attend
    only to the keys at ``kv_rows`` (positions ``kv_pos``) of the same sequence; under the
    causal mask a key is visible iff its position is <= the query's. Rows with no visible
    key get O = 0, LSE = -inf."""
    q_rows, q_pos = np.asarray(q_rows), np.asarray(q_pos)
    kv_rows, kv_pos = np.asarray(kv_rows), np.asarray(kv_pos)
    heads = list(range(hq)) if heads is None else list(heads)
    group = hq // hkv
    d = qf.shape[-1]
    sc = _scale(d, scale)
    out_o = np.zeros((len(q_rows), len(heads), d))
    out_l = np.full((len(q_rows), len(heads)), -np.inf)
    vis = (kv_pos[None, :] <= q_pos[:, None]) if causal else \
        np.ones((len(q_rows), len(kv_rows)), dtype=bool)
    live = vis.any(axis=1)
    for hi, h in enumerate(heads):
        g = h // group
        smat = np.where(vis, (qf[q_rows, h] @ kf[kv_rows, g].T) * sc, -np.inf)
        smat = smat[live]
        m = smat.max(axis=1, keepdims=True)
        lse = m[:, 0] + np.log(np.exp(smat - m).sum(axis=1))
        p = np.exp(smat - lse[:, None])
        out_o[live, hi] = p @ vf[kv_rows, g]
        out_l[live, hi] = lse
    return out_o, out_l


def merge(lses, outs):
    """Combine partials over disjoint key subsets: LSE = ln sum_i exp(LSE_i),
    O = sum_i exp(LSE_i - LSE) O_i. All-empty rows stay (O = 0, LSE = -inf)."""
    lse = np.stack([np.asarray(x, dtype=np.float64) for x in lses])
    o = np.stack([np.asarray(x, dtype=np.float64) for x in outs])
    m = lse.max(axis=0)
    empty = np.isneginf(m)
    msafe = np.where(empty, 0.0, m)
    w = np.exp(lse - msafe[None])
    tot = w.sum(axis=0)
    out_lse = np.where(empty, -np.inf, msafe + np.log(np.where(empty, 1.0, tot)))
    wn = w / np.where(empty, 1.0, tot)[None]
    out_o = (wn[..., None] * o).sum(axis=0)
    return out_o, out_lse


def backward(qf, kf, vf, dof, idx, scale=None, seqs=None, heads=None):
    """Exact gradients of sum_i <dO_i, O_i> over the owned query rows of the chosen
    sequences (all by default) and query heads (all by default; with a subset, dK and dV
    sum over those heads only). Returns dQ [q_rows, Hq, D], dK and dV [kv_rows, Hkv, D]
    (zeros outside those sequences and heads)."""
    heads = list(range(idx.hq)) if heads is None else list(heads)
    group = idx.hq // idx.hkv
    sc = _scale(idx.d, scale)
    dq = np.zeros(qf.shape)
    dk = np.zeros(kf.shape)
    dv = np.zeros(vf.shape)
    rows = idx.owned_rows()
    rseq = idx.q_row_seq[rows]
    for s in np.unique(rseq):
        if seqs is not None and s not in seqs:
            continue
        r = rows[rseq == s]
        pos = idx.q_row_pos[r]
        krows = idx.visible_key_rows(s, pos.max())
        kpos = np.arange(len(krows))
        step = _chunk(len(krows))
        for a in range(0, len(r), step):
            rc, qp = r[a:a + step], pos[a:a + step]
            mask = (kpos[None, :] <= qp[:, None]) if idx.causal else None
            for h in heads:
                g = h // group
                kk, vv = kf[krows, g], vf[krows, g]
                smat = (qf[rc, h] @ kk.T) * sc
                if mask is not None:
                    smat = np.where(mask, smat, -np.inf)
                m = smat.max(axis=1, keepdims=True)
                lse = m[:, 0] + np.log(np.exp(smat - m).sum(axis=1))
                p = np.exp(smat - lse[:, None])
                o = p @ vv
                dout = dof[rc, h]
                delta = (dout * o).sum(axis=1)
                dp = dout @ vv.T
                ds = p * (dp - delta[:, None])
                dq[rc, h] += (ds @ kk) * sc
                np.add.at(dk[:, g], krows, (ds.T @ qf[rc, h]) * sc)
                np.add.at(dv[:, g], krows, p.T @ dout)
    return dq, dk, dv


def dq_rows(qf, kf, vf, dof, idx, rows, scale=None):
    """dQ for the given owned query rows only (each row's gradient needs only its own
    forward). Returns [len(rows), Hq, D]."""
    rows = np.asarray(rows, dtype=np.int64)
    group = idx.hq // idx.hkv
    sc = _scale(idx.d, scale)
    out = np.zeros((len(rows), idx.hq, idx.d))
    seqs = idx.q_row_seq[rows]
    for s in np.unique(seqs):
        sel = np.nonzero(seqs == s)[0]
        pos = idx.q_row_pos[rows[sel]]
        krows = idx.visible_key_rows(s, pos.max())
        kpos = np.arange(len(krows))
        step = _chunk(len(krows))
        for a in range(0, len(sel), step):
            c, qp = sel[a:a + step], pos[a:a + step]
            mask = (kpos[None, :] <= qp[:, None]) if idx.causal else None
            for h in range(idx.hq):
                g = h // group
                kk, vv = kf[krows, g], vf[krows, g]
                smat = (qf[rows[c], h] @ kk.T) * sc
                if mask is not None:
                    smat = np.where(mask, smat, -np.inf)
                m = smat.max(axis=1, keepdims=True)
                lse = m[:, 0] + np.log(np.exp(smat - m).sum(axis=1))
                p = np.exp(smat - lse[:, None])
                dout = dof[rows[c], h]
                delta = (dout * (p @ vv)).sum(axis=1)
                ds = p * (dout @ vv.T - delta[:, None])
                out[c, h] = (ds @ kk) * sc
    return out


def dkv_rows(qf, kf, vf, dof, idx, kv_rows, scale=None):
    """dK and dV for the given KV rows only: each key's gradient sums over the owned
    queries of its sequence that see it, and each such query needs its own full forward
    (LSE, O, Delta). Returns (dK, dV), each [len(kv_rows), Hkv, D]."""
    kv_rows = np.asarray(kv_rows, dtype=np.int64)
    group = idx.hq // idx.hkv
    sc = _scale(idx.d, scale)
    dk = np.zeros((len(kv_rows), idx.hkv, idx.d))
    dv = np.zeros((len(kv_rows), idx.hkv, idx.d))
    pos_of = {}
    for s, m in idx.kv_row_of_pos.items():
        for p in np.nonzero(m >= 0)[0]:
            pos_of[int(m[p])] = (s, int(p))
    rows = idx.owned_rows()
    for ki, kr in enumerate(kv_rows):
        s, kp = pos_of[int(kr)]
        qsel = rows[(idx.q_row_seq[rows] == s) &
                    ((idx.q_row_pos[rows] >= kp) if idx.causal else True)]
        if len(qsel) == 0:
            continue
        pos = idx.q_row_pos[qsel]
        krows = idx.visible_key_rows(s, pos.max())
        kpos = np.arange(len(krows))
        step = _chunk(len(krows))
        for a in range(0, len(qsel), step):
            rc, qp = qsel[a:a + step], pos[a:a + step]
            mask = (kpos[None, :] <= qp[:, None]) if idx.causal else None
            for h in range(idx.hq):
                g = h // group
                kk, vv = kf[krows, g], vf[krows, g]
                smat = (qf[rc, h] @ kk.T) * sc
                if mask is not None:
                    smat = np.where(mask, smat, -np.inf)
                m = smat.max(axis=1, keepdims=True)
                lse = m[:, 0] + np.log(np.exp(smat - m).sum(axis=1))
                p = np.exp(smat[:, kp] - lse)
                dout = dof[rc, h]
                delta = (dout * (np.exp(smat - lse[:, None]) @ vv)).sum(axis=1)
                ds = p * (dout @ vf[kr, g] - delta)
                dk[ki, g] += (ds @ qf[rc, h]) * sc
                dv[ki, g] += p @ dout
    return dk, dv


def dkv_keys(qf, kf, vf, dof, idx, kv_rows, heads=None, scale=None):
    """dK and dV at the given KV rows, from the query heads in ``heads`` (all by default):
    for every sequence holding one of the rows, each owned query of that sequence is run
    forward once (its LSE, O and Delta over all of its visible keys), and only the
    requested keys' columns of P and dS are kept. A KV head's rows are exact when
    ``heads`` holds its whole query-head group (or when dO is zero on the other heads of
    the group). Returns (dK, dV), each [len(kv_rows), Hkv, D]."""
    kv_rows = np.asarray(kv_rows, dtype=np.int64)
    heads = list(range(idx.hq)) if heads is None else list(heads)
    group = idx.hq // idx.hkv
    sc = _scale(idx.d, scale)
    dk = np.zeros((len(kv_rows), idx.hkv, idx.d))
    dv = np.zeros((len(kv_rows), idx.hkv, idx.d))
    where = {}
    for s, m in idx.kv_row_of_pos.items():
        for p in np.nonzero(np.isin(m, kv_rows))[0]:
            for ki in np.nonzero(kv_rows == m[p])[0]:
                where.setdefault(s, []).append((int(ki), int(p)))
    rows = idx.owned_rows()
    for s, sel in where.items():
        kis = np.array([a for a, _ in sel])
        kps = np.array([b for _, b in sel])
        r = rows[idx.q_row_seq[rows] == s]
        if len(r) == 0:
            continue
        pos = idx.q_row_pos[r]
        krows = idx.visible_key_rows(s, pos.max())
        kpos = np.arange(len(krows))
        step = _chunk(len(krows))
        for a in range(0, len(r), step):
            rc, qp = r[a:a + step], pos[a:a + step]
            mask = (kpos[None, :] <= qp[:, None]) if idx.causal else None
            for h in heads:
                g = h // group
                kk, vv = kf[krows, g], vf[krows, g]
                smat = (qf[rc, h] @ kk.T) * sc
                if mask is not None:
                    smat = np.where(mask, smat, -np.inf)
                m = smat.max(axis=1, keepdims=True)
                lse = m[:, 0] + np.log(np.exp(smat - m).sum(axis=1))
                p = np.exp(smat - lse[:, None])
                dout = dof[rc, h]
                delta = (dout * (p @ vv)).sum(axis=1)
                # columns of the requested keys (keys past a query's position have P = 0)
                inside = kps < len(krows)
                cols = np.where(inside, kps, 0)
                psel = np.where(inside[None, :], p[:, cols], 0.0)
                ds = psel * (dout @ vv[cols].T - delta[:, None])
                dk[kis, g] += (ds.T @ qf[rc, h]) * sc
                dv[kis, g] += psel.T @ dout
    return dk, dv
