"""Block-pair descriptor builder (host side of the block-level varlen path).

Turns one worker's share -- its Q blocks and the KV blocks it computes against, each a
list of placed sequence segments -- into the table of block pairs the library consumes.
One pair is emitted per (Q segment, KV segment run) of the same sequence that the mask
needs: every key run for the non-causal mask, key runs starting at or before the last
query position for the causal mask (FCP paper Sec. 2.2: causal and non-causal masks;
Sec. 4.1: short sequences are packed into blocks and computed through the kernel's
variable-length interface, so a block holds several segments and pairs never cross
sequences). KV blocks are taken ``coalesce`` at a time; within a group, runs that are
contiguous both in position and in buffer rows become one KV range (the bottom-up
coalescer of FCP paper Sec. 4.2 decouples scheduling blocks from execution blocks).

Causal masking is encoded per pair as ``mask_offset = q_pos0 - kv_pos0``: key j of the
pair (0-based within its KV range) is visible to query i iff ``j - i <= mask_offset``.
Under the causal mask a KV range is trimmed so that it ends at the pair's last query
position; keys past it are invisible to every query of the pair.
"""
from collections import namedtuple

import numpy as np

PAIR_FIELDS = ("seq_id", "q_start", "q_len", "kv_start", "kv_len", "mask_offset",
               "out_row", "flags")
PAIR_DTYPE = np.dtype([(f, np.int32) for f in PAIR_FIELDS])
FLAG_CAUSAL = 1
# Pipeline tables (fcp_copy_t, fcp_stage_t).
COPY_DTYPE = np.dtype([("src_row", np.int64), ("dst_row", np.int64), ("n_rows", np.int64)])
STAGE_DTYPE = np.dtype([("n_copies", np.int32), ("n_pairs", np.int32)])


def _runs(segs):
    """Merge segments that continue each other in position and in buffer row."""
    out = []
    for s in segs:
        if out:
            seq, p0, n, r0 = out[-1]
            if s.seq == seq and s.pos0 == p0 + n and s.row0 == r0 + n:
                out[-1] = (seq, p0, n + s.length, r0)
                continue
        out.append((s.seq, s.pos0, s.length, s.row0))
    return out


def build_pairs(wl, coalesce=None, kv_split=None) -> np.ndarray:
    """Pairs for workload ``wl`` as a structured int32 array (``PAIR_DTYPE``).

    ``out_row`` numbers the partial-output rows: each pair owns ``q_len`` consecutive
    rows starting there, in table order. ``kv_split`` > 1 cuts every KV range into that
    many consecutive parts (part i starts at floor(i*kv_len/k)), each its own pair.
    """
    c = wl.coalesce if coalesce is None else coalesce
    k = wl.kv_split if kv_split is None else kv_split
    causal = wl.causal
    groups = [wl.kv_blocks[i:i + c] for i in range(0, len(wl.kv_blocks), c)]
    rows = []
    for qb in wl.q_blocks:
        for qs in qb:
            q_last = qs.pos0 + qs.length - 1
            for grp in groups:
                segs = [s for blk in grp for s in blk
                        if s.seq == qs.seq and (not causal or s.pos0 <= q_last)]
                for seq, p0, n, r0 in _runs(segs):
                    if causal:
                        n = min(n, q_last - p0 + 1)
                    for i in range(k):
                        a, b = (i * n) // k, ((i + 1) * n) // k
                        if b > a:
                            rows.append((seq, qs.row0, qs.length, r0 + a, b - a,
                                         qs.pos0 - (p0 + a), 0,
                                         FLAG_CAUSAL if causal else 0))
    pairs = np.array(rows, dtype=PAIR_DTYPE) if rows else np.zeros(0, PAIR_DTYPE)
    if len(pairs):
        pairs["out_row"] = np.concatenate([[0], np.cumsum(pairs["q_len"])[:-1]])
    return pairs


def part_rows(pairs) -> int:
    """Rows of the per-pair partial buffers."""
    return int(pairs["q_len"].sum()) if len(pairs) else 0


def visible_pairs_of(pairs) -> int:
    """Visible (query, key) pairs covered by a pair table, per head: each pair counts
    its own unmasked (i, j) with j - i <= mask_offset (causal) or q_len*kv_len."""
    total = 0
    for p in pairs:
        nq, nk, off = int(p["q_len"]), int(p["kv_len"]), int(p["mask_offset"])
        if not (p["flags"] & FLAG_CAUSAL):
            total += nq * nk
            continue
        # keys 0..min(nk-1, i+off) for each query i
        i = np.arange(nq, dtype=np.int64)
        total += int(np.clip(i + off + 1, 0, nk).sum())
    return total


_Seg = namedtuple("_Seg", "seq pos0 length row0")


def _stage_pairs(wl, kv_segs, rows):
    """Pairs of every Q segment of ``wl`` against the KV segments ``kv_segs`` (placed, in
    buffer-row order). Under the causal mask a segment that lies wholly at or before the
    query segment's first position is visible to all its queries; such segments of one
    sequence that are contiguous in buffer rows form one unmasked KV range whatever their
    positions (the coalescer's larger execution block, FCP paper Sec. 4.2). Segments that
    cross the diagonal keep a causal pair each, trimmed as in ``build_pairs``."""
    causal = wl.causal
    for qb in wl.q_blocks:
        for qs in qb:
            q_last = qs.pos0 + qs.length - 1
            full = []
            for s in kv_segs:
                if s.seq != qs.seq or (causal and s.pos0 > q_last):
                    continue
                if not causal or s.pos0 + s.length - 1 <= qs.pos0:
                    if full and full[-1][0] + full[-1][1] == s.row0:
                        full[-1][1] += s.length
                    else:
                        full.append([s.row0, s.length])
                else:
                    n = min(s.length, q_last - s.pos0 + 1)
                    rows.append((qs.seq, qs.row0, qs.length, s.row0, n, qs.pos0 - s.pos0, 0,
                                 FLAG_CAUSAL))
            for r0, n in full:
                rows.append((qs.seq, qs.row0, qs.length, r0, n, 0, 0, 0))


def build_pipeline(wl, local_ids, recv_stage, coalesce=1, depth=3):
    """Tables for ``fcp_pipeline_fwd`` (FCP paper Sec. 4.2: block-level pipelining,
    congestion-free sub-stages, bottom-up coalescing).

    ``wl`` is the worker's share with every KV block placed in a source buffer (its
    ``row0`` values index k_src / v_src). ``local_ids`` are the ids of the blocks the
    worker holds itself; every other KV block of ``wl`` is pulled, in the sub-stage
    ``recv_stage[block id]`` (e.g. from ``fcp_comm_plan``). Sub-stages are coalesced
    ``coalesce`` at a time (coarse stage = sub-stage // coalesce); coarse stages in which
    the worker receives nothing are skipped. Stage 0 computes the local blocks; stage
    t >= 1 copies the blocks of the t-th non-empty coarse stage into a buffer region and
    computes against them. ``depth`` regions are reused in turn (2: double buffering; 3:
    a copy may start one stage earlier; None: one region per stage, nothing reused);
    pass the returned ``depth`` to ``fcp_pipeline_fwd``.

    The worker's KV buffer holds the local blocks first, then the regions. Returns a dict
    with ``stages``, ``copies`` and ``pairs`` (out_row numbered in table order),
    ``local_copies`` (where the local blocks go in the worker's KV buffer, which the
    caller fills before the call: they are the worker's own data, not pulled),
    ``kv_rows`` (rows of the worker's KV buffer), ``part_rows`` and ``pulled`` (block ids
    per stage)."""
    ids = list(wl.kv_block_ids)
    by_id = dict(zip(ids, wl.kv_blocks))
    local = [i for i in ids if i in set(local_ids)]
    pulled = [i for i in ids if i not in set(local_ids)]
    coarse = {}
    for i in pulled:
        coarse.setdefault(int(recv_stage[i]) // coalesce, []).append(i)
    groups = [sorted(coarse[k], key=lambda i: (int(recv_stage[i]), i)) for k in sorted(coarse)]
    block_rows = lambda i: sum(s.length for s in by_id[i])
    region = max([sum(block_rows(i) for i in g) for g in groups], default=0)
    n_regions = len(groups) if depth is None else min(depth, len(groups))

    def placed(blocks_, row):
        """Segments of ``blocks_`` laid out from ``row``, and one copy per block (merged
        when consecutive in both buffers): a block's segments sit back to back in the
        source buffer."""
        segs, cps = [], []
        for i in blocks_:
            src0, n = by_id[i][0].row0, block_rows(i)
            if cps and cps[-1][0] + cps[-1][2] == src0 and cps[-1][1] + cps[-1][2] == row:
                cps[-1][2] += n
            else:
                cps.append([src0, row, n])
            for s in by_id[i]:
                segs.append(_Seg(s.seq, s.pos0, s.length, row + s.row0 - src0))
            row += n
        return segs, cps, row

    rows, stages, copies = [], [], []
    local_segs, local_cps, base = placed(local, 0)
    _stage_pairs(wl, local_segs, rows)
    stages.append((0, len(rows)))
    for t, g in enumerate(groups):
        segs, cps, _ = placed(g, base + (t % n_regions) * region)
        n_before = len(rows)
        copies += [tuple(c) for c in cps]
        _stage_pairs(wl, segs, rows)
        stages.append((len(cps), len(rows) - n_before))
    pairs = np.array(rows, dtype=PAIR_DTYPE) if rows else np.zeros(0, PAIR_DTYPE)
    if len(pairs):
        pairs["out_row"] = np.concatenate([[0], np.cumsum(pairs["q_len"])[:-1]])
    table = lambda c: np.array([tuple(x) for x in c], dtype=COPY_DTYPE) if c else \
        np.zeros(0, COPY_DTYPE)
    return {"stages": np.array(stages, dtype=STAGE_DTYPE), "copies": table(copies),
            "local_copies": table(local_cps),
            "pairs": pairs, "kv_rows": base + n_regions * region, "part_rows": part_rows(pairs),
            "depth": max(1, n_regions),
            "pulled": [local] + groups}
