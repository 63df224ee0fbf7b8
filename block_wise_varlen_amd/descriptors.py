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
import numpy as np

PAIR_FIELDS = ("seq_id", "q_start", "q_len", "kv_start", "kv_len", "mask_offset",
               "out_row", "flags")
PAIR_DTYPE = np.dtype([(f, np.int32) for f in PAIR_FIELDS])
FLAG_CAUSAL = 1


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
