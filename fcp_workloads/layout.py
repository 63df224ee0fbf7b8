"""Blocks, buffers and one worker's share of a batch.

A block is a list of segments; a segment is a run of consecutive tokens of one sequence.
Blocks are fixed-size slices of the token stream or of single sequences (FCP paper
Sec. 4.1, "Sharding Policy"). A worker's Q blocks and the KV blocks it computes against
(its own or pulled, FCP paper Sec. 2.2 and Sec. 4.2) are laid out back to back in a Q
buffer and a KV buffer; a segment's ``row0`` is the buffer row of its first token.
"""
from dataclasses import dataclass, field
import heapq


@dataclass(frozen=True)
class Seg:
    seq: int      # sequence id
    pos0: int     # in-sequence position of the first token
    length: int   # number of tokens
    row0: int = -1  # first row in the buffer that holds this segment (-1: not placed)


@dataclass
class Workload:
    """One worker's share: its Q blocks and the KV blocks it attends to.

    ``q_blocks[i]`` / ``kv_blocks[j]`` are lists of placed segments (row0 set). The KV
    blocks are in buffer order; bottom-up coalescing (FCP paper Sec. 4.2) groups
    ``coalesce`` consecutive KV blocks. ``kv_split`` > 1 splits every KV range of a
    block pair into that many partials (used to exercise the partial merge).
    """
    name: str
    seqlens: list
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    causal: bool
    q_blocks: list
    kv_blocks: list
    q_block_ids: list
    kv_block_ids: list
    coalesce: int = 1
    kv_split: int = 1
    rng: str = "host"
    meta: dict = field(default_factory=dict)

    @property
    def q_rows(self) -> int:
        return sum(s.length for b in self.q_blocks for s in b)

    @property
    def kv_rows(self) -> int:
        return sum(s.length for b in self.kv_blocks for s in b)

    def q_segments(self):
        return [s for b in self.q_blocks for s in b]

    def kv_segments(self):
        return [s for b in self.kv_blocks for s in b]


def pack_stream(seqlens, b):
    """Concatenate the sequences into one token stream and cut it every ``b`` tokens."""
    blocks, cur, fill = [], [], 0
    for s, length in enumerate(seqlens):
        pos = 0
        while pos < length:
            take = min(length - pos, b - fill)
            cur.append(Seg(s, pos, take))
            pos += take
            fill += take
            if fill == b:
                blocks.append(cur)
                cur, fill = [], 0
    if cur:
        blocks.append(cur)
    return blocks


def shard_ffd(seqlens, b):
    """Cut every sequence into ``b``-token blocks; pack the tails and the short sequences
    first-fit-decreasing into as few ``b``-token blocks as FFD finds.

    Full blocks come first (sequence order, then block order), then the packed blocks in
    the order FFD opens them.
    """
    full, pieces = [], []
    for s, length in enumerate(seqlens):
        nfull = length // b
        for i in range(nfull):
            full.append([Seg(s, i * b, b)])
        tail = length - nfull * b
        if tail:
            pieces.append(Seg(s, nfull * b, tail))
    pieces.sort(key=lambda g: (-g.length, g.seq))
    bins, room = [], []
    for p in pieces:
        for i, r in enumerate(room):
            if p.length <= r:
                bins[i].append(p)
                room[i] -= p.length
                break
        else:
            bins.append([p])
            room.append(b - p.length)
    return full + bins


def block_cost(block, causal=True, seqlens=None):
    """Visible (query, key) pairs of a block when it is the query side, over its whole
    sequence prefix (causal) or whole sequence (non-causal): the Comp(w) summand of FCP
    paper Sec. 3.3 with f counted in FLOP-proportional units."""
    c = 0
    for s in block:
        if causal:
            c += s.length * s.pos0 + s.length * (s.length + 1) // 2
        else:
            c += s.length * seqlens[s.seq]
    return c


def lpt_assign(blocks, costs, n_workers, cap_tokens):
    """LPT variant of FCP paper Sec. 4.1: blocks heaviest first (ties: lower block id),
    each to the least-loaded worker (ties: lower worker id) whose token count stays
    within ``cap_tokens``. Returns (assignment list, per-worker load, per-worker tokens).
    """
    order = sorted(range(len(blocks)), key=lambda i: (-costs[i], i))
    load = [0] * n_workers
    tokens = [0] * n_workers
    heap = [(0, w) for w in range(n_workers)]
    heapq.heapify(heap)
    assign = [-1] * len(blocks)
    for i in order:
        ntok = sum(s.length for s in blocks[i])
        skipped = []
        while heap:
            ld, w = heapq.heappop(heap)
            if tokens[w] + ntok <= cap_tokens:
                break
            skipped.append((ld, w))
        else:
            raise ValueError("no worker can take block %d under the token cap" % i)
        assign[i] = w
        load[w] += costs[i]
        tokens[w] += ntok
        heapq.heappush(heap, (load[w], w))
        for e in skipped:
            heapq.heappush(heap, e)
    return assign, load, tokens


def place(blocks):
    """Lay blocks out back to back in one buffer; returns blocks of placed segments."""
    out, row = [], 0
    for blk in blocks:
        placed = []
        for s in blk:
            placed.append(Seg(s.seq, s.pos0, s.length, row))
            row += s.length
        out.append(placed)
    return out
