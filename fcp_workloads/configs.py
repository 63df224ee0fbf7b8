"""The five synthetic workloads, built from seeded draws.

Model shape everywhere except the tiny case: 64 query heads, 8 KV heads, head dim 128,
the Llama-3-70B layout of FCP paper Sec. 6.1. Block sizes, the 64-worker group, the
128K-token per-worker budget and the coalesce degree echo FCP paper Sec. 4.1, Sec. 4.2
and Sec. 6.1 / 6.6. "K" is 1024 tokens throughout.
"""
import numpy as np

from .layout import Workload, pack_stream, shard_ffd, lpt_assign, block_cost, place
from .lengths import lognormal_lengths

CONFIG_NAMES = {
    1: "tiny-varlen-3seq-b256-h4kv1-d64",
    2: "worker-1K-blocks-16x1024-lognormal4K-h64kv8-d128",
    3: "sweep-32K-single-seq-h64kv8-d128",
    4: "zigzag-512K-b4096-N64-c4-h64kv8-d128",
    5: "hetero-lognormal8K-128Kx64-b4096-lpt-h64kv8-d128",
}


def _wl(name, seqlens, b, hq, hkv, d, causal, q_ids, kv_ids, blocks, **kw):
    return Workload(name=name, seqlens=list(seqlens), block_size=b, num_q_heads=hq,
                    num_kv_heads=hkv, head_dim=d, causal=causal,
                    q_blocks=place([blocks[i] for i in q_ids]),
                    kv_blocks=place([blocks[i] for i in kv_ids]),
                    q_block_ids=list(q_ids), kv_block_ids=list(kv_ids), **kw)


def config1(causal=True, kv_split=2):
    """Three packed sequences 300/128/596 cut into 256-token blocks; 4 Q heads, 1 KV
    head, head dim 64. The worker holds every block."""
    seqlens = [300, 128, 596]
    blocks = pack_stream(seqlens, 256)
    ids = list(range(len(blocks)))
    return _wl(CONFIG_NAMES[1], seqlens, 256, 4, 1, 64, causal, ids, ids, blocks,
               kv_split=kv_split)


def config2(seed=0, block=1024, n_blocks=16, causal=True):
    """One worker's 16 x 1024 tokens, packed from lognormal lengths (median 4K,
    sigma 1.2, truncated to [256, 64K]); the stream is cut every 1024 tokens."""
    rng = np.random.default_rng(seed)
    seqlens = lognormal_lengths(rng, 4096, 1.2, 256, 65536, block * n_blocks)
    blocks = pack_stream(seqlens, block)
    ids = list(range(len(blocks)))
    return _wl(CONFIG_NAMES[2], seqlens, block, 64, 8, 128, causal, ids, ids, blocks,
               meta={"seed": seed})


def config3(block=4096, causal=True, seqlen=32768, hq=64, hkv=8, d=128):
    """One 32K-token sequence cut into ``block``-token blocks; every needed pair."""
    blocks = pack_stream([seqlen], block)
    ids = list(range(len(blocks)))
    return _wl(CONFIG_NAMES[3], [seqlen], block, hq, hkv, d, causal, ids, ids, blocks,
               meta={"block": block})


def config4(worker=0, n_workers=64, seqlen=524288, block=4096, coalesce=4):
    """Zig-Zag worker: Q blocks ``w`` and ``2N-1-w`` of a 512K sequence in 4K blocks,
    against every causally needed KV block (blocks 0..max), coalesced 4 at a time."""
    blocks = pack_stream([seqlen], block)
    n = len(blocks)
    assert n == 2 * n_workers
    q_ids = [worker, n - 1 - worker]
    kv_ids = list(range(max(q_ids) + 1))
    return _wl(CONFIG_NAMES[4], [seqlen], block, 64, 8, 128, True, q_ids, kv_ids, blocks,
               coalesce=coalesce, meta={"worker": worker, "n_workers": n_workers})


def config5(seed=0, n_workers=64, budget_per_worker=131072, block=4096, coalesce=1,
            worker=None):
    """Heterogeneous batch: lognormal lengths (median 8K, sigma 1.5, truncated to
    [1, 512K]) fill 64 x 128K tokens; sequences are cut into 4K blocks, tails and short
    sequences packed FFD; blocks go to workers by LPT under a 128K + 4K token cap. The
    measured worker is the most loaded one (ties: lowest id); it holds its Q blocks and
    every KV block its Q segments need causally, placed locally as if pulled."""
    rng = np.random.default_rng(seed)
    seqlens = lognormal_lengths(rng, 8192, 1.5, 1, 524288, n_workers * budget_per_worker)
    blocks = shard_ffd(seqlens, block)
    costs = [block_cost(b) for b in blocks]
    assign, load, tokens = lpt_assign(blocks, costs, n_workers,
                                      budget_per_worker + block)
    if worker is None:
        worker = max(range(n_workers), key=lambda w: (load[w], -w))
    q_ids = [i for i, w in enumerate(assign) if w == worker]
    kv_ids = kv_needs(blocks, q_ids)
    return _wl(CONFIG_NAMES[5], seqlens, block, 64, 8, 128, True, q_ids, kv_ids, blocks,
               coalesce=coalesce, rng="device",
               meta={"seed": seed, "worker": worker, "load": load, "tokens": tokens,
                     "assign": assign, "n_blocks": len(blocks)})


def kv_needs(blocks, q_ids):
    """Ids of the blocks whose keys the Q blocks ``q_ids`` attend to causally: every block
    holding a position of one of their sequences below the last query position."""
    need = {}
    for i in q_ids:
        for s in blocks[i]:
            need[s.seq] = max(need.get(s.seq, 0), s.pos0 + s.length)
    return [i for i, blk in enumerate(blocks)
            if any(s.seq in need and s.pos0 < need[s.seq] for s in blk)]


def pull_graph(blocks, assign, n_workers):
    """The block transfers of one causal forward (FCP paper Sec. 4.2, Figure 8): every
    block's K/V live with the worker its Q is assigned to, and every worker pulls each
    block it needs that another worker holds. Returns (src, dst, block) int32 arrays, one
    entry per transfer (sender, receiver, block id), sorted by receiver then block id."""
    src, dst, blk = [], [], []
    for w in range(n_workers):
        mine = [i for i, a in enumerate(assign) if a == w]
        for j in kv_needs(blocks, mine):
            if assign[j] != w:
                src.append(assign[j])
                dst.append(w)
                blk.append(j)
    return tuple(np.asarray(x, dtype=np.int32) for x in (src, dst, blk))


def zigzag_graph(n_workers=64, seqlen=524288, block=4096):
    """Pull graph of the Zig-Zag assignment of one sequence: worker w holds blocks w and
    2N-1-w (FCP paper Sec. 3.2, Figure 4)."""
    blocks = pack_stream([seqlen], block)
    n = len(blocks)
    assert n == 2 * n_workers
    assign = [b if b < n_workers else n - 1 - b for b in range(n)]
    return pull_graph(blocks, assign, n_workers)


def hetero_graph(seed=0, n_workers=64, budget_per_worker=131072, block=4096):
    """Pull graph of the heterogeneous lognormal batch with its LPT assignment (the
    workload of ``config5``, all workers)."""
    rng = np.random.default_rng(seed)
    seqlens = lognormal_lengths(rng, 8192, 1.5, 1, 524288, n_workers * budget_per_worker)
    blocks = shard_ffd(seqlens, block)
    costs = [block_cost(b) for b in blocks]
    assign, _, _ = lpt_assign(blocks, costs, n_workers, budget_per_worker + block)
    return pull_graph(blocks, assign, n_workers)


def custom(seqlens, block, hq, hkv, d, causal=True, q_ids=None, kv_ids=None,
           coalesce=1, kv_split=1, shard="stream"):
    """A small workload for tests: ``shard`` is "stream" (cut the packed stream) or
    "ffd" (cut sequences, pack tails first-fit-decreasing)."""
    blocks = pack_stream(seqlens, block) if shard == "stream" else shard_ffd(seqlens, block)
    ids = list(range(len(blocks)))
    return _wl("custom", seqlens, block, hq, hkv, d, causal,
               ids if q_ids is None else q_ids, ids if kv_ids is None else kv_ids,
               blocks, coalesce=coalesce, kv_split=kv_split)


def visible_pairs(wl) -> int:
    """Same-sequence, unmasked (query, key) pairs over the worker's Q rows (one head).

    Causal: a query at in-sequence position i sees keys 0..i, so a segment of n queries
    starting at p0 sees n*p0 + n(n+1)/2 pairs (the L(L+1)/2 causal count of "Another View
    on Context Parallel for LLMs", section "Theory"). Non-causal: n * L_s.
    """
    total = 0
    for s in wl.q_segments():
        if wl.causal:
            total += s.length * s.pos0 + s.length * (s.length + 1) // 2
        else:
            total += s.length * wl.seqlens[s.seq]
    return total


def fwd_flops(wl) -> int:
    """Forward FLOPs: two contractions (QK^T and PV) of 2*D each per visible pair and
    query head."""
    return 4 * wl.head_dim * wl.num_q_heads * visible_pairs(wl)


def bwd_flops(wl) -> int:
    """Backward FLOPs: five contractions (S recompute, dP, dV, dK, dQ) of 2*D each."""
    return 10 * wl.head_dim * wl.num_q_heads * visible_pairs(wl)
