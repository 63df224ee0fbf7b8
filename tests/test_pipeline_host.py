"""Host side of the block-level pipelined forward (FCP paper Sec. 4.2, "Block-level
pipelining" and "Bottom-up coalescer"): the stage tables cover every visible (query,
key) pair exactly once, respect double buffering, and the library's table checks reject
what would race or fall out of range. No GPU call."""
import os

import numpy as np
import pytest

import fcp_workloads as W
from block_wise_varlen_amd import binding as B
from block_wise_varlen_amd.descriptors import (build_pipeline, FLAG_CAUSAL, COPY_DTYPE,
                                               STAGE_DTYPE, PAIR_DTYPE, visible_pairs_of)
from tests.test_workloads import _true_cover


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from block_wise_varlen_amd import build
        build.build()
    return B.load()




def zigzag_case(n_workers, block, worker, coalesce, hq=2, hkv=1, d=4):
    seqlen = 2 * n_workers * block
    wl = W.custom([seqlen], block, hq, hkv, d, True,
                  q_ids=[worker, 2 * n_workers - 1 - worker],
                  kv_ids=list(range(2 * n_workers - worker)), coalesce=coalesce)
    src, dst, blk = W.zigzag_graph(n_workers, seqlen=seqlen, block=block)
    stage, _ = B.fcp_comm_plan(n_workers, src, dst)
    m = dst == worker
    recv = {int(b): int(s) for b, s in zip(blk[m], stage[m])}
    return wl, recv


def pipeline_cover(P, wl):
    """Visible (q row, source kv row) pairs the tables cover, with multiplicity, mapping
    every stage's KV rows back through that stage's copies."""
    cover = {}
    copies = P["copies"]
    ci = pi = 0
    for t, (nc, np_) in enumerate(P["stages"]):
        cps = P["local_copies"] if t == 0 else copies[ci:ci + nc]
        ci += nc if t else 0
        back = {}
        for c in cps:
            for r in range(int(c["n_rows"])):
                back[int(c["dst_row"]) + r] = int(c["src_row"]) + r
        for p in P["pairs"][pi:pi + np_]:
            for i in range(p["q_len"]):
                for j in range(p["kv_len"]):
                    if (p["flags"] & FLAG_CAUSAL) and j - i > p["mask_offset"]:
                        continue
                    key = (int(p["q_start"]) + i, back[int(p["kv_start"]) + j])
                    cover[key] = cover.get(key, 0) + 1
        pi += np_
    return cover


def check_double_buffer(P):
    """Stage t's copies write no row that stages t-depth+1 .. t-1 read."""
    first_c = np.concatenate([[0], np.cumsum(P["stages"]["n_copies"])])
    first_p = np.concatenate([[0], np.cumsum(P["stages"]["n_pairs"])])
    for t in range(1, len(P["stages"])):
        w = P["copies"][first_c[t]:first_c[t + 1]]
        r = P["pairs"][first_p[max(0, t - P["depth"] + 1)]:first_p[t]]
        for c in w:
            for p in r:
                a0, a1 = c["dst_row"], c["dst_row"] + c["n_rows"]
                b0, b1 = p["kv_start"], p["kv_start"] + p["kv_len"]
                assert not (a0 < b1 and b0 < a1)


@pytest.mark.parametrize("n_workers,block,worker,coalesce,slots", [
    (4, 4, 0, 1, 2), (4, 4, 0, 2, 2), (4, 4, 2, 4, 2), (5, 3, 1, 3, None), (3, 4, 0, 1, None),
    (5, 4, 0, 1, 3), (4, 4, 0, 1, 1),
])
def test_zigzag_tables_cover_once(lib, n_workers, block, worker, coalesce, slots):
    wl, recv = zigzag_case(n_workers, block, worker, coalesce)
    P = build_pipeline(wl, wl.q_block_ids, recv, coalesce=coalesce, depth=slots)
    cover = pipeline_cover(P, wl)
    assert set(cover) == _true_cover(wl)
    assert all(c == 1 for c in cover.values())
    assert visible_pairs_of(P["pairs"]) == W.visible_pairs(wl)
    check_double_buffer(P)
    # Each stage pulls at most `coalesce` blocks; every remote block once.
    pulled = [b for g in P["pulled"][1:] for b in g]
    assert sorted(pulled) == sorted(set(wl.kv_block_ids) - set(wl.q_block_ids))
    assert all(len(g) <= coalesce for g in P["pulled"][1:])


@pytest.mark.parametrize("seed", [0, 1])
def test_packed_blocks_tables_cover_once(lib, seed):
    """Packed blocks of several sequences, arbitrary receive order."""
    rng = np.random.default_rng(seed)
    seqlens = [int(x) for x in rng.integers(1, 30, 9)]
    wl = W.custom(seqlens, 8, 2, 1, 4, True, shard="ffd", coalesce=2)
    n = len(wl.kv_block_ids)
    local = [wl.kv_block_ids[0], wl.kv_block_ids[n // 2]]
    order = rng.permutation([i for i in wl.kv_block_ids if i not in local])
    recv = {int(b): k for k, b in enumerate(order)}
    for slots in (1, 2, 3, None):
        P = build_pipeline(wl, local, recv, coalesce=2, depth=slots)
        cover = pipeline_cover(P, wl)
        assert set(cover) == _true_cover(wl) and all(c == 1 for c in cover.values())
        check_double_buffer(P)


def test_library_accepts_builder_tables(lib):
    wl, recv = zigzag_case(4, 4, 0, 2)
    P = build_pipeline(wl, wl.q_block_ids, recv, coalesce=2, depth=2)
    dims = B.make_dims(2, 1, 64, wl.q_rows, P["kv_rows"], P["part_rows"])
    assert B.fcp_pipeline_workspace_bytes(dims, P["stages"], P["copies"], P["pairs"],
                                          wl.kv_rows, P["depth"]) > 0
    # The same tables with more stages in flight than regions race.
    assert B.fcp_pipeline_workspace_bytes(dims, P["stages"], P["copies"], P["pairs"],
                                          wl.kv_rows, P["depth"] + 1) == 0
    assert "previous" in B.fcp_last_error()


def _tiny_tables():
    dims = B.make_dims(2, 1, 64, 8, 16, 16)
    stages = np.array([(1, 1), (1, 1)], STAGE_DTYPE)
    copies = np.array([(0, 0, 8), (8, 8, 8)], COPY_DTYPE)
    pairs = np.zeros(2, PAIR_DTYPE)
    pairs[0] = (0, 0, 8, 0, 8, 0, 0, 0)
    pairs[1] = (0, 0, 8, 8, 8, 0, 8, 0)
    return dims, stages, copies, pairs


def test_library_rejects_bad_tables(lib):
    dims, stages, copies, pairs = _tiny_tables()
    assert B.fcp_pipeline_workspace_bytes(dims, stages, copies, pairs, 16) > 0
    # Stage 1 copies into the rows stage 0 reads: a race with double buffering, none
    # when each stage's copies wait for the previous stage (depth 1).
    bad = copies.copy()
    bad[1]["dst_row"] = 4
    assert B.fcp_pipeline_workspace_bytes(dims, stages, bad, pairs, 16) == 0
    assert "previous" in B.fcp_last_error()
    assert B.fcp_pipeline_workspace_bytes(dims, stages, bad, pairs, 16, depth=1) > 0
    assert B.fcp_pipeline_workspace_bytes(dims, stages, copies, pairs, 16, depth=0) == 0
    # Copy source or destination out of range, empty copy.
    for field, val in (("src_row", 9), ("dst_row", 9), ("n_rows", 0), ("src_row", -1)):
        bad = copies.copy()
        bad[1][field] = val
        assert B.fcp_pipeline_workspace_bytes(dims, stages, bad, pairs, 16) == 0, field
    # Partial rows overlapping across stages.
    badp = pairs.copy()
    badp[1]["out_row"] = 4
    assert B.fcp_pipeline_workspace_bytes(dims, stages, copies, badp, 16) == 0
    # Negative counts.
    bads = stages.copy()
    bads[0]["n_pairs"] = -1
    assert B.fcp_pipeline_workspace_bytes(dims, bads, copies, pairs, 16) == 0
