"""Congestion-free communication plan (FCP paper Sec. 4.2, "Congestion-free solver",
Lemmas 1 and 2): the oracle pinned against exhaustive search and closed forms, then the
library's host-only planner checked against the oracle. Several plans are optimal, so
what is unique is compared (the number of stages) and the rest is checked for validity
(every stage a matching, every edge in exactly one stage)."""
import os

import numpy as np
import pytest

import fcp_workloads as W
from oracle import comm as C
from block_wise_varlen_amd import binding as B


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from block_wise_varlen_amd import build
        build.build()
    return B.load()


def random_multigraph(rng, n, e, self_loops=True):
    src = rng.integers(0, n, e).astype(np.int32)
    dst = rng.integers(0, n, e).astype(np.int32)
    if not self_loops:
        dst = np.where(dst == src, (dst + 1) % n, dst).astype(np.int32)
    return src, dst


# ---- oracle pins --------------------------------------------------------------------

def test_validity_check_rejects_planted_conflicts():
    src, dst = [0, 0, 1], [1, 2, 2]
    assert C.is_congestion_free(3, src, dst, [0, 1, 0], 2)
    assert not C.is_congestion_free(3, src, dst, [0, 0, 1], 2)   # worker 0 sends twice
    assert not C.is_congestion_free(3, src, dst, [0, 1, 1], 2)   # worker 2 receives twice
    assert not C.is_congestion_free(3, src, dst, [0, 1, 2], 2)   # stage out of range
    assert not C.is_congestion_free(3, src, dst, [0, 1], 2)      # an edge without stage
    # Parallel edges (two blocks between one pair) must go to different stages.
    assert not C.is_congestion_free(2, [0, 0], [1, 1], [0, 0], 1)
    assert C.is_congestion_free(2, [0, 0], [1, 1], [0, 1], 2)


def test_max_degree_closed_forms():
    assert C.max_degree(4, [], []) == 0
    # A star: one worker sends to all others (Delta = n-1 on the send side).
    assert C.max_degree(5, [0, 0, 0, 0], [1, 2, 3, 4]) == 4
    # Receive side dominates.
    assert C.max_degree(5, [1, 2, 3, 4, 1], [0, 0, 0, 0, 2]) == 4
    # All-to-all among n workers without self transfers: Delta = n - 1.
    n = 6
    src, dst = zip(*[(i, j) for i in range(n) for j in range(n) if i != j])
    assert C.max_degree(n, src, dst) == n - 1


def test_latin_square_plan_of_all_to_all():
    # K_{n,n}: stage (i + j) mod n is the classic optimal plan with n stages.
    n = 5
    src, dst = zip(*[(i, j) for i in range(n) for j in range(n)])
    stage = [(i + j) % n for i, j in zip(src, dst)]
    assert C.is_congestion_free(n, src, dst, stage, n)
    assert C.max_degree(n, src, dst) == n


@pytest.mark.parametrize("seed", range(12))
def test_brute_force_minimum_is_max_degree(seed):
    """Lemma 2 and the construction: the fewest stages of any plan, found by exhaustive
    search, equals Delta on tiny multigraphs (parallel edges and self transfers too)."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 5))
    e = int(rng.integers(1, 8))
    src, dst = random_multigraph(rng, n, e)
    assert C.min_stages_brute_force(n, src, dst) == C.max_degree(n, src, dst)


def test_brute_force_finds_lower_than_naive():
    # Two disjoint transfers fit one stage; a chain 0->1, 1->2 also fits one stage.
    assert C.min_stages_brute_force(3, [0, 1], [1, 2]) == 1
    # Two blocks into one receiver need two stages.
    assert C.min_stages_brute_force(3, [0, 1], [2, 2]) == 2


@pytest.mark.parametrize("seed", range(8))
def test_alternating_path_plan_is_optimal(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 40))
    e = int(rng.integers(0, 400))
    src, dst = random_multigraph(rng, n, e)
    stage, k = C.alternating_path_plan(n, src, dst)
    assert k == C.max_degree(n, src, dst)
    assert C.is_congestion_free(n, src, dst, stage, k)


@pytest.mark.parametrize("seed", range(6))
def test_alternating_path_plan_tiny_matches_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    src, dst = random_multigraph(rng, 3, 6)
    stage, k = C.alternating_path_plan(3, src, dst)
    assert C.is_congestion_free(3, src, dst, stage, k)
    assert k == C.min_stages_brute_force(3, src, dst)


# ---- library planner vs the oracle ---------------------------------------------------

def check_plan(n, src, dst):
    stage, k = B.fcp_comm_plan(n, src, dst)
    assert k == C.max_degree(n, src, dst)
    assert C.is_congestion_free(n, src, dst, stage, k)
    if len(src):
        # Every stage carries at least one transfer.
        assert np.array_equal(np.unique(stage), np.arange(k))
    return stage, k


@pytest.mark.parametrize("seed", range(12))
def test_tiny_graphs_match_brute_force(lib, seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 5))
    e = int(rng.integers(0, 8))
    src, dst = random_multigraph(rng, n, e)
    _, k = check_plan(n, src, dst)
    assert k == C.min_stages_brute_force(n, src, dst)


@pytest.mark.parametrize("n,e", [(2, 50), (7, 100), (33, 1000), (64, 6000), (200, 3000),
                                 (256, 65536)])
def test_random_multigraphs(lib, n, e):
    rng = np.random.default_rng(n * 1000 + e)
    src, dst = random_multigraph(rng, n, e)
    _, k = check_plan(n, src, dst)
    if e <= 6000:
        assert C.alternating_path_plan(n, src, dst)[1] == k


def test_irregular_shapes(lib):
    # Isolated workers, one hot receiver, all parallel edges between one pair.
    check_plan(10, np.array([0, 1, 2, 3, 4], np.int32), np.array([9, 9, 9, 9, 9], np.int32))
    check_plan(3, np.full(17, 1, np.int32), np.full(17, 2, np.int32))
    check_plan(1, np.zeros(5, np.int32), np.zeros(5, np.int32))
    n = 9
    src, dst = zip(*[(i, j) for i in range(n) for j in range(n) if i != j])
    check_plan(n, np.array(src, np.int32), np.array(dst, np.int32))


def test_empty_and_errors(lib):
    stage, k = B.fcp_comm_plan(4, np.zeros(0, np.int32), np.zeros(0, np.int32))
    assert k == 0 and stage.size == 0
    with pytest.raises(B.FcpError, match="outside"):
        B.fcp_comm_plan(4, np.array([0, 4], np.int32), np.array([1, 1], np.int32))
    with pytest.raises(B.FcpError, match="outside"):
        B.fcp_comm_plan(4, np.array([0, 1], np.int32), np.array([-1, 1], np.int32))
    with pytest.raises(B.FcpError):
        B.fcp_comm_plan(0, np.array([0], np.int32), np.array([0], np.int32))


def test_zigzag_pull_graph(lib):
    """Zig-Zag over 64 workers (512K tokens, 4K blocks): worker w pulls every causally
    needed block it does not hold. Worker 0 needs all 126 remote blocks, and worker 63
    sends its two blocks to 63 + 62 others, so Delta = 2N - 2."""
    n = 64
    src, dst, _ = W.zigzag_graph(n)
    assert len(src) == sum(2 * n - w - 2 for w in range(n))
    stage, k = check_plan(n, src, dst)
    assert k == 2 * n - 2
    ref, kr = C.alternating_path_plan(n, src, dst)
    assert kr == k and C.is_congestion_free(n, src, dst, ref, kr)


def test_heterogeneous_pull_graph(lib):
    """The lognormal batch over 64 workers with its LPT assignment."""
    src, dst, _ = W.hetero_graph()
    stage, k = check_plan(64, src, dst)
    _, kr = C.alternating_path_plan(64, src, dst)
    assert kr == k


@pytest.mark.parametrize("c", [2, 4, 8])
def test_coalesced_stages_stay_balanced(lib, c):
    """Bottom-up coalescing (FCP paper Sec. 4.2): merging c consecutive sub-stages gives
    ceil(Delta / c) stages in which every worker sends and receives at most c blocks."""
    n = 64
    src, dst, _ = W.zigzag_graph(n)
    stage, k = check_plan(n, src, dst)
    coarse = stage // c
    assert coarse.max() + 1 == -(-k // c)
    for s in range(coarse.max() + 1):
        m = coarse == s
        assert np.bincount(src[m], minlength=n).max() <= c
        assert np.bincount(dst[m], minlength=n).max() <= c
