"""Host-side workload generation and the descriptor builder."""
import os

import numpy as np
import pytest

import fcp_workloads as W
from block_wise_varlen_amd.descriptors import (build_pairs, visible_pairs_of, part_rows,
                                               PAIR_FIELDS, FLAG_CAUSAL)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_config1_golden_pairs():
    rows = np.loadtxt(os.path.join(GOLDEN, "config1_pairs.txt"), dtype=np.int64, comments="#")
    pairs = build_pairs(W.config1(kv_split=1))
    got = np.stack([pairs[f] for f in PAIR_FIELDS], axis=1)
    np.testing.assert_array_equal(got, rows)


def test_config1_counts():
    wl = W.config1()
    assert W.visible_pairs(wl) == 300 * 301 // 2 + 128 * 129 // 2 + 596 * 597 // 2 == 231312
    assert W.fwd_flops(wl) == 236863488
    assert W.visible_pairs(W.config1(causal=False)) == 300 ** 2 + 128 ** 2 + 596 ** 2
    assert len(build_pairs(W.config1(causal=False, kv_split=1))) == 14
    split = build_pairs(wl)
    assert len(split) == 20 and part_rows(split) == 2 * part_rows(build_pairs(wl, kv_split=1))


def _pair_cover(pairs, wl):
    """Multiset of visible (q row, kv row) pairs a table covers."""
    cover = {}
    for p in pairs:
        for i in range(p["q_len"]):
            for j in range(p["kv_len"]):
                if (p["flags"] & FLAG_CAUSAL) and j - i > p["mask_offset"]:
                    continue
                key = (p["q_start"] + i, p["kv_start"] + j)
                cover[key] = cover.get(key, 0) + 1
    return cover


def _true_cover(wl):
    kv = {}
    for s in wl.kv_segments():
        for t in range(s.length):
            kv[(s.seq, s.pos0 + t)] = s.row0 + t
    out = set()
    for s in wl.q_segments():
        for t in range(s.length):
            qp = s.pos0 + t
            last = qp if wl.causal else wl.seqlens[s.seq] - 1
            for kp in range(last + 1):
                out.add((s.row0 + t, kv[(s.seq, kp)]))
    return out


@pytest.mark.parametrize("args", [
    dict(seqlens=[5, 1, 9, 3], block=4, causal=True),
    dict(seqlens=[5, 1, 9, 3], block=4, causal=False),
    dict(seqlens=[17, 2, 30, 6, 11], block=8, causal=True, shard="ffd"),
    dict(seqlens=[40], block=4, causal=True, coalesce=3),
    dict(seqlens=[40, 9], block=4, causal=False, coalesce=4, kv_split=3),
    dict(seqlens=[23, 7], block=5, causal=True, coalesce=2, kv_split=2),
])
def test_pairs_cover_each_visible_pair_once(args):
    wl = W.custom(hq=2, hkv=1, d=4, **args)
    pairs = build_pairs(wl)
    cover = _pair_cover(pairs, wl)
    assert set(cover) == _true_cover(wl)
    assert all(c == 1 for c in cover.values())
    assert visible_pairs_of(pairs) == W.visible_pairs(wl)
    assert np.all(pairs["q_len"] >= 1) and np.all(pairs["kv_len"] >= 1)


def test_zigzag_subset_covers_once():
    wl = W.custom([64], 4, 1, 1, 4, True, q_ids=[2, 13], kv_ids=list(range(14)), coalesce=4)
    cover = _pair_cover(build_pairs(wl), wl)
    assert set(cover) == _true_cover(wl) and all(c == 1 for c in cover.values())


def test_config3_pair_counts_and_flops():
    for b in (512, 1024, 2048, 4096):
        n = 32768 // b
        assert len(build_pairs(W.config3(b, True))) == n * (n + 1) // 2
        assert len(build_pairs(W.config3(b, False))) == n * n
        assert W.fwd_flops(W.config3(b, True)) == 4 * 128 * 64 * (32768 * 32769 // 2)
        assert W.fwd_flops(W.config3(b, False)) == 4 * 128 * 64 * 32768 ** 2


def test_zigzag_balance():
    """Zig-Zag pairing gives every worker the same causal work (FCP paper Sec. 3.2,
    Figure 4; Sec. 3.4): Q blocks w and 2N-1-w of a 512K sequence in 4K blocks."""
    flops = {W.fwd_flops(W.config4(w)) for w in (0, 1, 17, 31, 63)}
    assert flops == {70368878395392}
    assert len(build_pairs(W.config4(0))) == 33


def test_lognormal_budget():
    rng = np.random.default_rng(5)
    ls = W.lognormal_lengths(rng, 4096, 1.2, 256, 65536, 1 << 20)
    assert sum(ls) == 1 << 20
    assert all(256 <= x <= 65536 for x in ls[:-1]) and 1 <= ls[-1] <= 65536
    assert 2500 < np.median(ls) < 6500


def test_lpt_distributor():
    wl = W.config5(0)
    m = wl.meta
    blocks = W.shard_ffd(wl.seqlens, 4096)
    assert len(m["assign"]) == len(blocks) == m["n_blocks"]
    assert all(0 <= a < 64 for a in m["assign"])
    assert max(m["tokens"]) <= 131072 + 4096
    assert sum(m["tokens"]) == sum(wl.seqlens) == 64 * 131072
    load = m["load"]
    assert (max(load) - np.mean(load)) / max(load) < 0.05   # FCP paper Sec. 6.2: < 5%
    assert m["worker"] == int(np.argmax(load))
    # every sequence's tokens appear exactly once across blocks
    seen = {}
    for blk in blocks:
        assert sum(s.length for s in blk) <= 4096
        for s in blk:
            seen.setdefault(s.seq, []).append((s.pos0, s.length))
    for sq, segs in seen.items():
        segs.sort()
        pos = 0
        for p0, n in segs:
            assert p0 == pos
            pos += n
        assert pos == wl.seqlens[sq]


def test_lpt_greedy_property():
    """Each block goes to a least-loaded worker among those with room (replayed)."""
    rng = np.random.default_rng(3)
    seqlens = W.lognormal_lengths(rng, 300, 1.0, 1, 5000, 8 * 2000)
    blocks = W.shard_ffd(seqlens, 256)
    costs = [W.block_cost(b) for b in blocks]
    assign, load, tokens = W.lpt_assign(blocks, costs, 8, 2000 + 256)
    cur_l, cur_t = [0] * 8, [0] * 8
    for i in sorted(range(len(blocks)), key=lambda i: (-costs[i], i)):
        n = sum(s.length for s in blocks[i])
        ok = [w for w in range(8) if cur_t[w] + n <= 2256]
        best = min(ok, key=lambda w: (cur_l[w], w))
        assert assign[i] == best
        cur_l[best] += costs[i]
        cur_t[best] += n


def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    x[:4] = [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(W.round_to_bf16_bits(x), ref)
    assert W.bf16_bits_to_f64(W.round_to_bf16_bits(x[:2])).tolist() == [1.0, 1 + 2 ** -6]


def test_host_inputs_deterministic_and_blockwise():
    wl = W.config1()
    a = W.make_host_inputs(wl, seed=1)
    b = W.make_host_inputs(wl, seed=1)
    c = W.make_host_inputs(wl, seed=2)
    for n in a:
        np.testing.assert_array_equal(a[n], b[n])
        assert not np.array_equal(a[n], c[n])
    assert a["q"].shape == (1024, 4, 64) and a["k"].shape == (1024, 1, 64)
