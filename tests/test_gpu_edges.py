"""Edge cases of the C ABI on the GPU: empty pair tables, single-row and single-key
pairs, ragged lengths around the tile sizes, queries that see no key (O = 0, LSE = -inf)
through the forward, the merge and the backward. Forward partials are checked pair by
pair against the float64 oracle; rows without a visible key must come out exact."""
import numpy as np
import pytest

import fcp_workloads as W
import oracle
from block_wise_varlen_amd import binding as B
from block_wise_varlen_amd.descriptors import PAIR_DTYPE, FLAG_CAUSAL, COPY_DTYPE, STAGE_DTYPE
from tests import gpu_util as U
from tests.test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu


def buffers(rows, hq, hkv, d, seed, causal=False):
    """bf16 Q/K/V/dO of `rows` rows each (one sequence of that length), device and host."""
    wl = W.custom([rows], rows, hq, hkv, d, causal)
    return wl, U.inputs(wl, seed=seed)


def table(rows):
    """Pairs from (q_start, q_len, kv_start, kv_len, mask_offset, causal), out_row in order."""
    p = np.zeros(len(rows), PAIR_DTYPE)
    out = 0
    for i, (qs, ql, ks, kl, mo, causal) in enumerate(rows):
        p[i] = (0, qs, ql, ks, kl, mo, out, FLAG_CAUSAL if causal else 0)
        out += ql
    return p


def oracle_partial(x, p, hq, hkv):
    qr = np.arange(p["q_start"], p["q_start"] + p["q_len"])
    kr = np.arange(p["kv_start"], p["kv_start"] + p["kv_len"])
    # Key j of the pair sits at position j, query i at position i + mask_offset.
    return oracle.partial(x["q"], x["k"], x["v"], qr, int(p["mask_offset"]) + np.arange(len(qr)),
                          kr, np.arange(len(kr)), bool(p["flags"] & FLAG_CAUSAL), hq, hkv)


def test_empty_tables_touch_nothing(gpu):
    import torch
    wl, (dev, _) = buffers(64, 8, 2, 128, seed=20)
    empty = np.zeros(0, PAIR_DTYPE)
    sentinel = 3.25
    o_part = torch.full((4, 8, 128), sentinel, dtype=torch.float32, device=gpu)
    lse_part = torch.full((4, 8), sentinel, dtype=torch.float32, device=gpu)
    B.fcp_block_attn_fwd(dev["q"], dev["k"], dev["v"], empty, o_part=o_part, lse_part=lse_part)
    o = torch.full_like(dev["q"], sentinel)
    lse = torch.full((64, 8), sentinel, dtype=torch.float32, device=gpu)
    B.fcp_merge_partials(empty, o_part, lse_part, 64, 2, o=o, lse=lse)
    B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], empty, o=o, lse=lse)
    dq = torch.full((64, 8, 128), sentinel, dtype=torch.float32, device=gpu)
    dk = torch.full((64, 2, 128), sentinel, dtype=torch.float32, device=gpu)
    dv = torch.full_like(dk, sentinel)
    B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], empty, dq=dq, dk=dk,
                         dv=dv)
    k2, v2 = dev["k"].clone(), dev["v"].clone()
    B.fcp_pipeline_fwd(dev["q"], k2, v2, dev["k"], dev["v"], np.zeros(0, STAGE_DTYPE),
                       np.zeros(0, COPY_DTYPE), empty, o_part, lse_part, o=o, lse=lse,
                       copy_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    for t in (o_part, lse_part, o.float(), lse, dq, dk, dv):
        assert bool((t == sentinel).all())
    assert torch.equal(k2, dev["k"]) and torch.equal(v2, dev["v"])


@pytest.mark.parametrize("d,hq,hkv", [(128, 8, 2), (64, 4, 4), (128, 16, 1)])
def test_degenerate_pairs_forward(gpu, d, hq, hkv):
    """Single-row and single-key pairs, lengths just around 32/64/128, causal offsets that
    leave some or all queries without a key (down to INT32_MIN) or let all see every key
    (up to INT32_MAX), overlapping Q ranges (allowed for partials)."""
    import torch
    wl, (dev, x) = buffers(200, hq, hkv, d, seed=21)
    rows = [(0, 1, 0, 1, 0, False), (1, 1, 5, 1, 0, True), (2, 1, 6, 1, -1, True),
            (3, 33, 10, 32, -5, True), (36, 28, 0, 64, 100, True), (0, 64, 1, 1, 0, False),
            (64, 31, 64, 127, 0, True), (95, 65, 40, 129, 64, True), (160, 40, 0, 200, -300, True),
            (160, 40, 0, 200, 0, False), (199, 1, 199, 1, 0, True),
            (0, 64, 100, 50, 2 ** 31 - 1, True), (64, 20, 0, 10, -2 ** 31, True)]
    pairs = table(rows)
    o_part, lse_part = B.fcp_block_attn_fwd(dev["q"], dev["k"], dev["v"], pairs,
                                            part_rows=int(pairs["q_len"].sum()))
    torch.cuda.synchronize()
    o_part, lse_part = o_part.cpu().numpy(), lse_part.cpu().numpy()
    for i, p in enumerate(pairs):
        o_ref, l_ref = oracle_partial(x, p, hq, hkv)
        sl = slice(p["out_row"], p["out_row"] + p["q_len"])
        U.check_attn(o_part[sl], lse_part[sl], o_ref, l_ref, "pair %d %s" % (i, rows[i]))


def test_merge_with_dead_partials(gpu):
    """A Q range whose partials include one that sees no key at all, and a Q range that
    sees nothing in any partial (merged O = 0, LSE = -inf exactly)."""
    import torch
    hq, hkv, d = 8, 2, 128
    wl, (dev, x) = buffers(96, hq, hkv, d, seed=22)
    rows = [(0, 32, 0, 32, -40, True), (0, 32, 32, 64, 0, False), (0, 32, 0, 16, 3, True),
            (32, 16, 0, 16, -20, True), (32, 16, 40, 8, -16, True)]
    pairs = table(rows)
    o_part, lse_part = B.fcp_block_attn_fwd(dev["q"], dev["k"], dev["v"], pairs,
                                            part_rows=int(pairs["q_len"].sum()))
    o, lse = B.fcp_merge_partials(pairs, o_part, lse_part, 96, hkv)
    torch.cuda.synchronize()
    parts = [oracle_partial(x, p, hq, hkv) for p in pairs]
    o_ref0, l_ref0 = oracle.merge([parts[i][1] for i in range(3)], [parts[i][0] for i in range(3)])
    o_ref1, l_ref1 = oracle.merge([parts[i][1] for i in (3, 4)], [parts[i][0] for i in (3, 4)])
    og, lg = U.bf16_to_f64(o), lse.cpu().numpy()
    U.check_attn(og[0:32], lg[0:32], o_ref0, l_ref0, "live range")
    assert np.isneginf(l_ref1).all()
    U.check_attn(og[32:48], lg[32:48], o_ref1, l_ref1, "dead range")


def test_backward_with_dead_queries(gpu):
    """Queries that see no key have LSE = -inf: their dQ is exactly zero and they add
    nothing to dK / dV, so the result equals the backward of the live queries alone."""
    import torch
    hq, hkv, d = 8, 2, 128
    wl, (dev, _) = buffers(64, hq, hkv, d, seed=23)
    full = table([(0, 40, 0, 48, -4, True)])        # queries 0..3 see nothing
    live = table([(4, 36, 0, 48, 0, True)])         # the same visibility for queries 4..39
    o, lse = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], full)
    o2, lse2 = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], live)
    dq, dk, dv = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], full)
    dq2, dk2, dv2 = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o2, lse2, dev["do"], live)
    torch.cuda.synchronize()
    assert torch.isneginf(lse[0:4]).all() and bool((o[0:4] == 0).all())
    assert torch.equal(o[4:40], o2[4:40]) and torch.equal(lse[4:40], lse2[4:40])
    for t in (dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    assert bool((dq[0:4] == 0).all())
    check_grad(dq[4:40].cpu().numpy(), dq2[4:40].cpu().numpy().astype(np.float64), "dq")
    for got, ref, nm in ((dk, dk2, "dk"), (dv, dv2, "dv")):
        g, r = got.cpu().numpy().astype(np.float64), ref.cpu().numpy().astype(np.float64)
        assert np.abs(g - r).max() <= 1e-5 * max(np.abs(r).max(), 1e-30), nm


@pytest.mark.parametrize("d,hkv", [(128, 2), (64, 1)])
def test_tiny_sequences_forward_backward(gpu, d, hkv):
    """Sequences of 1, 2, 31, 33 and 129 tokens packed into 32-token blocks, every KV
    range cut in three (so single-key and empty-remainder parts occur)."""
    import torch
    wl = W.custom([1, 1, 31, 33, 129, 2], 32, 8, hkv, d, True, kv_split=3)
    dev, x = U.inputs(wl, seed=24)
    from block_wise_varlen_amd.descriptors import build_pairs
    pairs = build_pairs(wl)
    o, lse = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], pairs)
    dq, dk, dv = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], pairs)
    torch.cuda.synchronize()
    idx = oracle.SeqIndex(wl)
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], idx)
    rows = idx.owned_rows()
    U.check_attn(U.bf16_to_f64(o)[rows], lse.cpu().numpy()[rows], o_ref, l_ref, "tiny fwd")
    rq, rk, rv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)
    check_grad(dq.cpu().numpy(), rq, "dq")
    check_grad(dk.cpu().numpy(), rk, "dk")
    check_grad(dv.cpu().numpy(), rv, "dv")
