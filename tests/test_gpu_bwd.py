"""GPU parity of the backward (dQ, dK, dV) against the float64 oracle, through the C ABI.

Gate per gradient tensor (the pages give none; the arithmetic is bf16 products with fp32
accumulation, and the GPU's Delta uses the bf16-stored merged O): relative L2 <= 1e-2 and
max-abs <= 5e-2 * max|reference|.
"""
import ctypes

import numpy as np
import pytest

import fcp_workloads as W
import oracle
from block_wise_varlen_amd import binding as B
from block_wise_varlen_amd.descriptors import build_pairs
from tests import gpu_util as U
from tests.test_gpu_fwd import SMALL

pytestmark = pytest.mark.gpu

G_REL_L2 = 1e-2
G_MAX_REL = 5e-2


def check_grad(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    assert not np.isnan(got).any(), "%s: NaN" % what
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(got - ref).max()
    assert err <= G_MAX_REL * scale, "%s: max-abs %.3g vs max|ref| %.3g" % (what, err, scale)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= G_REL_L2, "%s: rel-L2 %.3g" % (what, rel)


def _fwd_bwd(wl, dev, pairs):
    o, lse = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], pairs)
    dq, dk, dv = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], pairs)
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_matches_oracle(gpu, name):
    import torch
    wl = SMALL[name]()
    dev, x = U.inputs(wl, seed=5)
    pairs = build_pairs(wl)
    _, _, dq, dk, dv = _fwd_bwd(wl, dev, pairs)
    torch.cuda.synchronize()
    idx = oracle.SeqIndex(wl)
    rq, rk, rv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)
    rows = idx.owned_rows()
    check_grad(dq.cpu().numpy()[rows], rq[rows], name + " dQ")
    check_grad(dk.cpu().numpy(), rk, name + " dK")
    check_grad(dv.cpu().numpy(), rv, name + " dV")


def test_backward_accumulates_and_is_deterministic(gpu):
    """Outputs are added to (+=); two runs give bitwise-equal results (no atomics)."""
    import torch
    wl = SMALL["g4-d128-ffd-coalesce"]()
    dev, _ = U.inputs(wl, seed=6)
    pairs = build_pairs(wl)
    o, lse, dq, dk, dv = _fwd_bwd(wl, dev, pairs)
    dq2, dk2, dv2 = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"],
                                         pairs)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], pairs, dq=dq2,
                         dk=dk2, dv=dv2)
    torch.cuda.synchronize()
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        torch.testing.assert_close(b, 2 * a, rtol=1e-6, atol=1e-6)



@pytest.mark.parametrize("drop_last_q_range", [False, True])
def test_overwrite_mode(gpu, drop_last_q_range):
    """FCP_BWD_OVERWRITE writes the rows the pairs cover (bitwise what zeroing and adding
    gives) and leaves every other row as it was; the workload's heavy key tiles are split
    by heads, so the reduce kernel's write path runs too. With the last Q range's pairs
    dropped, its Q rows (and any KV rows only those pairs read) stay untouched."""
    import torch
    wl = SMALL["g4-d128-ffd-coalesce"]()
    dev, _ = U.inputs(wl, seed=9)
    pairs = build_pairs(wl)
    if drop_last_q_range:
        pairs = pairs[pairs["q_start"] != pairs["q_start"].max()]
    dims = B.make_dims(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.q_rows, wl.kv_rows)
    assert B.fcp_plan_info(dims, pairs, B.FCP_OP_BWD)["slots"] > 0
    o, lse = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], pairs)
    ref = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], pairs)
    fill = 7.0
    out = [torch.full(t.shape, fill, dtype=torch.float32, device=t.device) for t in ref]
    B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], pairs, dq=out[0],
                         dk=out[1], dv=out[2], overwrite=True)
    torch.cuda.synchronize()
    qcov = np.zeros(wl.q_rows, dtype=bool)
    kcov = np.zeros(wl.kv_rows, dtype=bool)
    for p in pairs:
        qcov[p["q_start"]:p["q_start"] + p["q_len"]] = True
        kcov[p["kv_start"]:p["kv_start"] + p["kv_len"]] = True
    assert qcov.any() and kcov.any()
    if drop_last_q_range:
        assert not qcov.all()
    for got, want, cov, name in ((out[0], ref[0], qcov, "dq"), (out[1], ref[1], kcov, "dk"),
                                 (out[2], ref[2], kcov, "dv")):
        c = torch.as_tensor(cov, device=got.device)
        assert torch.equal(got[c], want[c]), name + ": covered rows differ"
        assert bool((got[~c] == fill).all()), name + ": uncovered rows were written"
    # Unknown flag bits are rejected before any work is enqueued.
    _, pp, n = B._pairs_arg(pairs)
    st = B.load().fcp_block_attn_bwd_ex(
        ctypes.byref(dims), B._ptr(dev["q"]), B._ptr(dev["k"]), B._ptr(dev["v"]), B._ptr(o),
        B._ptr(lse), B._ptr(dev["do"]), pp, n, B._ptr(out[0]), B._ptr(out[1]), B._ptr(out[2]),
        2, None, 0, None)
    assert st == 1  # FCP_ERR_INVALID_ARG

def _key_sample(wl):
    rows = []
    for s, length in enumerate(wl.seqlens):
        for p in (length - 1, length - 17, length // 2 if length <= 4096 else length - 200):
            for seg in wl.kv_segments():
                if seg.seq == s and seg.pos0 <= p < seg.pos0 + seg.length:
                    rows.append(seg.row0 + p - seg.pos0)
    return np.array(sorted(set(rows)), dtype=np.int64)


@pytest.mark.parametrize("cfg", ["config2", "config2-s1", "config2-s2"])
def test_full_size_sampled(gpu, cfg):
    import torch
    seed = {"config2-s1": 1, "config2-s2": 2}.get(cfg, 0)
    wl = {"config2": lambda: W.config2(0),
          "config2-s1": lambda: W.config2(1),
          "config2-s2": lambda: W.config2(2)}[cfg]()
    dev, x = U.inputs(wl, seed=seed)
    pairs = build_pairs(wl)
    _, _, dq, dk, dv = _fwd_bwd(wl, dev, pairs)
    torch.cuda.synchronize()
    idx = oracle.SeqIndex(wl)
    rows = U.sample_rows(wl, 24)
    rq = oracle.dq_rows(x["q"], x["k"], x["v"], x["do"], idx, rows)
    check_grad(dq.index_select(0, torch.as_tensor(rows, device=dq.device)).cpu().numpy(), rq,
               cfg + " dQ rows")
    if wl.causal:
        # Keys near the end of each sequence are seen by few queries, so the oracle can
        # afford them. (Under the non-causal mask every query sees every key, which puts
        # a per-key oracle out of reach at 32K; the dV sum below covers all keys.)
        krows = _key_sample(wl)
        rk, rv = oracle.dkv_rows(x["q"], x["k"], x["v"], x["do"], idx, krows)
        kidx = torch.as_tensor(krows, device=dk.device)
        check_grad(dk.index_select(0, kidx).cpu().numpy(), rk, cfg + " dK keys")
        check_grad(dv.index_select(0, kidx).cpu().numpy(), rv, cfg + " dV keys")
    # Rows of P sum to one: per sequence and KV head, sum_j dV_j = sum over the group's
    # query heads and the sequence's owned queries of dO.
    g = wl.num_q_heads // wl.num_kv_heads
    dv_h = dv.cpu().numpy()
    do_h = x["do"]
    for s in range(len(wl.seqlens)):
        kr = idx.kv_row_of_pos[s]
        qr = np.nonzero(idx.q_row_seq == s)[0]
        lhs = dv_h[kr].sum(axis=0)
        rhs = do_h[qr].reshape(len(qr), wl.num_kv_heads, g, -1).sum(axis=(0, 2))
        rel = np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs)
        assert rel < 2e-2, (s, rel)


def test_full_size_heterogeneous(gpu):
    """The heaviest worker of the heterogeneous batch (33 Q blocks of many packed
    sequences, up to 511K tokens long), forward + backward as the bench runs it: dQ on
    sampled rows against the oracle, and per sequence and KV head the sum of dV over all
    keys against the sum of dO over the owned queries (rows of P sum to one)."""
    import torch
    wl = W.config5(0)
    dev = W.make_device_inputs(wl, seed=0)
    pairs = build_pairs(wl)
    _, _, dq, dk, dv = _fwd_bwd(wl, dev, pairs)
    torch.cuda.synchronize()
    assert not torch.isnan(dk).any() and not torch.isnan(dv).any()
    idx = oracle.SeqIndex(wl)
    rng = np.random.default_rng(11)
    rows = U.sample_rows(wl, 8, seed=11)
    if len(rows) > 24:
        rows = np.sort(rng.choice(rows, 24, replace=False))
    rq = oracle.dq_rows(U.DeviceRows(dev["q"]), U.DeviceRows(dev["k"]), U.DeviceRows(dev["v"]),
                        U.DeviceRows(dev["do"]), idx, rows)
    check_grad(dq.index_select(0, torch.as_tensor(rows, device=dq.device)).cpu().numpy(), rq,
               "config5 dQ rows")
    g = wl.num_q_heads // wl.num_kv_heads
    owned = set(np.unique(idx.q_row_seq[idx.owned_rows()]).tolist())
    for s in sorted(owned):
        # Keys past the last owned query of the sequence are not in the KV buffer (-1);
        # no owned query sees them.
        kpos = np.asarray(idx.kv_row_of_pos[s])
        kpos = kpos[kpos >= 0]
        assert kpos.size and kpos.max() < wl.kv_rows
        qpos = np.nonzero(idx.q_row_seq == s)[0]
        assert qpos.size and qpos.max() < wl.q_rows
        kr = torch.as_tensor(kpos, device=dv.device)
        qr = torch.as_tensor(qpos, device=dv.device)
        lhs = dv.index_select(0, kr).double().sum(dim=0)
        rhs = dev["do"].index_select(0, qr).double().reshape(len(qr), wl.num_kv_heads, g, -1) \
            .sum(dim=(0, 2))
        rel = (torch.linalg.norm(lhs - rhs) / torch.linalg.norm(rhs)).item()
        assert rel < 2e-2, (s, rel)


def _plan(wl, pairs):
    dims = B.make_dims(wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.q_rows, wl.kv_rows)
    return B.fcp_plan_info(dims, pairs, B.FCP_OP_BWD)


def _seq_rows(wl, idx, s):
    qrows = np.nonzero(idx.q_row_seq == s)[0]
    krows = np.asarray(idx.kv_row_of_pos[s])
    return qrows, krows[krows >= 0]


def test_whole_sequence_with_head_split_tiles(gpu):
    """The 1K worker share at full size (seed 0: sequences of 4763, 3496 and 8125
    tokens): every dQ row and every dK/dV key of the 8125-token sequence, element-wise
    against the oracle's full backward of that sequence. Its first key tiles are seen by
    so many query tiles that the scheduler splits them into two parts of four query
    heads each (the second starting at head 4), summed by the reduce kernel."""
    import torch
    wl = W.config2(0)
    dev, x = U.inputs(wl, seed=0)
    pairs = build_pairs(wl)
    info = _plan(wl, pairs)
    assert info["split_tiles"] > 0 and info["multihead_offset_parts"] > 0, info
    _, _, dq, dk, dv = _fwd_bwd(wl, dev, pairs)
    torch.cuda.synchronize()
    idx = oracle.SeqIndex(wl)
    s = int(np.argmax(wl.seqlens))
    rq, rk, rv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx, seqs=[s])
    qrows, krows = _seq_rows(wl, idx, s)
    check_grad(dq.cpu().numpy()[qrows], rq[qrows], "seq %d dQ" % s)
    check_grad(dk.cpu().numpy()[krows], rk[krows], "seq %d dK" % s)
    check_grad(dv.cpu().numpy()[krows], rv[krows], "seq %d dV" % s)


def test_multihead_parts_mid_size(gpu):
    """A mid-size share (3000, 1100 and 2900 tokens in 1K blocks, 64/8 heads, D 128) whose
    heavy key tiles the scheduler splits into 2 to 4 parts of 2 or 3 query heads, most of
    them starting past the group's first head: all of dQ, dK and dV element-wise."""
    import torch
    wl = W.custom([3000, 1100, 2900], 1024, 64, 8, 128, True)
    dev, x = U.inputs(wl, seed=8)
    pairs = build_pairs(wl)
    info = _plan(wl, pairs)
    assert info["multihead_parts"] > 0 and info["multihead_offset_parts"] > 0, info
    assert info["slots"] < 8 * info["split_tiles"], info   # not one head per part
    _, _, dq, dk, dv = _fwd_bwd(wl, dev, pairs)
    torch.cuda.synchronize()
    idx = oracle.SeqIndex(wl)
    rq, rk, rv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)
    rows = idx.owned_rows()
    check_grad(dq.cpu().numpy()[rows], rq[rows], "mid dQ")
    check_grad(dk.cpu().numpy(), rk, "mid dK")
    check_grad(dv.cpu().numpy(), rv, "mid dV")


def _one_head(do, h0):
    import torch
    out = torch.zeros_like(do)
    out[:, h0] = do[:, h0]
    return out


def test_heterogeneous_dk_dv(gpu):
    """The heaviest worker of the heterogeneous batch: dK and dV element-wise on every
    key of each of its fully owned short packed sequences (all query heads); then, with
    the upstream gradient kept on one query head, at early keys (seen by every owned
    query) and late keys of a 15K-token and a 262K-token sequence whose KV blocks were
    pulled."""
    import torch
    wl = W.config5(0)
    dev = W.make_device_inputs(wl, seed=0)
    pairs = build_pairs(wl)
    o, lse = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], pairs)
    _, dk, dv = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], pairs)
    torch.cuda.synchronize()
    idx = oracle.SeqIndex(wl)
    xr = {n: U.DeviceRows(dev[n]) for n in ("q", "k", "v", "do")}
    rows = idx.owned_rows()
    seqs, counts = np.unique(idx.q_row_seq[rows], return_counts=True)
    short = [int(s) for s, c in zip(seqs, counts) if c == wl.seqlens[s] and c <= 4096]
    assert len(short) >= 3, short
    keys = np.concatenate([_seq_rows(wl, idx, s)[1] for s in short])
    rk, rv = oracle.dkv_keys(xr["q"], xr["k"], xr["v"], xr["do"], idx, keys)
    kidx = torch.as_tensor(keys, device=dk.device)
    check_grad(dk.index_select(0, kidx).cpu().numpy(), rk, "config5 short seqs dK")
    check_grad(dv.index_select(0, kidx).cpu().numpy(), rv, "config5 short seqs dV")
    del dk, dv

    h0 = 29
    g0 = h0 // (wl.num_q_heads // wl.num_kv_heads)
    _, dk1, dv1 = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse,
                                       _one_head(dev["do"], h0), pairs)
    torch.cuda.synchronize()
    picks = []
    for length in (15189, 262094):
        s = wl.seqlens.index(length)
        qrows, krows = _seq_rows(wl, idx, s)
        assert len(qrows) > 0 and len(krows) > 0
        p0, p1 = int(idx.q_row_pos[qrows].min()), int(idx.q_row_pos[qrows].max())
        for p in (0, 1, 127, 128, 4095, p0 - 1, p0, p0 + 100, p1):
            picks.append(int(idx.kv_row_of_pos[s][p]))
    keys = np.array(sorted(set(picks)))
    rk, rv = oracle.dkv_keys(xr["q"], xr["k"], xr["v"], xr["do"], idx, keys, heads=[h0])
    kidx = torch.as_tensor(keys, device=dk1.device)
    check_grad(dk1.index_select(0, kidx)[:, g0].cpu().numpy(), rk[:, g0], "config5 dK keys")
    check_grad(dv1.index_select(0, kidx)[:, g0].cpu().numpy(), rv[:, g0], "config5 dV keys")


def test_zigzag_worker_backward(gpu):
    """The Zig-Zag worker (Q blocks 0 and 127 of a 512K sequence, 33 KV ranges of 16K)
    forward + backward as the bench runs it: dQ on sampled rows of both Q blocks; dK and
    dV at keys across the sequence with the upstream gradient kept on one query head."""
    import torch
    wl = W.config4(0)
    dev = W.make_device_inputs(wl, seed=0)
    pairs = build_pairs(wl)
    o_part, lse_part = B.fcp_block_attn_fwd(dev["q"], dev["k"], dev["v"], pairs,
                                            part_rows=int(pairs["q_len"].sum()))
    o, lse = B.fcp_merge_partials(pairs, o_part, lse_part, wl.q_rows, wl.num_kv_heads)
    del o_part, lse_part
    dq, _, _ = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], pairs)
    torch.cuda.synchronize()
    idx = oracle.SeqIndex(wl)
    xr = {n: U.DeviceRows(dev[n]) for n in ("q", "k", "v", "do")}
    rows = np.array([0, 1, 2047, 4095, 4096, 4097, 6000, 8191])
    rq = oracle.dq_rows(xr["q"], xr["k"], xr["v"], xr["do"], idx, rows)
    check_grad(dq.index_select(0, torch.as_tensor(rows, device=dq.device)).cpu().numpy(), rq,
               "config4 dQ rows")
    del dq
    h0 = 50
    g0 = h0 // (wl.num_q_heads // wl.num_kv_heads)
    _, dk1, dv1 = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse,
                                       _one_head(dev["do"], h0), pairs)
    torch.cuda.synchronize()
    pos = [0, 1, 4095, 4096, 65536, 262143, 262144, 500000, 520191, 520192, 524287]
    keys = np.array([int(idx.kv_row_of_pos[0][p]) for p in pos])
    rk, rv = oracle.dkv_keys(xr["q"], xr["k"], xr["v"], xr["do"], idx, keys, heads=[h0])
    kidx = torch.as_tensor(keys, device=dk1.device)
    check_grad(dk1.index_select(0, kidx)[:, g0].cpu().numpy(), rk[:, g0], "config4 dK keys")
    check_grad(dv1.index_select(0, kidx)[:, g0].cpu().numpy(), rv[:, g0], "config4 dV keys")
