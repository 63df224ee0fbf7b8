"""GPU parity of the block-level pipelined forward (FCP paper Sec. 4.2, "Block-level
pipelining"): stages copy pulled KV blocks into the worker's double-buffered KV buffer on
a second stream while the previous stage computes, then the partials are merged. Checked
against the float64 oracle, and bit for bit across copy engines, stream arrangements and
buffer layouts (the same kernels see the same pairs in the same order)."""
import numpy as np
import pytest

import fcp_workloads as W
import oracle
from block_wise_varlen_amd import binding as B
from block_wise_varlen_amd.descriptors import build_pipeline
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def zigzag(n_workers, block, worker, coalesce, hq, hkv, d):
    seqlen = 2 * n_workers * block
    wl = W.custom([seqlen], block, hq, hkv, d, True,
                  q_ids=[worker, 2 * n_workers - 1 - worker],
                  kv_ids=list(range(2 * n_workers - worker)), coalesce=coalesce)
    src, dst, blk = W.zigzag_graph(n_workers, seqlen=seqlen, block=block)
    stage, _ = B.fcp_comm_plan(n_workers, src, dst)
    m = dst == worker
    return wl, wl.q_block_ids, {int(b): int(s) for b, s in zip(blk[m], stage[m])}


def packed(seed, causal, hq, hkv, d):
    rng = np.random.default_rng(seed)
    seqlens = [int(x) for x in rng.integers(1, 700, 7)]
    wl = W.custom(seqlens, 256, hq, hkv, d, causal, shard="ffd", coalesce=2)
    ids = wl.kv_block_ids
    local = [ids[0], ids[len(ids) // 2]]
    order = rng.permutation([i for i in ids if i not in local])
    return wl, local, {int(b): k for k, b in enumerate(order)}


def run(wl, dev, P, overlap=True, flags=0, depth=None, part_dtype=None):
    import torch
    shape = (P["kv_rows"], wl.num_kv_heads, wl.head_dim)
    k = torch.zeros(shape, dtype=torch.bfloat16, device=dev["q"].device)
    v = torch.zeros_like(k)
    for c in P["local_copies"]:
        s, t, n = int(c["src_row"]), int(c["dst_row"]), int(c["n_rows"])
        k[t:t + n] = dev["k"][s:s + n]
        v[t:t + n] = dev["v"][s:s + n]
    o_part = torch.empty((P["part_rows"], wl.num_q_heads, wl.head_dim),
                         dtype=part_dtype or torch.float32, device=k.device)
    lse_part = torch.empty((P["part_rows"], wl.num_q_heads), dtype=torch.float32,
                           device=k.device)
    cs = torch.cuda.Stream() if overlap else None
    o, lse = B.fcp_pipeline_fwd(dev["q"], k, v, dev["k"], dev["v"], P["stages"], P["copies"],
                                P["pairs"], o_part, lse_part, flags=flags, copy_stream=cs,
                                depth=P["depth"] if depth is None else depth)
    torch.cuda.synchronize()
    return o, lse


CASES = {
    "zigzag-N4-w0-c2": lambda: zigzag(4, 512, 0, 2, 8, 1, 128),
    "zigzag-N4-w2-c1": lambda: zigzag(4, 256, 2, 1, 8, 2, 128),
    "zigzag-N3-w1-c3-d64": lambda: zigzag(3, 384, 1, 3, 4, 2, 64),
    "packed-causal": lambda: packed(0, True, 8, 2, 128),
    "packed-noncausal-d64": lambda: packed(1, False, 4, 1, 64),
}


@pytest.mark.parametrize("name", list(CASES))
def test_pipeline_matches_oracle(gpu, name):
    wl, local, recv = CASES[name]()
    print("case", name, "q_rows", wl.q_rows, "kv_rows", wl.kv_rows, flush=True)
    dev, x = U.inputs(wl, seed=11, which=("q", "k", "v"))
    P = build_pipeline(wl, local, recv, coalesce=wl.coalesce)
    o, lse = run(wl, dev, P)
    idx = oracle.SeqIndex(wl)
    rows = idx.owned_rows()
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], idx)
    U.check_attn(U.bf16_to_f64(o)[rows], lse.cpu().numpy()[rows], o_ref, l_ref, name)


@pytest.mark.parametrize("name", ["zigzag-N4-w0-c2", "packed-causal", "packed-noncausal-d64"])
def test_pipeline_bf16_partials_match_oracle(gpu, name):
    """The pipelined forward with its stage partials stored in bf16 (FCP_PIPE_PART_BF16)."""
    import torch
    wl, local, recv = CASES[name]()
    dev, x = U.inputs(wl, seed=13, which=("q", "k", "v"))
    P = build_pipeline(wl, local, recv, coalesce=wl.coalesce)
    o, lse = run(wl, dev, P, part_dtype=torch.bfloat16)
    idx = oracle.SeqIndex(wl)
    rows = idx.owned_rows()
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], idx)
    U.check_attn(U.bf16_to_f64(o)[rows], lse.cpu().numpy()[rows], o_ref, l_ref,
                 name + " bf16 partials")


@pytest.mark.parametrize("name", ["zigzag-N4-w0-c2", "packed-causal"])
def test_pipeline_modes_bit_identical(gpu, name):
    import torch
    wl, local, recv = CASES[name]()
    dev, _ = U.inputs(wl, seed=12, which=("q", "k", "v"))
    P = build_pipeline(wl, local, recv, coalesce=wl.coalesce)
    ref = run(wl, dev, P)
    variants = {
        "serial": run(wl, dev, P, overlap=False),
        "shader-copy": run(wl, dev, P, flags=B.FCP_PIPE_COPY_SHADER),
        "resident": run(wl, dev, build_pipeline(wl, local, recv, coalesce=wl.coalesce,
                                                 depth=None)),
        "depth3": run(wl, dev, build_pipeline(wl, local, recv, coalesce=wl.coalesce, depth=3)),
        "depth1": run(wl, dev, build_pipeline(wl, local, recv, coalesce=wl.coalesce, depth=1)),
    }
    for what, (o, lse) in variants.items():
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), what


def test_pipeline_full_size_zigzag(gpu):
    """Zig-Zag worker 0 of 64 (512K tokens, 4K blocks, 64/8 heads, D 128): 126 blocks
    pulled in the congestion-free order, 4 per stage, double-buffered; sampled rows
    against the oracle (inputs drawn on the device; the oracle reads the rows it needs)."""
    import torch
    wl = W.config4(0)
    src, dst, blk = W.zigzag_graph(64)
    stage, _ = B.fcp_comm_plan(64, src, dst)
    m = dst == 0
    recv = {int(b): int(s) for b, s in zip(blk[m], stage[m])}
    P = build_pipeline(wl, wl.q_block_ids, recv, coalesce=4)
    assert len(P["stages"]) == 33
    dev = W.make_device_inputs(wl, seed=0, which=("q", "k", "v"))
    o, lse = run(wl, dev, P)
    rows = U.sample_rows(wl, 16, seed=3)
    idx = oracle.SeqIndex(wl)
    o_ref, l_ref = oracle.forward(U.DeviceRows(dev["q"]), U.DeviceRows(dev["k"]),
                                  U.DeviceRows(dev["v"]), idx, rows=rows)
    ridx = torch.as_tensor(rows, device=o.device)
    U.check_attn(U.bf16_to_f64(o.index_select(0, ridx)), lse.index_select(0, ridx).cpu().numpy(),
                 o_ref, l_ref, "zigzag pipeline")


def test_pipeline_full_size_heterogeneous(gpu):
    """The heaviest worker of the heterogeneous lognormal batch (64 workers, 4K blocks,
    packed short sequences, LPT): the KV blocks it does not hold are pulled in the
    congestion-free order of the whole batch's pull graph, 4 sub-stages per stage;
    sampled rows against the oracle."""
    import torch
    wl = W.config5(0)
    src, dst, blk = W.hetero_graph()
    stage, _ = B.fcp_comm_plan(64, src, dst)
    w = wl.meta["worker"]
    m = dst == w
    recv = {int(b): int(s) for b, s in zip(blk[m], stage[m])}
    local = [i for i in wl.kv_block_ids if wl.meta["assign"][i] == w]
    assert set(recv) == set(wl.kv_block_ids) - set(local)
    P = build_pipeline(wl, local, recv, coalesce=4)
    print("stages", len(P["stages"]), "pairs", len(P["pairs"]), flush=True)
    dev = W.make_device_inputs(wl, seed=0, which=("q", "k", "v"))
    o, lse = run(wl, dev, P)
    rng = np.random.default_rng(5)
    rows = U.sample_rows(wl, 12, seed=5)
    if len(rows) > 40:
        rows = np.sort(rng.choice(rows, 40, replace=False))
    idx = oracle.SeqIndex(wl)
    o_ref, l_ref = oracle.forward(U.DeviceRows(dev["q"]), U.DeviceRows(dev["k"]),
                                  U.DeviceRows(dev["v"]), idx, rows=rows)
    ridx = torch.as_tensor(rows, device=o.device)
    U.check_attn(U.bf16_to_f64(o.index_select(0, ridx)), lse.index_select(0, ridx).cpu().numpy(),
                 o_ref, l_ref, "heterogeneous pipeline")


def test_pipeline_rejects_racing_tables(gpu):
    import torch
    wl, local, recv = CASES["zigzag-N4-w0-c2"]()
    dev, _ = U.inputs(wl, seed=13, which=("q", "k", "v"))
    P = build_pipeline(wl, local, recv, coalesce=wl.coalesce, depth=1)
    with pytest.raises(B.FcpError) as e:   # one region, but two stages in flight
        run(wl, dev, P, depth=2)
    assert e.value.status == B.FCP_ERR_INVALID_ARG and "previous" in str(e.value)
