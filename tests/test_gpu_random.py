"""Seeded random workloads through the whole path (per-pair partials + merge, fused
forward, backward) against the float64 oracle, through the C ABI.

Each case draws its sequence lengths (1..700 tokens, a few very short), block size, head
layout (grouped-query groups 1, 2, 4, 8 and 16), head dimension, mask, sharding (stream
cut or first-fit-decreasing) and either a coalescing degree or a KV split from one numpy
generator seeded by the case number, so a failure names a reproducible case. The sizes
keep the float64 oracle to about a second per case while the kernels still see several
tiles, ragged tails and multi-segment blocks.
"""
import numpy as np
import pytest

import fcp_workloads as W
import oracle
from block_wise_varlen_amd import binding as B
from block_wise_varlen_amd.descriptors import build_pairs, part_rows
from tests import gpu_util as U
from tests.test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu

HEADS = [(8, 1), (8, 2), (8, 4), (4, 4), (16, 2), (2, 1), (32, 4), (16, 1)]
BLOCKS = [32, 64, 128, 256, 512]
N_CASES = 24


def draw_case(case):
    """(workload, description) of random case ``case``."""
    rng = np.random.default_rng(1000 + case)
    n_seq = int(rng.integers(1, 6))
    lens = []
    for _ in range(n_seq):
        lens.append(int(rng.integers(1, 8)) if rng.random() < 0.2 else int(rng.integers(8, 700)))
    block = int(rng.choice(BLOCKS))
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    d = int(rng.choice([64, 128]))
    causal = bool(rng.random() < 0.7)
    shard = "ffd" if rng.random() < 0.4 else "stream"
    coalesce, kv_split = 1, 1
    if rng.random() < 0.5:
        coalesce = int(rng.integers(1, 4))
    else:
        kv_split = int(rng.integers(1, 4))
    wl = W.custom(lens, block, hq, hkv, d, causal, coalesce=coalesce, kv_split=kv_split,
                  shard=shard)
    desc = "lens=%s b=%d h=%d/%d d=%d %s %s c=%d split=%d" % (
        lens, block, hq, hkv, d, "causal" if causal else "noncausal", shard, coalesce, kv_split)
    return wl, desc


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_workload(gpu, case):
    import torch
    wl, desc = draw_case(case)
    print("case %d: %s" % (case, desc), flush=True)
    dev, x = U.inputs(wl, seed=case)
    pairs = build_pairs(wl)
    o_part, lse_part = B.fcp_block_attn_fwd(dev["q"], dev["k"], dev["v"], pairs,
                                            part_rows=part_rows(pairs))
    o, lse = B.fcp_merge_partials(pairs, o_part, lse_part, wl.q_rows, wl.num_kv_heads)
    of, lf = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], pairs)
    dq, dk, dv = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], of, lf, dev["do"], pairs)
    torch.cuda.synchronize()
    idx = oracle.SeqIndex(wl)
    rows = idx.owned_rows()
    o_ref, l_ref = oracle.forward(x["q"], x["k"], x["v"], idx)
    U.check_attn(U.bf16_to_f64(o)[rows], lse.cpu().numpy()[rows], o_ref, l_ref,
                 "case %d merge (%s)" % (case, desc))
    U.check_attn(U.bf16_to_f64(of)[rows], lf.cpu().numpy()[rows], o_ref, l_ref,
                 "case %d fused (%s)" % (case, desc))
    rq, rk, rv = oracle.backward(x["q"], x["k"], x["v"], x["do"], idx)
    check_grad(dq.cpu().numpy()[rows], rq[rows], "case %d dQ (%s)" % (case, desc))
    check_grad(dk.cpu().numpy(), rk, "case %d dK (%s)" % (case, desc))
    check_grad(dv.cpu().numpy(), rv, "case %d dV (%s)" % (case, desc))
