"""GPU parity at every point of the 32K-token block-size sweep that bench.py reports
(one sequence; blocks of 512 .. 16384 tokens; causal and non-causal), through the C ABI,
in the bench's launch configuration: per-pair partials (fp32, and bf16 with fp32 LSE) +
LSE merge, and the fused forward, on sampled rows; the backward from the merged output on sampled dQ rows, with
the per-sequence dV sum; and dK and dV element-wise at sampled keys, heavy ones at the
start of the sequence (seen by nearly every query) and light ones at its end, in a
second backward whose upstream gradient is kept on one query head (the other heads then
contribute exactly nothing, so the oracle runs that head alone and the other KV heads'
dK/dV must be exactly zero).

The oracle never reads the pair table, so one reference per mask serves all block sizes;
the inputs are drawn once (seed 0) and shared by every point.
"""
import numpy as np
import pytest

import fcp_workloads as W
import oracle
from fcp_workloads.tensors import host_to_device
from block_wise_varlen_amd import binding as B
from block_wise_varlen_amd.descriptors import build_pairs, part_rows
from tests import gpu_util as U
from tests.test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu

BLOCKS = (512, 1024, 2048, 4096, 8192, 16384)
L = 32768
# query rows: every block boundary of every block size, its neighbours, and random rows
ROWS = np.unique(np.concatenate([
    np.arange(0, L, 512), np.arange(511, L, 512)[::3], [1, 31, 32, 33, 16385, L - 2],
    np.random.default_rng(21).integers(0, L, 24)]))
# keys: heavy (start) to light (end)
KEYS = np.array([0, 1, 31, 127, 128, 129, 511, 512, 1023, 1024, 4095, 4096, 8191, 8192,
                 12345, 16383, 16384, 24576, 30000, 32639, 32640, L - 1])
# the query head the second backward keeps, per block size (KV heads 0 and 5)
HEAD = {512: 5, 1024: 43, 2048: 5, 4096: 43, 8192: 5, 16384: 43}

_cache = {}


@pytest.fixture(scope="module")
def inputs(gpu):
    wl = W.config3(4096, True)
    bits = W.make_host_inputs(wl, seed=0)
    dev = {n: host_to_device(b) for n, b in bits.items()}
    host = {n: W.bf16_bits_to_f64(b) for n, b in bits.items()}
    return dev, host


def _ref(kind, causal, x, h0=None):
    key = (kind, causal, h0)
    if key not in _cache:
        idx = oracle.SeqIndex(W.config3(4096, causal))
        if kind == "fwd":
            _cache[key] = oracle.forward(x["q"], x["k"], x["v"], idx, rows=ROWS)
        elif kind == "dq":
            _cache[key] = oracle.dq_rows(x["q"], x["k"], x["v"], x["do"], idx, ROWS)
        else:
            _cache[key] = oracle.dkv_keys(x["q"], x["k"], x["v"], x["do"], idx, KEYS,
                                          heads=[h0])
    return _cache[key]


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
@pytest.mark.parametrize("block", BLOCKS)
def test_sweep_point(inputs, block, causal):
    import torch
    dev, x = inputs
    wl = W.config3(block, causal)
    pairs = build_pairs(wl)
    name = "b%d-%s" % (block, "causal" if causal else "noncausal")
    ridx = torch.as_tensor(ROWS, device=dev["q"].device)

    o_part, lse_part = B.fcp_block_attn_fwd(dev["q"], dev["k"], dev["v"], pairs,
                                            part_rows=part_rows(pairs))
    o, lse = B.fcp_merge_partials(pairs, o_part, lse_part, wl.q_rows, wl.num_kv_heads)
    del o_part, lse_part
    o16, l16 = B.fcp_block_attn_fwd(dev["q"], dev["k"], dev["v"], pairs,
                                    part_rows=part_rows(pairs), part_dtype=torch.bfloat16)
    om, lm = B.fcp_merge_partials(pairs, o16, l16, wl.q_rows, wl.num_kv_heads)
    del o16, l16
    of, lf = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], pairs)
    torch.cuda.synchronize()
    o_ref, l_ref = _ref("fwd", causal, x)
    U.check_attn(U.bf16_to_f64(om.index_select(0, ridx)), lm.index_select(0, ridx).cpu().numpy(),
                 o_ref, l_ref, name + " bf16 partials+merge")
    del om, lm
    U.check_attn(U.bf16_to_f64(o.index_select(0, ridx)), lse.index_select(0, ridx).cpu().numpy(),
                 o_ref, l_ref, name + " partials+merge")
    U.check_attn(U.bf16_to_f64(of.index_select(0, ridx)), lf.index_select(0, ridx).cpu().numpy(),
                 o_ref, l_ref, name + " fused")
    del of, lf

    dq, dk, dv = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], pairs)
    torch.cuda.synchronize()
    check_grad(dq.index_select(0, ridx).cpu().numpy(), _ref("dq", causal, x), name + " dQ rows")
    g = wl.num_q_heads // wl.num_kv_heads
    lhs = dv.double().sum(dim=0)
    rhs = dev["do"].double().reshape(L, wl.num_kv_heads, g, -1).sum(dim=(0, 2))
    rel = (torch.linalg.norm(lhs - rhs) / torch.linalg.norm(rhs)).item()
    assert rel < 2e-2, (name, "dV sum", rel)
    del dq, dk, dv

    h0 = HEAD[block]
    g0 = h0 // g
    do1 = torch.zeros_like(dev["do"])
    do1[:, h0] = dev["do"][:, h0]
    _, dk1, dv1 = B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, do1, pairs)
    torch.cuda.synchronize()
    others = [h for h in range(wl.num_kv_heads) if h != g0]
    assert not dk1[:, others].any().item() and not dv1[:, others].any().item(), \
        name + ": KV heads outside the kept query head's group got gradient"
    rk, rv = _ref("dkv", causal, x, h0)
    kidx = torch.as_tensor(KEYS, device=dk1.device)
    check_grad(dk1.index_select(0, kidx)[:, g0].cpu().numpy(), rk[:, g0], name + " dK keys")
    check_grad(dv1.index_select(0, kidx)[:, g0].cpu().numpy(), rv[:, g0], name + " dV keys")
