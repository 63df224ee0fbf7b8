"""fcp_block_attn_fwd_fused_noalloc (work lists in the library's static device array, no
workspace, no allocation) against fcp_block_attn_fwd_fused (workspace argument), through
the C ABI: two calls in a row on one stream, the second with a smaller input, each
compared with the workspace entry point's output (bitwise, which implies the forward
parity gates of the oracle comparison)."""
import numpy as np
import pytest

import fcp_workloads as W
from block_wise_varlen_amd import binding as B
from block_wise_varlen_amd.descriptors import build_pairs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _case(wl, seed):
    import torch
    dev, _ = U.inputs(wl, seed=seed, which=("q", "k", "v"))
    pairs = build_pairs(wl)
    ref = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], pairs)
    # Outputs start from a sentinel, so a row the call fails to write shows up.
    o = torch.full_like(dev["q"], 3.0)
    lse = torch.full((wl.q_rows, wl.num_q_heads), 5.0, dtype=torch.float32, device=dev["q"].device)
    return dev, pairs, ref, o, lse


def _compare(wl, ref, o, lse, what):
    import torch
    o_ref, l_ref = ref
    rows = np.array(sorted({r for s in wl.q_segments() for r in range(s.row0, s.row0 + s.length)}))
    ridx = torch.as_tensor(rows, device=o.device)
    got_o, got_l = o.index_select(0, ridx), lse.index_select(0, ridx)
    ref_o, ref_l = o_ref.index_select(0, ridx), l_ref.index_select(0, ridx)
    U.check_attn(U.bf16_to_f64(got_o), got_l.cpu().numpy(), U.bf16_to_f64(ref_o),
                 ref_l.cpu().numpy().astype(np.float64), what)
    assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l), what + ": not bitwise equal"


def test_noalloc_matches_workspace_entry_point(gpu):
    import torch
    big = W.config2(0)                 # 16 x 1024 tokens, 64/8 heads, D 128, causal
    small = W.config1(causal=False)    # 1024 tokens, 4/1 heads, D 64, non-causal
    cases = [(big, 0), (small, 3)]
    prepared = [_case(wl, seed) for wl, seed in cases]
    torch.cuda.synchronize()
    # Back to back on one stream: the second call's work lists replace the first's in the
    # shared array only after the first call's kernel has read them.
    for (wl, _), (dev, pairs, _, o, lse) in zip(cases, prepared):
        B.fcp_block_attn_fwd_fused_noalloc(dev["q"], dev["k"], dev["v"], pairs, o=o, lse=lse)
    torch.cuda.synchronize()
    for (wl, _), (dev, pairs, ref, o, lse) in zip(cases, prepared):
        _compare(wl, ref, o, lse, wl.name)
    # Again, smaller first: stale lists of a larger table must not leak into a smaller one.
    for (wl, _), (dev, pairs, ref, o, lse) in reversed(list(zip(cases, prepared))):
        o.fill_(3.0)
        lse.fill_(5.0)
        B.fcp_block_attn_fwd_fused_noalloc(dev["q"], dev["k"], dev["v"], pairs, o=o, lse=lse)
        torch.cuda.synchronize()
        _compare(wl, ref, o, lse, wl.name + " (second pass)")
