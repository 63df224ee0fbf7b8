"""The optional timing hook through the C ABI: per-kernel launch times from HIP events on
the call's stream, and the shader clock the forward, dQ and dK/dV kernels sample while
timing is on (s_memtime over the 100 MHz s_memrealtime, per workgroup)."""
import pytest

import fcp_workloads as W
from block_wise_varlen_amd import binding as B
from block_wise_varlen_amd.descriptors import build_pairs
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def test_timing_hook_times_and_clocks(gpu):
    import torch
    wl = W.config2(0)
    dev, _ = U.inputs(wl, seed=0)
    pairs = build_pairs(wl)
    B.fcp_timing_read_clock()   # drop anything recorded before
    o, lse = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], pairs)
    torch.cuda.synchronize()
    assert B.fcp_timing_read_clock() == {}, "timing is off: nothing recorded"
    B.fcp_timing_enable(True)
    try:
        for _ in range(2):
            o, lse = B.fcp_block_attn_fwd_fused(dev["q"], dev["k"], dev["v"], pairs)
            B.fcp_block_attn_bwd(dev["q"], dev["k"], dev["v"], o, lse, dev["do"], pairs)
        torch.cuda.synchronize()
    finally:
        B.fcp_timing_enable(False)
    kt = B.fcp_timing_read_clock()
    for name in ("fwd_fused", "bwd_dq", "bwd_dkdv"):
        ms, n, mhz = kt[name]
        assert n == 2 and ms > 0, (name, kt[name])
        # the part's shader clock lies between its 500 MHz floor and its 2.4 GHz peak
        assert 500 <= mhz <= 2500, (name, mhz)
    assert kt["bwd_dkdv_reduce"][2] == 0.0   # the reduce takes no samples
    assert B.fcp_timing_read_clock() == {}, "a read resets the records"
