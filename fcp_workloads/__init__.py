"""Seeded synthetic workloads for block-level varlen attention.

This package is the one module shared by the HIP path (its tests and bench) and the
float64 oracle. It draws sequence lengths, cuts and packs them into fixed-size blocks,
picks one worker's blocks, places them in Q and KV buffers, draws the bf16 tensors and
counts the visible (query, key) pairs used for FLOP accounting. It holds none of the
attention arithmetic itself.

Sources (FCP paper, arXiv 2605.08524, and its review page):
  * lognormal, long-tailed context lengths up to 512K: FCP paper Sec. 2.1, Figure 2;
  * fixed-size block sharding, short sequences packed into the minimal number of
    blocks: FCP paper Sec. 4.1 ("Sharding Policy");
  * LPT assignment under a per-worker token cap: FCP paper Sec. 4.1 ("Assignment
    Policy"), Sec. 3.2 ("Memory");
  * Zig-Zag pairing of blocks: FCP paper Sec. 3.2 and Sec. 3.4, Figure 4;
  * bottom-up coalescing of consecutive KV blocks: FCP paper Sec. 4.2;
  * the pull graph of block transfers among workers: FCP paper Sec. 4.2, Figure 8;
  * budget filling that cuts the sample crossing the budget: "Another View on Context
    Parallel for LLMs", section "Computational Simulation".
"""
from .bf16 import round_to_bf16_bits, bf16_bits_to_f64, bf16_bits_to_f32
from .layout import Seg, Workload, pack_stream, shard_ffd, lpt_assign, block_cost
from .lengths import lognormal_lengths
from .configs import (config1, config2, config3, config4, config5, CONFIG_NAMES, custom,
                      visible_pairs, fwd_flops, bwd_flops, kv_needs, pull_graph,
                      zigzag_graph, hetero_graph)
from .tensors import make_host_inputs, make_device_inputs, rows_of

__all__ = [
    "round_to_bf16_bits", "bf16_bits_to_f64", "bf16_bits_to_f32", "Seg", "Workload",
    "pack_stream", "shard_ffd", "lpt_assign", "block_cost", "lognormal_lengths",
    "config1", "config2", "config3", "config4", "config5", "CONFIG_NAMES", "custom",
    "visible_pairs", "fwd_flops", "bwd_flops", "make_host_inputs",
    "make_device_inputs", "rows_of", "kv_needs", "pull_graph", "zigzag_graph",
    "hetero_graph",
]
