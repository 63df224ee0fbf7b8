"""Block-level variable-length attention for MI355X (gfx950).

One worker's share of FCP-style context parallelism: block-pair descriptors, per-pair
partial attention, LSE merge, a fused forward and the backward, all computed by the
hand-written HIP kernels of libfcp.so. ``descriptors`` builds the pair table on the
host; ``binding`` exposes the C entry points under their own names.
"""
from .descriptors import build_pairs, part_rows, PAIR_DTYPE, FLAG_CAUSAL
from .binding import (fcp_abi_version, fcp_status_string, fcp_last_error, fcp_validate,
                      fcp_workspace_bytes, fcp_block_attn_fwd, fcp_merge_partials,
                      fcp_block_attn_fwd_fused, fcp_block_attn_bwd, fcp_comm_plan,
                      fcp_pipeline_fwd, fcp_pipeline_workspace_bytes, make_dims, FcpError,
                      FCP_OP_FWD, FCP_OP_MERGE, FCP_OP_BWD, FCP_OP_FWD_FUSED)
