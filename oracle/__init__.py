"""Float64 CPU oracle for block-level varlen attention (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package. The product path (the HIP library and its binding) never
does, and this package imports nothing from it. Parity status per function:
  forward, partial, merge, backward, dq_rows, dkv_rows, dkv_keys: pinned (brute force, closed forms,
  invariants, finite differences; see tests/test_oracle.py).
  comm.max_degree, comm.is_congestion_free, comm.min_stages_brute_force,
  comm.alternating_path_plan: pinned (exhaustive search, closed forms, planted invalid
  plans; see tests/test_comm_plan.py).
"""
from .attention import SeqIndex, forward, partial, merge, backward, dq_rows, dkv_rows, \
    dkv_keys
from . import comm

__all__ = ["SeqIndex", "forward", "partial", "merge", "backward", "dq_rows", "dkv_rows",
           "dkv_keys",
           "comm"]
