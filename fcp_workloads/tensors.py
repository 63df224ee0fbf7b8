"""Seeded bf16 input tensors.

Values are float32 N(0,1) draws rounded to bfloat16 (round to nearest even), laid out
token-major: Q and dO as [q_rows, Hq, D], K and V as [kv_rows, Hkv, D]. Every block of
every tensor draws from its own child stream keyed by (seed, tensor, block id), so any
block can be regenerated on its own.

Two generators exist. ``make_host_inputs`` uses numpy's PCG64 and returns uint16 bit
patterns; the small and medium workloads use it. ``make_device_inputs`` uses torch's
device Philox generator with the same per-block keying and returns device bf16 tensors;
the multi-gigabyte heterogeneous batch uses it, and the oracle then receives host copies
of just the rows it checks (``rows_of``).
"""
import numpy as np

from .bf16 import round_to_bf16_bits

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4}


def _side(wl, name):
    if name in ("q", "do"):
        return wl.q_blocks, wl.q_block_ids, wl.num_q_heads, wl.q_rows
    return wl.kv_blocks, wl.kv_block_ids, wl.num_kv_heads, wl.kv_rows


def _block_rows(blk):
    return blk[0].row0, sum(s.length for s in blk)


def make_host_inputs(wl, seed=0, which=("q", "k", "v", "do")) -> dict:
    """Returns {name: uint16 array of bf16 bits}."""
    out = {}
    d = wl.head_dim
    for name in which:
        blocks, ids, h, rows = _side(wl, name)
        arr = np.empty((rows, h, d), dtype=np.uint16)
        tid = TENSOR_IDS[name]
        for blk, bid in zip(blocks, ids):
            r0, n = _block_rows(blk)
            rng = np.random.default_rng(np.random.SeedSequence([seed, tid, bid]))
            arr[r0:r0 + n] = round_to_bf16_bits(
                rng.standard_normal((n, h, d), dtype=np.float32))
        out[name] = arr
    return out


def host_to_device(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bits (host) -> torch.bfloat16 tensor on ``device``."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def device_seed(seed, tid, bid) -> int:
    return (int(seed) << 40) | (int(tid) << 32) | int(bid)


def make_device_inputs(wl, seed=0, which=("q", "k", "v", "do"), device="cuda") -> dict:
    """Returns {name: torch.bfloat16 tensor on ``device``}, drawn block by block."""
    import torch
    out = {}
    d = wl.head_dim
    for name in which:
        blocks, ids, h, rows = _side(wl, name)
        t = torch.empty((rows, h, d), dtype=torch.bfloat16, device=device)
        tid = TENSOR_IDS[name]
        g = torch.Generator(device=device)
        for blk, bid in zip(blocks, ids):
            r0, n = _block_rows(blk)
            g.manual_seed(device_seed(seed, tid, bid))
            t[r0:r0 + n] = torch.randn((n, h, d), generator=g, device=device,
                                       dtype=torch.float32).to(torch.bfloat16)
        out[name] = t
    return out


def rows_of(x, rows) -> np.ndarray:
    """Host uint16 bf16 bits of the given rows of a torch bf16 tensor or uint16 array."""
    rows = np.asarray(rows, dtype=np.int64)
    if isinstance(x, np.ndarray):
        return x[rows]
    import torch
    idx = torch.as_tensor(rows, device=x.device)
    return x.index_select(0, idx).cpu().view(torch.int16).numpy().view(np.uint16)
