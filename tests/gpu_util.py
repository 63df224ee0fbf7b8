"""Helpers for the GPU parity tests: seeded inputs on both sides and the parity gates.

Gates (bf16 inputs, fp32 accumulation): on O, max-abs <= 2e-2 and relative L2 <= 5e-3
over all checked elements; on finite LSE, max-abs <= 1e-3; -inf LSE rows must match
exactly and carry O == 0.
"""
import numpy as np

import fcp_workloads as W
from fcp_workloads.tensors import host_to_device

O_MAX_ABS = 2e-2
O_REL_L2 = 5e-3
LSE_MAX_ABS = 1e-3


def inputs(wl, seed=0, which=("q", "k", "v", "do")):
    """(device bf16 tensors, host float64 arrays) drawn from the same seeded bits."""
    if wl.rng == "device":
        dev = W.make_device_inputs(wl, seed=seed, which=which)
        return dev, None
    bits = W.make_host_inputs(wl, seed=seed, which=which)
    dev = {n: host_to_device(b) for n, b in bits.items()}
    host = {n: W.bf16_bits_to_f64(b) for n, b in bits.items()}
    return dev, host


def bf16_to_f64(t):
    """torch bf16 tensor -> float64 numpy (exact)."""
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32) \
        .__lshift__(16).view(np.float32).astype(np.float64)


def kv_row_pos(wl):
    pos = np.full(wl.kv_rows, -1, dtype=np.int64)
    for s in wl.kv_segments():
        pos[s.row0:s.row0 + s.length] = np.arange(s.pos0, s.pos0 + s.length)
    return pos


def check_attn(o, lse, o_ref, lse_ref, what=""):
    """Parity gates for an (O, LSE) pair of arrays with matching shapes."""
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    ninf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), ninf_ref), "%s: -inf LSE rows differ" % what
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "%s: NaN in output" % what
    fin = ~ninf_ref
    if fin.any():
        lerr = np.abs(lse[fin] - lse_ref[fin]).max()
        assert lerr <= LSE_MAX_ABS, "%s: LSE max-abs %.3g" % (what, lerr)
    if ninf_ref.any():
        assert np.all(o[ninf_ref] == 0.0), "%s: empty rows must have O == 0" % what
    err = np.abs(o - o_ref)
    assert err.max() <= O_MAX_ABS, "%s: O max-abs %.3g" % (what, err.max())
    rel = np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-30)
    assert rel <= O_REL_L2, "%s: O rel-L2 %.3g" % (what, rel)
    return float(err.max()), float(rel)


def sample_rows(wl, n, seed=0):
    """Owned Q rows to check at full size: segment starts and ends plus random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for s in wl.q_segments():
        rows.update({s.row0, s.row0 + s.length - 1, s.row0 + s.length // 2})
    rows.update(rng.integers(0, wl.q_rows, size=n).tolist())
    return np.array(sorted(rows), dtype=np.int64)


class DeviceRows:
    """Float64 view of a device bf16 tensor [rows, heads, D] for the oracle at full size:
    ``x[row_array, head]`` copies just those rows of one head to the host (exactly: bf16
    -> float64). The last fetch is cached, since the oracle reads the same key rows for
    every query head of a KV group."""

    def __init__(self, t):
        self.t = t
        self._key = None
        self._val = None

    def __getitem__(self, key):
        import torch
        rows, h = key
        rows = np.asarray(rows, dtype=np.int64)
        ck = (id(rows) if rows.base is None else id(rows.base), rows.shape,
              int(rows[0]) if rows.size else -1, int(rows[-1]) if rows.size else -1, int(h))
        if ck == self._key:
            return self._val
        idx = torch.as_tensor(rows, device=self.t.device)
        val = bf16_to_f64(self.t[:, h].index_select(0, idx))
        if rows.size > 4096:
            self._key, self._val = ck, val
        return val
