"""Host-side checks of bench.py's reporting contract (no GPU): the one-GPU refusal, the
roofline fields derived from per-kernel launch times, and the tie between a recorded
HBM-traffic figure and the kernel sources it was measured on."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import fcp_workloads as W  # noqa: E402
from block_wise_varlen_amd.descriptors import build_pairs  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_roofline_takes_the_dominant_kernel_and_counts_visible_pairs():
    wl = W.config2(0)
    pairs = build_pairs(wl)
    # (total ms, launches) per kernel over 10 steps; dK/dV has the largest total.
    kt = {"fwd_partial": (20.0, 10), "merge": (4.75, 10), "bwd_dq": (24.5, 10),
          "bwd_dkdv": (34.0, 10)}
    rl = bench.roofline(kt, 10, wl, pairs)
    assert rl["kernel"] == "bwd_dkdv" and rl["bound"] == "mfma" and rl["unit"] == "TFLOP/s"
    # Causal, no attention across sequences: every sequence of length L contributes
    # L (L + 1) / 2 visible (query, key) pairs; dK/dV counts 8 D flop per pair and head.
    n_vis = sum(L * (L + 1) // 2 for L in wl.seqlens)
    flop = 8 * wl.head_dim * wl.num_q_heads * n_vis
    assert rl["avg_launch_ms"] == pytest.approx(3.4)
    assert rl["achieved"] == pytest.approx(flop / 3.4e-3 / 1e12, rel=1e-3)
    assert rl["frac"] == pytest.approx(rl["achieved"] / rl["peak"], rel=1e-3)
    assert rl["peak"] == pytest.approx(2516.6)
    rates = bench.kernel_rates(kt, wl, pairs)
    assert rates["merge"]["unit"] == "GB/s" and rates["merge"]["bound"] == "hbm"
    # forward: 4 D flop per pair and head
    assert rates["fwd_partial"]["achieved"] == pytest.approx(
        4 * wl.head_dim * wl.num_q_heads * n_vis / 2.0e-3 / 1e12, rel=1e-3)


def _recorded(kernel, workload):
    for name in sorted(os.listdir(os.path.join(ROOT, "profiles"))):
        with open(os.path.join(ROOT, "profiles", name)) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    if rec["kernel"] == kernel and rec["workload"] == workload:
                        return rec
    return None


def test_traffic_figure_is_dropped_when_the_kernel_sources_change(monkeypatch):
    wl = W.config3(4096, True)   # the headline workload
    name = bench.label(wl)
    rec = _recorded("bwd_dkdv", name)
    assert rec is not None, "no recorded traffic for the headline workload's dominant kernel"
    monkeypatch.setattr(bench, "sources_sha256", lambda: rec["sources_sha256"])
    assert bench.recorded_traffic("bwd_dkdv", name) == rec["bytes_per_launch"]
    monkeypatch.setattr(bench, "sources_sha256", lambda: "0" * 64)
    assert bench.recorded_traffic("bwd_dkdv", name) is None


def test_labels_name_the_pair_table_knobs():
    assert bench.label(W.config3(512, False)).endswith("/b512-noncausal")
    assert bench.label(W.config3(4096, True)).endswith("/b4096-causal")
    assert bench.label(W.config5(0, coalesce=4)).endswith("/c4")
    assert bench.label(W.config2(0)) == W.config2(0).name


def test_sclk_is_time_weighted_over_sampled_kernels():
    kt = {"a": (10.0, 2, 2000.0), "b": (30.0, 2, 1800.0), "merge": (5.0, 2, 0.0)}
    assert bench.leg_sclk(kt) == round((10 * 2000 + 30 * 1800) / 40)
    assert bench.leg_sclk({"merge": (1.0, 1, 0.0)}) is None


def test_covers_all_decides_the_gradient_mode():
    """The bench step writes the gradients (overwrite mode) only when the pairs' Q ranges
    cover every Q row and their KV ranges every KV row."""
    wl = W.config3(1024, True)
    pairs = build_pairs(wl)
    assert bench.covers_all(pairs, wl.q_rows, wl.kv_rows)
    # Dropping the pairs of the last Q block leaves its rows uncovered.
    last = pairs["q_start"] == pairs["q_start"].max()
    assert not bench.covers_all(pairs[~last], wl.q_rows, wl.kv_rows)
    # A KV row past every KV range is uncovered too.
    assert not bench.covers_all(pairs, wl.q_rows, wl.kv_rows + 1)
    assert bench.covers_all(pairs[:0], 0, 0)
