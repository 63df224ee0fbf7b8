#!/usr/bin/env python
"""Throughput of one worker's block-level varlen attention on one MI355X.

A step is one pass of the whole path over one batch: the host builds the block-pair
descriptors, the library plans and uploads its work lists, then the per-pair forward
partials, the LSE merge, and the backward (Delta, dQ, dK/dV) run on the GPU. The metric
is attention TFLOP/s (forward 4*D, backward 10*D per visible query-key pair and query
head) and its fraction of the MI355X dense bf16 MFMA peak, against block size.

Headline (``value``): forward + backward on one 32K-token causal sequence cut into
4096-token blocks (every needed pair as a partial, then merged), 64 query / 8 KV heads,
head dim 128. By default the run adds the block-size sweep (512 .. 16384, causal and
non-causal: forward, fused forward, forward + backward, per-kernel rates and shader
clock per row), the 1K-block worker share, the Zig-Zag worker of a 512K sequence and
the heaviest worker of the heterogeneous lognormal batch (forward + backward), and the
float64 oracle timed on the host cores. Inputs are seeded synthetic bf16 N(0,1) data,
resident in HBM before timing starts.

Prints one JSON line. ``--gpus`` above 1 is refused: the library runs on one GPU.
"""
import argparse
import json
import os
import sys
import time

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 bf16 flop/clk x 2.4 GHz, dense
PEAK_HBM_GBS = 8000.0
METRIC = "block-attention TFLOP/s and % BF16 MFMA peak vs block size (fwd, fwd+bwd)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="config3", choices=["config2", "config3", "config4",
                                                              "config5"])
    ap.add_argument("--block", type=int, default=4096, help="block size for config3")
    ap.add_argument("--non-causal", action="store_true", help="non-causal mask for config3")
    ap.add_argument("--no-legs", dest="legs", action="store_false", default=True,
                    help="skip the 1K share, Zig-Zag and heterogeneous legs")
    ap.add_argument("--coalesce", type=int, default=None,
                    help="KV blocks coalesced per range for the Zig-Zag (default 4) and "
                         "heterogeneous (default 1) workloads")
    ap.add_argument("--sweep", dest="sweep", action="store_true", default=True)
    ap.add_argument("--no-sweep", dest="sweep", action="store_false")
    ap.add_argument("--no-cpu-baseline", dest="cpu", action="store_false", default=True)
    ap.add_argument("--fused", action="store_true",
                    help="use the fused forward (merge folded in) inside the step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain device copy of known size (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters of a profiler run)")
    ap.add_argument("--pipeline", action="store_true",
                    help="instead of the attention step, time the block-level pipelined "
                         "forward of the Zig-Zag worker (pulls overlapped with compute) "
                         "against the same stages with every block already resident")
    ap.add_argument("--comm-plan", action="store_true",
                    help="instead of the attention step, time the host-only congestion-free "
                         "planner on Zig-Zag pull graphs of 64..512 workers and on the "
                         "heterogeneous 64-worker batch (one JSON line per graph; no GPU)")
    return ap.parse_args()


PIPE_HEADLINE = "shader_depth3"


def pipeline_bench(args):
    """eta of FCP paper Sec. 3.3 on one GPU: time of the pipelined forward of Zig-Zag
    worker 0 of 64 (126 blocks pulled in the congestion-free order, 4 per stage, copies
    on a second stream) over the time of the same stages with every block resident."""
    import numpy as np
    import torch
    import fcp_workloads as W
    from block_wise_varlen_amd import binding as B
    from block_wise_varlen_amd.descriptors import build_pipeline
    wl = W.config4(0)
    src, dst, blk = W.zigzag_graph(64)
    stage, _ = B.fcp_comm_plan(64, src, dst)
    m = dst == 0
    recv = {int(b): int(s) for b, s in zip(blk[m], stage[m])}
    dev = W.make_device_inputs(wl, seed=args.seed, which=("q", "k", "v"))
    hkv, d, hq = wl.num_kv_heads, wl.head_dim, wl.num_q_heads

    def buffers(P, fill):
        k = torch.zeros((P["kv_rows"], hkv, d), dtype=torch.bfloat16, device="cuda")
        v = torch.zeros_like(k)
        for c in fill:
            s0, t0, n = int(c["src_row"]), int(c["dst_row"]), int(c["n_rows"])
            k[t0:t0 + n] = dev["k"][s0:s0 + n]
            v[t0:t0 + n] = dev["v"][s0:s0 + n]
        return k, v

    pipes = {d: build_pipeline(wl, wl.q_block_ids, recv, coalesce=4, depth=d) for d in (2, 3)}
    res = build_pipeline(wl, wl.q_block_ids, recv, coalesce=4, depth=None)
    # Resident: every stage's blocks already in place, no copies in the tables.
    res_fill = np.concatenate([res["local_copies"], res["copies"]])
    res_stages = res["stages"].copy()
    res_stages["n_copies"] = 0
    bufs = {d: buffers(P, P["local_copies"]) for d, P in pipes.items()}
    kr, vr = buffers(res, res_fill)
    pipe = pipes[2]
    o_part = torch.empty((pipe["part_rows"], hq, d), dtype=torch.float32, device="cuda")
    lse_part = torch.empty((pipe["part_rows"], hq), dtype=torch.float32, device="cuda")
    o = torch.empty_like(dev["q"])
    lse = torch.empty((wl.q_rows, hq), dtype=torch.float32, device="cuda")
    cs = torch.cuda.Stream()
    nothing = np.zeros(0, dtype=pipe["copies"].dtype)

    def leg(depth, flags, stream):
        P, (kp, vp) = pipes[depth], bufs[depth]
        return lambda: B.fcp_pipeline_fwd(dev["q"], kp, vp, dev["k"], dev["v"], P["stages"],
                                          P["copies"], P["pairs"], o_part, lse_part, o, lse,
                                          depth=depth, flags=flags, copy_stream=stream)

    legs = {
        "resident": lambda: B.fcp_pipeline_fwd(dev["q"], kr, vr, dev["k"], dev["v"], res_stages,
                                               nothing, res["pairs"], o_part, lse_part, o, lse,
                                               depth=res["depth"]),
        "dma_depth2": leg(2, 0, cs),
        "dma_depth3": leg(3, 0, cs),
        "shader_depth2": leg(2, B.FCP_PIPE_COPY_SHADER, cs),
        "shader_depth3": leg(3, B.FCP_PIPE_COPY_SHADER, cs),
        "serial_dma": leg(2, 0, None),
    }
    ms, copy_rate = {}, {}
    copy_bytes = 2 * int(pipe["copies"]["n_rows"].sum()) * hkv * d * 2
    for name, fn in legs.items():
        log("timing pipeline leg", name)
        ms[name], kt = timed(fn, args.steps, args.warmup, True)
        if "pipe_copy" in kt:
            t, n = kt["pipe_copy"][:2]
            # bytes over the summed duration of the stages' copy batches
            copy_rate[name] = round(copy_bytes * args.steps / (t * 1e-3) / 1e9, 1)
    flops = W.fwd_flops(wl)
    result = {
        "metric": "pipeline_eta", "value": round(ms[PIPE_HEADLINE] / ms["resident"], 4),
        "unit": "ratio", "higher_is_better": False, "steps": args.steps, "warmup": args.warmup,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": wl.name + "-pipelined", "leg": PIPE_HEADLINE, "worker": 0,
                   "n_workers": 64,
                   "stages": len(pipe["stages"]), "pulled_blocks": len(recv),
                   "copy_bytes_per_step": copy_bytes},
        "ms_per_step": {k: round(v, 3) for k, v in ms.items()},
        "eta": {k: round(v / ms["resident"], 4) for k, v in ms.items()},
        "fwd_tflops": {k: round(flops / v / 1e9, 1) for k, v in ms.items()},
        "copy_GBps": copy_rate,
    }
    print(json.dumps(result), flush=True)


def comm_plan_bench(repeats=5):
    """Wall time of fcp_comm_plan (median of ``repeats``) on FCP pull graphs."""
    import fcp_workloads as W
    from block_wise_varlen_amd import binding as B
    B.load()
    graphs = [("zigzag-N%d-b4096" % n, n, W.zigzag_graph(n, seqlen=2 * n * 4096))
              for n in (64, 128, 256, 512)]
    graphs.append(("hetero-lognormal8K-128Kx64-b4096-lpt", 64, W.hetero_graph()))
    for name, n, (src, dst, _) in graphs:
        times = []
        for _ in range(repeats):
            t0 = time.perf_counter()
            _, k = B.fcp_comm_plan(n, src, dst)
            times.append((time.perf_counter() - t0) * 1e3)
        print(json.dumps({"metric": "comm_plan_ms", "value": round(sorted(times)[len(times) // 2], 3),
                          "unit": "ms", "higher_is_better": False,
                          "config": {"graph": name, "workers": n, "transfers": int(len(src)),
                                     "stages": k}}), flush=True)


def covers_all(pairs, q_rows, kv_rows):
    """True when the union of the pairs' Q ranges is [0, q_rows) and that of their KV
    ranges is [0, kv_rows)."""
    import numpy as np

    def union_is(start, length, total):
        if total == 0:
            return True
        mark = np.zeros(total + 1, dtype=np.int64)
        np.add.at(mark, start, 1)
        np.add.at(mark, start + length, -1)
        return bool((np.cumsum(mark)[:total] > 0).all())

    return (union_is(np.asarray(pairs["q_start"], np.int64), np.asarray(pairs["q_len"], np.int64),
                     q_rows) and
            union_is(np.asarray(pairs["kv_start"], np.int64),
                     np.asarray(pairs["kv_len"], np.int64), kv_rows))


class Path:
    """Preallocated buffers and the step function for one workload."""

    def __init__(self, wl, dev, fused=False, part16=False):
        import torch
        from block_wise_varlen_amd import binding as B
        from block_wise_varlen_amd.descriptors import build_pairs, part_rows
        self.B, self.build_pairs, self.wl, self.dev, self.fused = B, build_pairs, wl, dev, fused
        pairs = build_pairs(wl)
        self.pairs = pairs
        self.n_pairs = len(pairs)
        self.prow = part_rows(pairs)
        q, k = dev["q"], dev["k"]
        hq, d = wl.num_q_heads, wl.head_dim
        f32 = torch.float32
        self.o_part = None if fused else torch.empty(
            (self.prow, hq, d), dtype=torch.bfloat16 if part16 else f32, device=q.device)
        self.lse_part = None if fused else torch.empty((self.prow, hq), dtype=f32, device=q.device)
        self.o = torch.zeros_like(q)
        self.lse = torch.zeros((q.shape[0], hq), dtype=f32, device=q.device)
        self.dq = torch.zeros(q.shape, dtype=f32, device=q.device)
        self.dk = torch.zeros(k.shape, dtype=f32, device=q.device)
        self.dv = torch.zeros(k.shape, dtype=f32, device=q.device)
        dims = B.make_dims(hq, wl.num_kv_heads, d, q.shape[0], k.shape[0], self.prow)
        need = max(B.fcp_workspace_bytes(dims, pairs, op) for op in
                   (B.FCP_OP_FWD, B.FCP_OP_MERGE, B.FCP_OP_BWD, B.FCP_OP_FWD_FUSED))
        # One workspace serves every call: the calls are ordered on one stream.
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        # When the pairs cover every Q row and every KV row, the backward writes the
        # gradients (FCP_BWD_OVERWRITE: one writer per row) instead of adding them into
        # zeroed buffers; otherwise the step zeroes them and accumulates.
        self.overwrite = covers_all(pairs, q.shape[0], k.shape[0])

    def forward(self, pairs):
        B, x = self.B, self.dev
        if self.fused:
            B.fcp_block_attn_fwd_fused(x["q"], x["k"], x["v"], pairs, o=self.o, lse=self.lse,
                                       ws=self.ws)
        else:
            B.fcp_block_attn_fwd(x["q"], x["k"], x["v"], pairs, o_part=self.o_part,
                                 lse_part=self.lse_part, part_rows=self.prow, ws=self.ws)
            B.fcp_merge_partials(pairs, self.o_part, self.lse_part, self.wl.q_rows,
                                 self.wl.num_kv_heads, o=self.o, lse=self.lse, ws=self.ws)

    def step(self, backward=True):
        pairs = self.build_pairs(self.wl)
        self.forward(pairs)
        if backward:
            if not self.overwrite:
                self.dq.zero_()
                self.dk.zero_()
                self.dv.zero_()
            x = self.dev
            self.B.fcp_block_attn_bwd(x["q"], x["k"], x["v"], self.o, self.lse, x["do"], pairs,
                                      dq=self.dq, dk=self.dk, dv=self.dv, ws=self.ws,
                                      overwrite=self.overwrite)


def timed(fn, steps, warmup, kernel_times=False, per_step=None):
    """Runs fn warmup + steps times; returns (ms per step, per-kernel {name: (ms, n, MHz)}):
    summed HIP-event time of each kernel's launches on the stream it ran on, their count,
    and the average shader clock sampled inside the kernel (0 where not sampled). With a
    list as per_step, also appends each timed step's own duration (events between the
    steps, inside the same bracketed region)."""
    import torch
    from block_wise_varlen_amd import binding as B
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    B.fcp_timing_read_clock()
    if kernel_times:
        B.fcp_timing_enable(True)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        fn()
        if per_step is not None or i == steps - 1:
            ev[i + 1].record()
    torch.cuda.synchronize()
    B.fcp_timing_enable(False)
    kt = B.fcp_timing_read_clock()
    if per_step is not None:
        per_step.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return ev[0].elapsed_time(ev[steps]) / steps, kt


def kernel_work(name, wl, pairs):
    """Algorithmic work of one launch of a kernel: (amount, unit, bound)."""
    import fcp_workloads as W
    n_vis = W.visible_pairs(wl)
    per = wl.head_dim * wl.num_q_heads * n_vis
    d, hq = wl.head_dim, wl.num_q_heads
    if name in ("fwd_partial", "fwd_fused"):
        return 4 * per, "flop", "mfma"
    if name == "bwd_dkdv":
        return 8 * per, "flop", "mfma"     # S recompute, dP, dV, dK
    if name == "bwd_dq":
        return 2 * per, "flop", "mfma"     # dQ (its S and dP recompute are not counted)
    q_rows = sum(s.length for s in wl.q_segments())
    if name == "merge":
        parts = int(pairs["q_len"].sum())
        return parts * hq * (4 * d + 4) + q_rows * hq * (2 * d + 4), "byte", "hbm"
    if name == "bwd_dkdv_reduce":
        return None, "byte", "hbm"   # depends on the split; never the dominant kernel
    raise KeyError(name)


# Kernel sources whose hash a recorded HBM-traffic figure is tied to.
KERNEL_SOURCES = ["fcp_common.h", "fcp_types.h", "fcp_kernels.h", "fcp_cursor.h",
                  "fcp_fwd.hip", "fcp_bwd.hip", "fcp_bwd_dq.hip", "fcp_merge.hip"]


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_wise_varlen_amd",
                        "csrc")
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from a committed counter summary
    under profiles/ (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or
    None when there is none or the kernel sources changed since it was taken."""
    import glob
    here = os.path.dirname(os.path.abspath(__file__))
    sha = None
    for path in sorted(glob.glob(os.path.join(here, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                if not line.startswith("traffic-json: "):
                    continue
                rec = json.loads(line[len("traffic-json: "):])
                if rec.get("kernel") != kernel or rec.get("workload") != workload:
                    continue
                sha = sha or sources_sha256()
                if rec.get("sources_sha256") == sha:
                    return rec["bytes_per_launch"]
    return None


def run_env():
    """What the numbers were measured with: device architecture and CU count, HIP and
    torch versions, the kernel sources' hash (the key of recorded traffic figures) and
    the git revision when the tree has one."""
    import subprocess
    import torch
    prop = torch.cuda.get_device_properties(0)
    env = {"arch": getattr(prop, "gcnArchName", ""), "cus": prop.multi_processor_count,
           "hip": torch.version.hip, "torch": torch.__version__,
           "kernel_sources_sha256": sources_sha256()}
    try:
        env["git"] = subprocess.run(["git", "rev-parse", "--short=12", "HEAD"],
                                    cwd=os.path.dirname(os.path.abspath(__file__)),
                                    capture_output=True, text=True, timeout=10).stdout.strip() or None
    except Exception:
        env["git"] = None
    return env


def label(wl):
    """Workload name with the knobs that change its pair table (block size and mask of
    the 32K sweep, coalescing degree of the Zig-Zag and heterogeneous workers)."""
    if wl.name.startswith("sweep-"):
        return "%s/b%d-%s" % (wl.name, wl.block_size, "causal" if wl.causal else "noncausal")
    if wl.coalesce and wl.coalesce > 1 or wl.name.startswith(("zigzag", "hetero")):
        return "%s/c%d" % (wl.name, wl.coalesce or 1)
    return wl.name


def roofline(kt, steps, wl, pairs):
    name = max(kt, key=lambda n: kt[n][0])
    total_ms, launches = kt[name][0], kt[name][1]
    avg_s = total_ms / launches / 1e3
    work, unit, bound = kernel_work(name, wl, pairs)
    if unit == "flop":
        achieved, peak, u = work / avg_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, u = work / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
    return {"bound": bound, "kernel": name, "achieved": round(achieved, 2), "peak": peak,
            "unit": u, "frac": round(achieved / peak, 4),
            "traffic": recorded_traffic(name, label(wl)),
            "avg_launch_ms": round(total_ms / launches, 4), "launches": launches}


def kernel_rates(kt, wl, pairs):
    """Achieved rate of every timed kernel against its own roofline (TFLOP/s of counted
    work for the MFMA kernels, GB/s of algorithmic bytes for the HBM-bound ones), its
    average launch time, and the shader clock sampled inside it."""
    out = {}
    for name, rec in kt.items():
        total_ms, launches = rec[0], rec[1]
        mhz = rec[2] if len(rec) > 2 else 0.0
        try:
            work, unit, bound = kernel_work(name, wl, pairs)
        except (KeyError, ValueError):
            continue
        avg_s = total_ms / launches / 1e3
        row = {"ms": round(total_ms / launches, 4), "bound": bound}
        if work is not None:
            if unit == "flop":
                achieved, peak, u = work / avg_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
            else:
                achieved, peak, u = work / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
            row.update(achieved=round(achieved, 2), unit=u, frac=round(achieved / peak, 4))
        if mhz:
            row["sclk_mhz"] = round(mhz)
        out[name] = row
    return out


def leg_sclk(kt):
    """Shader clock over a step: the kernels' sampled clocks weighted by their time."""
    num = sum(r[0] * r[2] for r in kt.values() if len(r) > 2 and r[2])
    den = sum(r[0] for r in kt.values() if len(r) > 2 and r[2])
    return round(num / den) if den else None


def calibration_copy(n_bytes=512 << 20, reps=3):
    """A plain device-to-device copy of n_bytes (read n_bytes, write n_bytes per launch),
    whose FETCH_SIZE / WRITE_SIZE counters scale the other kernels' counts to bytes."""
    import torch
    src = torch.empty(n_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    log("calibration copy: %d bytes read and %d bytes written per launch, %d launches, "
        "%.3f ms each = %.0f GB/s read+write" % (n_bytes, n_bytes, reps + 1, ms,
                                                 2 * n_bytes / ms / 1e6))


def measure(wl, dev, steps, warmup, forward_only=False, fused=False, per_step=None,
            part16=False):
    """One leg: (ms per step, kernel times) of the step on ``wl``, plus its summary.
    ``part16``: the per-pair partials in bf16 (FCP_PART_BF16) instead of fp32."""
    import fcp_workloads as W
    path = Path(wl, dev, fused=fused, part16=part16)
    ms, kt = timed(lambda: path.step(backward=not forward_only), steps, warmup, True,
                   per_step=per_step)
    fl = W.fwd_flops(wl) + (0 if forward_only else W.bwd_flops(wl))
    tf = fl / ms / 1e9
    summary = {"ms": round(ms, 3), "tflops": round(tf, 1),
               "mfu": round(tf / PEAK_BF16_TFLOPS, 4), "sclk_mhz": leg_sclk(kt),
               "kernel_rates": kernel_rates(kt, wl, path.pairs)}
    return ms, kt, path.pairs, summary


SWEEP_BLOCKS = (512, 1024, 2048, 4096, 8192, 16384)


def sweep(base, steps=5, warmup=2):
    """The 32K block-size sweep: per block size and mask, the forward (fp32 partials +
    merge, and bf16 partials + merge), the fused forward and forward + backward, each with
    per-kernel rates and clocks."""
    import fcp_workloads as W
    out = []
    for causal in (True, False):
        for b in SWEEP_BLOCKS:
            wl = W.config3(b, causal)
            _, _, pairs, f = measure(wl, base, steps, warmup, forward_only=True)
            _, _, _, h = measure(wl, base, steps, warmup, forward_only=True, part16=True)
            _, _, _, u = measure(wl, base, steps, warmup, forward_only=True, fused=True)
            _, _, _, fb = measure(wl, base, steps, warmup)
            row = {"block": b, "mask": "causal" if causal else "non-causal",
                   "pairs": len(pairs),
                   "fwd_ms": f["ms"], "fwd_tflops": f["tflops"], "fwd_mfu": f["mfu"],
                   "fwd_bf16part_ms": h["ms"], "fwd_bf16part_tflops": h["tflops"],
                   "fwd_bf16part_mfu": h["mfu"],
                   "fused_fwd_ms": u["ms"], "fused_fwd_tflops": u["tflops"],
                   "fused_fwd_mfu": u["mfu"],
                   "fwdbwd_ms": fb["ms"], "fwdbwd_tflops": fb["tflops"], "fwdbwd_mfu": fb["mfu"],
                   "sclk_mhz": fb["sclk_mhz"], "kernel_rates": fb["kernel_rates"],
                   "fwd_kernel_rates": f["kernel_rates"]}
            log("sweep", json.dumps(row))
            out.append(row)
    return out


def legs(seed, steps=3, warmup=1):
    """Forward + backward on the other workers' shares: the 1K-block worker share, the
    Zig-Zag worker (coalescing 4) and the heaviest heterogeneous worker (coalescing 1
    and 4); also the fused-forward step on the share."""
    import torch
    import fcp_workloads as W
    from fcp_workloads.tensors import host_to_device
    out = {}
    wl = W.config2(seed)
    bits = W.make_host_inputs(wl, seed=seed)
    dev = {n: host_to_device(b) for n, b in bits.items()}
    for fused in (False, True):
        _, _, pairs, r = measure(wl, dev, 10, 3, fused=fused)
        r.update(workload=label(wl), pairs=len(pairs), seqlens=wl.seqlens,
                 forward="fused" if fused else "partials+merge")
        out["worker_1K_share" + ("_fused" if fused else "")] = r
        log("leg", json.dumps(r))
    del dev
    for name, mk in (("zigzag_512K_c4", lambda: W.config4(0, coalesce=4)),
                     ("hetero_c1", lambda: W.config5(seed, coalesce=1)),
                     ("hetero_c4", lambda: W.config5(seed, coalesce=4))):
        wl = mk()
        torch.cuda.empty_cache()
        dev = W.make_device_inputs(wl, seed=seed)
        _, _, pairs, r = measure(wl, dev, steps, warmup)
        _, _, _, f = measure(wl, dev, steps, warmup, forward_only=True)
        r.update(workload=label(wl), pairs=len(pairs), q_rows=wl.q_rows, kv_rows=wl.kv_rows,
                 fwd_ms=f["ms"], fwd_tflops=f["tflops"], fwd_mfu=f["mfu"])
        out[name] = r
        log("leg", json.dumps(r))
        del dev
    return out


def _threads():
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        return max(i["num_threads"] for i in info) if info else 1
    except Exception:
        return None


def cpu_baseline(dev, seed):
    """The float64 oracle (forward + backward, as it stands) on the host cores.

    Headline sample: query head 0 (with KV head 0) of the headline workload over its
    first 23170 rows (their causal keys are the first 23170 positions, so this is exactly
    that part of the headline's work: half of its visible pairs, 1/128 of the whole), on
    the same bf16 values the GPU step read. Also: the tiny three-sequence case in full and
    the 1K-block worker share's 3496-token sequence (all heads). The full headline and the
    Zig-Zag and heterogeneous workers are extrapolated from the measured rate (labelled as
    such)."""
    import numpy as np
    import fcp_workloads as W
    import oracle

    def f64(t):
        import torch
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32) \
            .__lshift__(16).view(np.float32).astype(np.float64)

    def run(wl, x, seqs=None):
        idx = oracle.SeqIndex(wl)
        t0 = time.perf_counter()
        oracle.forward(x["q"], x["k"], x["v"], idx)
        oracle.backward(x["q"], x["k"], x["v"], x["do"], idx, seqs=seqs)
        return time.perf_counter() - t0

    def flops(wl, n_vis):
        return 14 * wl.head_dim * wl.num_q_heads * n_vis

    # headline sample: one query head and its KV head over the sequence's first rows, as
    # a 1-head workload of that prefix (query head 0 reads KV head 0 in the 64/8 layout too)
    n = 23170
    head = W.custom([n], 4096, 1, 1, 128, True)
    x = {"q": f64(dev["q"][:n, :1]), "k": f64(dev["k"][:n, :1]), "v": f64(dev["v"][:n, :1]),
         "do": f64(dev["do"][:n, :1])}
    dt = run(head, x)
    fl = flops(head, W.visible_pairs(head))
    rate = fl / dt
    tiny = W.config1()
    bits = W.make_host_inputs(tiny, seed=seed)
    dt1 = run(tiny, {n: W.bf16_bits_to_f64(b) for n, b in bits.items()})
    share = W.config2(seed)
    bits = W.make_host_inputs(share, seed=seed)
    xs = {n: W.bf16_bits_to_f64(b) for n, b in bits.items()}
    cands = [(L, s) for s, L in enumerate(share.seqlens) if L >= 2048] or \
        [(L, s) for s, L in enumerate(share.seqlens)]
    length, s = min(cands)
    idx = oracle.SeqIndex(share)
    t0 = time.perf_counter()
    rows = np.nonzero(idx.q_row_seq == s)[0]
    oracle.forward(xs["q"], xs["k"], xs["v"], idx, rows=rows)
    oracle.backward(xs["q"], xs["k"], xs["v"], xs["do"], idx, seqs=[s])
    dt2 = time.perf_counter() - t0
    fl2 = flops(share, length * (length + 1) // 2)
    extrap = {}
    for name, wl in (("sweep_32K_b4096_causal", W.config3(4096, True)),
                     ("sweep_32K_b4096_noncausal", W.config3(4096, False)),
                     ("zigzag_512K", W.config4(0)), ("hetero_heaviest_worker", W.config5(seed))):
        extrap[name] = round(flops(wl, W.visible_pairs(wl)) / rate, 1)
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": _threads(),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": "float64 oracle forward + backward of query head 0 (KV head 0) over the "
                      "first 23170 rows of the headline workload (32K causal sequence): half of "
                      "that head's visible pairs, 1/128 of the step's work, %.3g FLOP" % fl,
            "cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "blas_threads": _threads(),
            "tiny_config_full": {"seconds": round(dt1, 3),
                                 "tflops": round(flops(tiny, W.visible_pairs(tiny)) / dt1 / 1e12, 6)},
            "worker_1K_share_sample": {"seconds": round(dt2, 2),
                                       "tflops": round(fl2 / dt2 / 1e12, 6),
                                       "sample": "sequence %d (%d tokens), all 64 query heads"
                                                 % (s, length)},
            "extrapolated_full_seconds": extrap}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.comm_plan:
        comm_plan_bench()
        return
    if args.pipeline:
        import torch
        if not torch.cuda.is_available():
            print("no GPU available", file=sys.stderr)
            sys.exit(1)
        pipeline_bench(args)
        return
    import torch
    import fcp_workloads as W
    from fcp_workloads.tensors import host_to_device
    from block_wise_varlen_amd import binding as B
    B.load()
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)

    wl = {"config2": lambda: W.config2(args.seed),
          "config3": lambda: W.config3(args.block, not args.non_causal),
          "config4": lambda: W.config4(0, coalesce=args.coalesce or 4),
          "config5": lambda: W.config5(args.seed, coalesce=args.coalesce or 1)}[args.workload]()
    log("workload", label(wl), "q_rows", wl.q_rows, "kv_rows", wl.kv_rows)
    if args.workload == "config2":
        bits = W.make_host_inputs(wl, seed=args.seed)
        dev = {n: host_to_device(b) for n, b in bits.items()}
        del bits
    else:
        dev = W.make_device_inputs(wl, seed=args.seed)
    if args.calibrate_copy:
        calibration_copy()
    fl_f, fl_b = W.fwd_flops(wl), W.bwd_flops(wl)

    log("timing fwd+merge")
    ms_f, _, _, fwd = measure(wl, dev, args.steps, args.warmup, forward_only=True,
                              fused=args.fused)
    log("timing full step (fwd + merge + bwd)")
    steps_ms = []
    ms, kt, pairs, full = measure(wl, dev, args.steps, args.warmup, fused=args.fused,
                                  per_step=steps_ms)
    steps_ms.sort()
    value = (fl_f + fl_b) / ms / 1e9
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": label(wl), "block_size": wl.block_size, "tokens": wl.q_rows,
                   "seqlens": wl.seqlens if len(wl.seqlens) <= 16 else len(wl.seqlens),
                   "heads_q": wl.num_q_heads, "heads_kv": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "mask": "causal" if wl.causal else "non-causal",
                   "pairs": len(pairs), "coalesce": wl.coalesce, "seed": args.seed,
                   "forward": "fused" if args.fused else "partials+merge",
                   "step": "descriptors + forward + merge + backward (dQ, dK, dV)",
                   "gradients": "written (FCP_BWD_OVERWRITE)" if covers_all(
                       pairs, wl.q_rows, wl.kv_rows) else "zeroed, then added"},
        "mfu": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(fl_f / ms_f / 1e9, 2),
        "fwd_mfu": round(fl_f / ms_f / 1e9 / PEAK_BF16_TFLOPS, 4),
        "fwd_ms": round(ms_f, 4),
        "step_ms": {"median": round(steps_ms[len(steps_ms) // 2], 4),
                    "min": round(steps_ms[0], 4), "max": round(steps_ms[-1], 4)},
        "flops_per_step": fl_f + fl_b,
        "sclk_mhz": full["sclk_mhz"],
        "kernel_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in kt.items()},
        "roofline": roofline(kt, args.steps, wl, pairs),
        "kernel_rates": full["kernel_rates"],
        "fwd_kernel_rates": fwd["kernel_rates"],
        "device": torch.cuda.get_device_name(0),
        "env": run_env(),
    }
    if not args.fused:
        log("timing the full step with bf16 partials")
        ms16, _, _, p16 = measure(wl, dev, args.steps, args.warmup, part16=True)
        result["fwdbwd_bf16part"] = {"ms": p16["ms"], "tflops": p16["tflops"],
                                     "mfu": p16["mfu"], "kernel_rates": p16["kernel_rates"]}
    log(json.dumps(result))
    if args.sweep and args.workload == "config3":
        torch.cuda.empty_cache()
        result["sweep"] = sweep(dev)
    if args.cpu:
        log("timing the oracle on the host")
        if args.workload == "config3" and args.block == 4096 and not args.non_causal:
            result["cpu_baseline"] = cpu_baseline(dev, args.seed)
    if args.legs and args.workload == "config3":
        del dev
        torch.cuda.empty_cache()
        result["legs"] = legs(args.seed)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
