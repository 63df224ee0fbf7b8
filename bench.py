#!/usr/bin/env python
"""Throughput of one worker's block-level varlen attention on one MI355X.

A step is one pass of the whole path over one batch: the host builds the block-pair
descriptors, the library plans and uploads its work lists, then the per-pair forward
partials, the LSE merge, and the backward (Delta, dQ, dK/dV) run on the GPU. The metric
is attention TFLOP/s (forward 4*D, backward 10*D per visible query-key pair and query
head) and its fraction of the MI355X dense bf16 MFMA peak.

Default workload: one worker's 16 x 1024-token share packed from lognormal lengths
(median 4K, sigma 1.2), 64 query / 8 KV heads, head dim 128, causal. ``--sweep`` (on by
default) adds the 32K single-sequence block-size sweep (512..4096, causal and
non-causal, forward and forward+backward) as extra fields. Inputs are seeded synthetic
bf16 N(0,1) data, resident in HBM before timing starts.

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
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--workload", default="config2", choices=["config2", "config3", "config4",
                                                              "config5"])
    ap.add_argument("--block", type=int, default=4096, help="block size for config3")
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
            t, n = kt["pipe_copy"]
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


class Path:
    """Preallocated buffers and the step function for one workload."""

    def __init__(self, wl, dev, fused=False):
        import torch
        from block_wise_varlen_amd import binding as B
        from block_wise_varlen_amd.descriptors import build_pairs, part_rows
        self.B, self.build_pairs, self.wl, self.dev, self.fused = B, build_pairs, wl, dev, fused
        pairs = build_pairs(wl)
        self.n_pairs = len(pairs)
        self.prow = part_rows(pairs)
        q, k = dev["q"], dev["k"]
        hq, d = wl.num_q_heads, wl.head_dim
        f32 = torch.float32
        self.o_part = None if fused else torch.empty((self.prow, hq, d), dtype=f32, device=q.device)
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
            self.dq.zero_()
            self.dk.zero_()
            self.dv.zero_()
            x = self.dev
            self.B.fcp_block_attn_bwd(x["q"], x["k"], x["v"], self.o, self.lse, x["do"], pairs,
                                      dq=self.dq, dk=self.dk, dv=self.dv, ws=self.ws)


def timed(fn, steps, warmup, kernel_times=False, per_step=None):
    """Runs fn warmup + steps times; returns (ms per step, per-kernel {name: (ms, n)}).
    With a list as per_step, also appends each timed step's own duration (events between
    the steps, inside the same bracketed region)."""
    import torch
    from block_wise_varlen_amd import binding as B
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    B.fcp_timing_read()
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
    kt = B.fcp_timing_read()
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
                  "fcp_fwd.hip", "fcp_bwd.hip", "fcp_merge.hip"]


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


def roofline(kt, steps, wl, pairs):
    name = max(kt, key=lambda n: kt[n][0])
    total_ms, launches = kt[name]
    avg_s = total_ms / launches / 1e3
    work, unit, bound = kernel_work(name, wl, pairs)
    if unit == "flop":
        achieved, peak, u = work / avg_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
    else:
        achieved, peak, u = work / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
    return {"bound": bound, "kernel": name, "achieved": round(achieved, 2), "peak": peak,
            "unit": u, "frac": round(achieved / peak, 4),
            "traffic": recorded_traffic(name, wl.name),
            "avg_launch_ms": round(total_ms / launches, 4), "launches": launches}


def kernel_rates(kt, wl, pairs):
    """Achieved rate of every timed kernel against its own roofline: TFLOP/s of counted
    work for the MFMA kernels, GB/s of algorithmic bytes for the HBM-bound ones."""
    out = {}
    for name, (total_ms, launches) in kt.items():
        try:
            work, unit, bound = kernel_work(name, wl, pairs)
        except (KeyError, ValueError):
            continue
        if work is None:
            continue
        avg_s = total_ms / launches / 1e3
        if unit == "flop":
            achieved, peak, u = work / avg_s / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s"
        else:
            achieved, peak, u = work / avg_s / 1e9, PEAK_HBM_GBS, "GB/s"
        out[name] = {"achieved": round(achieved, 2), "unit": u, "frac": round(achieved / peak, 4),
                     "bound": bound}
    return out


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


def cpu_baseline(wl, seed):
    """The float64 oracle (forward + backward) on one sequence of the same workload."""
    import numpy as np
    import fcp_workloads as W
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max(i["num_threads"] for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        cores = os.cpu_count()
    bits = W.make_host_inputs(wl, seed=seed)
    x = {n: W.bf16_bits_to_f64(b) for n, b in bits.items()}
    idx = oracle.SeqIndex(wl)
    # the shortest sequence with at least 2048 tokens keeps the sample near 10-30 s
    cands = [(L, s) for s, L in enumerate(wl.seqlens) if L >= 2048] or \
        [(L, s) for s, L in enumerate(wl.seqlens)]
    length, s = min(cands)
    t0 = time.perf_counter()
    oracle.backward(x["q"], x["k"], x["v"], x["do"], idx, seqs=[s])
    dt = time.perf_counter() - t0
    n_vis = length * (length + 1) // 2 if wl.causal else length * length
    flops = 14 * wl.head_dim * wl.num_q_heads * n_vis
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": "float64 oracle forward+backward of sequence %d (%d tokens, all %d "
                      "query heads) of the same workload, %.3g FLOP" % (s, length,
                                                                       wl.num_q_heads, flops)}


def sweep(seed, steps=5, warmup=2):
    import fcp_workloads as W
    out = []
    base = W.make_device_inputs(W.config3(4096, True), seed=seed)
    for causal in (True, False):
        for b in (512, 1024, 2048, 4096):
            wl = W.config3(b, causal)
            path = Path(wl, base)
            fl_f, fl_b = W.fwd_flops(wl), W.bwd_flops(wl)
            ms_f, _ = timed(lambda: path.step(backward=False), steps, warmup)
            ms_fb, kt = timed(lambda: path.step(backward=True), steps, warmup, True)
            fused = Path(wl, base, fused=True)
            ms_u, _ = timed(lambda: fused.step(backward=False), steps, warmup)
            row = {"block": b, "mask": "causal" if causal else "non-causal",
                   "pairs": path.n_pairs,
                   "fwd_ms": round(ms_f, 3), "fwd_tflops": round(fl_f / ms_f / 1e9, 1),
                   "fwd_mfu": round(fl_f / ms_f / 1e9 / PEAK_BF16_TFLOPS, 4),
                   "fused_fwd_ms": round(ms_u, 3),
                   "fused_fwd_tflops": round(fl_f / ms_u / 1e9, 1),
                   "fwdbwd_ms": round(ms_fb, 3),
                   "fwdbwd_tflops": round((fl_f + fl_b) / ms_fb / 1e9, 1),
                   "fwdbwd_mfu": round((fl_f + fl_b) / ms_fb / 1e9 / PEAK_BF16_TFLOPS, 4),
                   "kernel_ms": {k: round(v[0] / v[1], 4) for k, v in kt.items()}}
            log("sweep", json.dumps(row))
            out.append(row)
            del path, fused
    return out


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
    from block_wise_varlen_amd.descriptors import build_pairs
    B.load()
    if not torch.cuda.is_available():
        print("no GPU available", file=sys.stderr)
        sys.exit(1)

    wl = {"config2": lambda: W.config2(args.seed),
          "config3": lambda: W.config3(args.block, True),
          "config4": lambda: W.config4(0, coalesce=args.coalesce or 4),
          "config5": lambda: W.config5(args.seed, coalesce=args.coalesce or 1)}[args.workload]()
    log("workload", wl.name, "q_rows", wl.q_rows, "kv_rows", wl.kv_rows)
    if wl.rng == "host":
        bits = W.make_host_inputs(wl, seed=args.seed)
        dev = {n: host_to_device(b) for n, b in bits.items()}
        del bits
    else:
        dev = W.make_device_inputs(wl, seed=args.seed)
    if args.calibrate_copy:
        calibration_copy()
    path = Path(wl, dev, fused=args.fused)
    pairs = build_pairs(wl)
    fl_f, fl_b = W.fwd_flops(wl), W.bwd_flops(wl)

    log("timing fwd+merge")
    ms_f, _ = timed(lambda: path.step(backward=False), args.steps, args.warmup)
    log("timing full step (fwd + merge + bwd)")
    steps_ms = []
    ms, kt = timed(lambda: path.step(backward=True), args.steps, args.warmup, True,
                   per_step=steps_ms)
    steps_ms.sort()
    value = (fl_f + fl_b) / ms / 1e9
    rl = roofline(kt, args.steps, wl, pairs)
    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "block_size": wl.block_size, "tokens": wl.q_rows,
                   "seqlens": wl.seqlens if len(wl.seqlens) <= 16 else len(wl.seqlens),
                   "heads_q": wl.num_q_heads, "heads_kv": wl.num_kv_heads,
                   "head_dim": wl.head_dim, "mask": "causal" if wl.causal else "non-causal",
                   "pairs": len(pairs), "coalesce": wl.coalesce, "seed": args.seed,
                   "forward": "fused" if args.fused else "partials+merge"},
        "mfu": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(fl_f / ms_f / 1e9, 2),
        "fwd_mfu": round(fl_f / ms_f / 1e9 / PEAK_BF16_TFLOPS, 4),
        "fwd_ms": round(ms_f, 4),
        "step_ms": {"median": round(steps_ms[len(steps_ms) // 2], 4),
                    "min": round(steps_ms[0], 4), "max": round(steps_ms[-1], 4)},
        "flops_per_step": fl_f + fl_b,
        "kernel_ms_per_step": {k: round(v[0] / args.steps, 4) for k, v in kt.items()},
        "roofline": rl,
        "kernel_rates": kernel_rates(kt, wl, pairs),
        "device": torch.cuda.get_device_name(0),
    }
    log(json.dumps(result))
    if args.sweep:
        del path
        torch.cuda.empty_cache()
        result["sweep"] = sweep(args.seed)
    if args.cpu:
        log("timing the oracle on the host")
        result["cpu_baseline"] = cpu_baseline(wl, args.seed)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
