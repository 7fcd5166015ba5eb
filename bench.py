"""Benchmark of the deterministic gated FFN on one MI355X.

A step is one pass of the whole hot path over one batch: the training forward
(gate/up tree GEMM with the fused activation, down tree GEMM) and the backward
(dA with dsilu, the two dX lanes and their ordered add, the dW tree GEMMs) at
M=32 tokens, H=4096, I=12288 (the Qwen3-8B FFN shape), BF16, synthetic seeded
inputs already resident in HBM.  Weights rotate over three resident copies so
every step reads them from HBM rather than from the 256 MB last-level cache.

Prints one JSON line.  `value` is the step's algorithmic HBM throughput
(bytes that must cross HBM once per step / step time).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak, published
METRIC = "FFN fwd & fwd+bwd µs + HBM GB/s, H=4096 I=12288 BF16 M=1/8/32"
H, I = 4096, 12288
BF = 2


def step_bytes(M: int) -> int:
    """Algorithmic HBM bytes of a training fwd+bwd step: weights read twice, dW
    written, g/u saved and reloaded, x read twice, y and dX written, dY read."""
    w = 3 * H * I * BF
    return 2 * w + w + 2 * 2 * M * I * BF + 5 * M * H * BF


def fwd_bytes(M: int) -> int:
    return 3 * H * I * BF + 2 * M * H * BF


def kernel_bytes(name: str, M: int) -> int | None:
    """Algorithmic bytes of one launch: every weight and activation operand read
    once and one BF16 copy of each product's result written (K-piece partial
    roots and their joins are not counted).  None for launch-bound joins."""
    W = H * I * BF
    act_mi, act_mh = M * I * BF, M * H * BF
    table = {
        "gate/up + act": 2 * W + act_mh + 3 * act_mi,            # W_gate, W_up, x -> g, u, a
        "gate/up tree GEMM": 2 * W + act_mh + 2 * act_mi,        # W_gate, W_up, x -> g, u
        "down tree GEMM": W + act_mi + act_mh,                    # W_down, a -> y
        "down all-K tree GEMM": W + act_mi + act_mh,              # W_down, a -> y (M <= 16)
        "dA tree GEMM": W + act_mh + act_mi,                      # W_down, dY -> dA
        "dX lanes tree GEMM": 2 * W + 2 * act_mi + 2 * act_mh,    # W_gate, W_up, dG, dU -> G, U
        "dW_gate/dW_up tree GEMM": 2 * W + 2 * act_mi + act_mh,   # dG, dU, x -> dW_gate, dW_up
        "dW_gate/dW_up + dX join": 2 * W + 2 * act_mi + 2 * act_mh,  # the same, and dX from the lanes' roots
        "dW_down tree GEMM": W + act_mh + act_mi,                 # dY, a -> dW_down
    }
    return table.get(name)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ffn_train_step_M32_hbm_traffic.md")


# the source file of each timed kernel; its digest and the shared headers'
# digests must match the ones recorded with the counters
KERNEL_SOURCE = {
    "gate/up + act": "dgf_gu.hip",
    "gate/up tree GEMM": "dgf_xs.hip",
    "down tree GEMM": "dgf_xs.hip",
    "down all-K tree GEMM": "dgf_dn.hip",
    "dA tree GEMM": "dgf_xs.hip",
    "dX lanes tree GEMM": "dgf_xs.hip",
    "dW_gate/dW_up tree GEMM": "dgf_gemm.hip",
    "dW_gate/dW_up + dX join": "dgf_gemm.hip",
    "dW_down tree GEMM": "dgf_gemm.hip",
}
SHARED_HEADERS = ("dgf_device.hpp", "dgf_kernels.hpp", "dgf_join.hpp")


def source_digest(name: str) -> str:
    import hashlib
    with open(os.path.join(ROOT, "deterministic_gated_ffn_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel: str) -> int | None:
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None when it has no figure or the kernel's source (or a shared
    header) changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    figures, digests = {}, {}
    for line in text.splitlines():
        if line.startswith("traffic: "):
            name, _, value = line[len("traffic: "):].rpartition(" = ")
            figures[name] = int(value)
        elif line.startswith("source_sha256: "):
            name, _, value = line[len("source_sha256: "):].rpartition(" = ")
            digests[name] = value.strip()
    src = KERNEL_SOURCE.get(kernel)
    if src is None or kernel not in figures:
        return None
    for f in (src,) + SHARED_HEADERS:
        if digests.get(f) != source_digest(f):
            return None
    return figures[kernel]


def sample_us(run, steps: int, samples: int) -> dict:
    """Times `samples` independent regions of `steps` calls of run(k) (k counts
    calls), each bracketed by device synchronisations and HIP events on the
    current stream; returns the per-call microseconds of every region and their
    median, min and max."""
    import statistics

    import torch
    per, k = [], 0
    for _ in range(samples):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            run(k)
            k += 1
        e1.record()
        torch.cuda.synchronize()
        per.append(1e3 * e0.elapsed_time(e1) / steps)
    return {"median": statistics.median(per), "min": min(per), "max": max(per), "samples": [round(v, 3) for v in per]}


def stats_entry(st: dict, nbytes: int | None = None, flops: int | None = None) -> dict:
    out = {"us": round(st["median"], 2), "us_min": round(st["min"], 2), "us_max": round(st["max"], 2),
           "samples_us": st["samples"]}
    if nbytes:
        gbps = nbytes / (st["median"] * 1e-6) / 1e9
        out.update({"GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4), "algorithmic_bytes": nbytes})
    if flops:
        tf = flops / (st["median"] * 1e-6) / 1e12
        out.update({"TFLOPs": round(tf, 2), "frac_mfma_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "flops": flops})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--samples", type=int, default=5, help="independent timed regions of --steps calls each")
    ap.add_argument("--copies", type=int, default=3, help="resident weight copies rotated per step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--quick", action="store_true", help="skip the forward-only and CPU legs (profiling runs)")
    ap.add_argument("--workload", choices=("train32", "long4096", "rank32"), default="train32",
                    help="long4096: only the M=4096 training step (--warmup, then --samples regions of --steps "
                         "steps); rank32: only one rank's share of the I-sharded M=32 forward and step (shard 0 "
                         "of --shards); both for profiling, printing that leg's JSON instead of the benchmark line")
    ap.add_argument("--dtype", choices=("bf16", "fp16"), default="bf16", help="stored type of the long4096 workload")
    ap.add_argument("--shards", type=int, choices=(2, 4, 8), default=8, help="I shards of the rank32 workload")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}).", file=sys.stderr)
        sys.exit(2)

    import torch
    from deterministic_gated_ffn_amd import binding as dgf
    from deterministic_gated_ffn_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dgf.load()
    print(f"[bench] device {torch.cuda.get_device_name(0)}; building inputs", file=sys.stderr, flush=True)

    if args.workload == "long4096":
        dt = torch.float16 if args.dtype == "fp16" else torch.bfloat16
        weights = tuple(t.cuda() for t in inputs.ffn_weights(dtype=dt))
        # one runtime device copy of known size (W_gate, 100,663,296 bytes read and written): the
        # calibration of a profiler's memory counters
        calibration = weights[0].clone()
        torch.cuda.synchronize()
        del calibration
        out = long_sequence(weights, steps=args.steps, warmup=args.warmup, samples=args.samples)
        out["dtype"] = args.dtype
        print(json.dumps({"long_sequence": out}), flush=True)
        return

    if args.workload == "rank32":
        print(json.dumps({"one_rank": one_rank(args)}), flush=True)
        return

    M = 32
    wg_c, wu_c, wd_c = inputs.ffn_weights()
    W = [(wg_c.cuda(), wu_c.cuda(), wd_c.cuda())]
    for _ in range(args.copies - 1):
        W.append(tuple(t.clone() for t in W[0]))
    x_c, dy_c = inputs.activations(M)
    x, dy = x_c.cuda(), dy_c.cuda()
    torch.cuda.synchronize()

    def step(k):
        wg, wu, wd = W[k % len(W)]
        y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
        return dgf.ffn_bwd(dy, x, g, u, wg, wu, wd)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    print("[bench] warmup done", file=sys.stderr, flush=True)

    # the timed regions: `samples` regions of exactly K steps, each between two
    # synchronisations, nothing else recorded; the step time is their median
    wall0 = time.perf_counter()
    st = sample_us(step, args.steps, args.samples)
    wall = time.perf_counter() - wall0
    ms_step = st["median"] * 1e-3
    value = step_bytes(M) / (ms_step * 1e-3) / 1e9
    print(f"[bench] fwd+bwd M=32: {ms_step * 1e3:.1f} us/step (median of {args.samples}; "
          f"{st['min']:.1f}..{st['max']:.1f}), {value:.0f} GB/s", file=sys.stderr, flush=True)

    # a second, profiled region of K steps: HIP events around every launch, on
    # the launch stream (they add their own gaps, so the step time comes from
    # the region above)
    timer = dgf.KernelTimer(max_kernels=32 * args.steps + 64)
    torch.cuda.synchronize()
    p_start, p_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p_start.record()
    timer.start()
    for k in range(args.steps):
        step(k)
    timer.stop()
    p_end.record()
    torch.cuda.synchronize()
    ms_step_profiled = p_start.elapsed_time(p_end) / args.steps

    per = {}
    for name, ms in timer.durations_ms():
        per.setdefault(name, []).append(ms)
    kernels = {n: {"launches": len(v), "avg_us": 1e3 * sum(v) / len(v), "median_us": round(1e3 * sorted(v)[len(v) // 2], 2),
                   "min_us": round(1e3 * min(v), 2), "max_us": round(1e3 * max(v), 2)} for n, v in per.items()}
    dom = max(per, key=lambda n: sum(per[n]))
    dom_us = kernels[dom]["avg_us"]
    dom_bytes = kernel_bytes(dom, M)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9 if dom_bytes else None
    for n, v in kernels.items():
        b = kernel_bytes(n, M)
        v["GBps"] = round(b / (v["avg_us"] * 1e-6) / 1e9, 1) if b else None
        v["avg_us"] = round(v["avg_us"], 2)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "samples": args.samples,
        "ms_per_step": round(ms_step, 4),
        "us_per_step_min": round(st["min"], 2),
        "us_per_step_max": round(st["max"], 2),
        "us_per_step_samples": st["samples"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "deterministic gated FFN training step (forward + backward), Qwen3-8B shape, "
                               "M=32 tokens, H=4096, I=12288, BF16, weights [out,in] N(0,0.02), x and dY N(0,1)",
                   "M": M, "H": H, "I": I, "weight_copies_rotated": len(W),
                   "step_algorithmic_bytes": step_bytes(M)},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1) if achieved else None,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None,
                     "bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 2),
                     "traffic": measured_traffic(dom)},
        "kernels": kernels,
        "kernels_note": "per-launch HIP events in a second region of the same K steps "
                        f"({ms_step_profiled * 1e3:.1f} us/step with the events)",
        "wall_s_timed_region": round(wall, 3),
    }

    if not args.quick:
        fwd = {}
        for Mf in (1, 8, 32):
            xf = x[:Mf]

            def fwd_m(k, xf=xf):
                wg, wu, wd = W[k % len(W)]
                dgf.ffn_fwd(xf, wg, wu, wd)

            for k in range(args.warmup):
                fwd_m(k)
            fwd[str(Mf)] = stats_entry(sample_us(fwd_m, args.steps, args.samples), fwd_bytes(Mf))
            print(f"[bench] forward M={Mf}: {fwd[str(Mf)]['us']:.1f} us, {fwd[str(Mf)]['GBps']:.0f} GB/s",
                  file=sys.stderr, flush=True)
        result["forward"] = fwd
        result["fwd_bwd_us"] = round(ms_step * 1e3, 2)
        # the training step (forward with g/u saved, then backward) at 1 and 8 tokens as well
        fb = {}
        for Mf in (1, 8):
            xf, dyf = x[:Mf], dy[:Mf]

            def step_m(k, xf=xf, dyf=dyf):
                wg, wu, wd = W[k % len(W)]
                y, g, u = dgf.ffn_fwd(xf, wg, wu, wd, training=True)
                return dgf.ffn_bwd(dyf, xf, g, u, wg, wu, wd)

            for k in range(args.warmup):
                step_m(k)
            fb[str(Mf)] = stats_entry(sample_us(step_m, args.steps, args.samples), step_bytes(Mf))
            print(f"[bench] fwd+bwd M={Mf}: {fb[str(Mf)]['us']:.1f} us, {fb[str(Mf)]['GBps']:.0f} GB/s",
                  file=sys.stderr, flush=True)
        fb["32"] = stats_entry(st, step_bytes(M))
        result["fwd_bwd"] = fb
        result["two_stream_lanes"] = two_stream_lanes(W, x, dy, args, kernels)
        result["shards"] = shard_legs(W, x, dy, args, fwd["32"]["us"], result["fwd_bwd"]["32"]["us"])

    if not args.quick:
        result["long_sequence"] = long_sequence(W[0], samples=args.samples)
        result["fp16"] = fp16_leg(args)

    if not args.no_cpu_baseline and not args.quick:
        # the outputs of one step, kept as BF16 bits for the comparison with the oracle's sample
        wg, wu, wd = W[0]
        y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
        r = dgf.ffn_bwd(dy, x, g, u, wg, wu, wd)
        torch.cuda.synchronize()
        gpu = {k: inputs.bits(t) for k, t in {"y": y, "g": g, "u": u, **r}.items()}
        result["cpu_baseline"], result["oracle_parity"] = cpu_baseline(M, gpu)

    print(json.dumps(result), flush=True)


def fp16_leg(args) -> dict:
    """The same workloads in FP16 storage (the *_typed entry points, one tree for
    both types): the M=32 training step, the forward at 1/8/32 tokens and the
    M=4096 step.  Bytes and flops per step are those of the BF16 workloads."""
    import torch
    from deterministic_gated_ffn_amd import binding as dgf
    from deterministic_gated_ffn_amd import inputs

    F16 = torch.float16
    wg_c, wu_c, wd_c = inputs.ffn_weights(dtype=F16)
    W = [(wg_c.cuda(), wu_c.cuda(), wd_c.cuda())]
    for _ in range(args.copies - 1):
        W.append(tuple(t.clone() for t in W[0]))
    M = 32
    x_c, dy_c = inputs.activations(M, dtype=F16)
    x, dy = x_c.cuda(), dy_c.cuda()

    def step(k):
        wg, wu, wd = W[k % len(W)]
        y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
        return dgf.ffn_bwd(dy, x, g, u, wg, wu, wd)

    for k in range(args.warmup):
        step(k)
    out = {"dtype": "f16", "fwd_bwd": {"32": stats_entry(sample_us(step, args.steps, args.samples), step_bytes(M))}}
    fwd = {}
    for Mf in (1, 8, 32):
        xf = x[:Mf]

        def fwd_m(k, xf=xf):
            wg, wu, wd = W[k % len(W)]
            dgf.ffn_fwd(xf, wg, wu, wd)

        for k in range(args.warmup):
            fwd_m(k)
        fwd[str(Mf)] = stats_entry(sample_us(fwd_m, args.steps, args.samples), fwd_bytes(Mf))
    out["forward"] = fwd
    print(f"[bench] FP16: fwd+bwd M=32 {out['fwd_bwd']['32']['us']:.1f} us; forward M=1/8/32 "
          f"{fwd['1']['us']:.1f}/{fwd['8']['us']:.1f}/{fwd['32']['us']:.1f} us", file=sys.stderr, flush=True)
    out["long_sequence"] = long_sequence(W[0], samples=args.samples)
    del W
    return out


def long_sequence(weights, M: int = 4096, steps: int = 5, warmup: int = 2, samples: int = 5) -> dict:
    """The compute-bound shape: fwd+bwd at M=4096 tokens (8 sequences x 512),
    `samples` regions of `steps` steps; 18 M H I flops per step (nine products).
    The stored type is the weights' (FP16 takes the same 2.5 PFLOP/s MFMA peak)."""
    import torch
    from deterministic_gated_ffn_amd import binding as dgf
    from deterministic_gated_ffn_amd import inputs

    wg, wu, wd = weights
    x_c, dy_c = inputs.activations(M, dtype=wg.dtype)
    x, dy = x_c.cuda(), dy_c.cuda()

    def step(k):
        y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
        return dgf.ffn_bwd(dy, x, g, u, wg, wu, wd)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    st = sample_us(step, steps, samples)
    flops = 18 * M * H * I
    out = {"M": M, "ms_per_step": round(st["median"] * 1e-3, 4), "ms_min": round(st["min"] * 1e-3, 4),
           "ms_max": round(st["max"] * 1e-3, 4), "flops_per_step": flops,
           "TFLOPs": round(flops / (st["median"] * 1e-6) / 1e12, 2), "peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS,
           "steps": steps, "samples": samples, "samples_ms": [round(v * 1e-3, 4) for v in st["samples"]]}
    out["frac_mfma_peak"] = round(out["TFLOPs"] / BF16_MFMA_PEAK_TFLOPS, 4)
    # the forward alone at the same shape (inference mode)
    for k in range(warmup):
        dgf.ffn_fwd(x, wg, wu, wd)
    fs = sample_us(lambda k: dgf.ffn_fwd(x, wg, wu, wd), steps, samples)
    out["forward"] = stats_entry(fs, flops=6 * M * H * I)
    print(f"[bench] fwd+bwd M={M}: {out['ms_per_step']:.3f} ms, {out['TFLOPs']:.1f} TFLOP/s; "
          f"forward {fs['median'] * 1e-3:.3f} ms", file=sys.stderr, flush=True)
    return out


def two_stream_lanes(W, x, dy, args, kernels) -> dict:
    """The dX lanes at M=32 three ways, from the same dG and dU: the two lane
    GEMMs on two streams joined by events, then the ordered add (the pages'
    next step for the backward); the same calls on one stream; and the
    library's own one-launch lanes (its kernel time, from the profiled region,
    plus the join that runs inside the weight-gradient launch)."""
    import torch
    from deterministic_gated_ffn_amd import binding as dgf
    from deterministic_gated_ffn_amd import schedules

    wg, wu, wd = W[0]
    y, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
    dA = dgf.gemm_tree("NN", dy, wd)
    dG, dU, _ = dgf.act_bwd(dA, g, u)
    torch.cuda.synchronize()
    two = schedules.TwoStreamLanes()
    copies = [(W[k][0], W[k][1]) for k in range(len(W))]
    run_two = lambda k: two(dG, dU, *copies[k % len(copies)])
    run_serial = lambda k: schedules.serial_lanes(dG, dU, *copies[k % len(copies)])
    for k in range(args.warmup):
        run_two(k)
        run_serial(k)
    out = {"two_streams": stats_entry(sample_us(run_two, args.steps, args.samples)),
           "one_stream": stats_entry(sample_us(run_serial, args.steps, args.samples)),
           "fused_lanes_kernel_us": kernels.get("dX lanes tree GEMM", {}).get("avg_us"),
           "note": "two NN tree GEMMs (gate lane, up lane) and the two-part rank tree for the ordered add; "
                   "the fused figure is the library's one-launch lanes kernel, whose join runs on extra "
                   "workgroups of the dW_gate/dW_up launch"}
    print(f"[bench] dX lanes: two streams {out['two_streams']['us']:.1f} us, one stream "
          f"{out['one_stream']['us']:.1f} us, fused launch {out['fused_lanes_kernel_us']} us",
          file=sys.stderr, flush=True)
    return out


def shard_legs(W, x, dy, args, fwd_us: float, step_us: float) -> dict:
    """The I-sharded forward and training step at M=32 on one GPU, S = 2, 4, 8:
    every shard's forward (and backward, its dX lanes kept) on the weight
    shard views (W_gate, W_up rows and W_down columns of the I range), then
    the rank-tree combines: y over the shards; the gate lane and the up lane
    over the shards, then dX = combine(G, U), the gate lane first.  Checked
    bitwise against the unsharded call before timing; the overhead is against
    the unsharded figures of the same run."""
    import torch
    from deterministic_gated_ffn_amd import binding as dgf
    from deterministic_gated_ffn_amd import inputs

    H, I = x.shape[1], W[0][0].shape[0]
    out = {}
    for S in (2, 4, 8):
        Is = I // S
        # the shard views of every weight copy, made once: slicing tensors in the timed calls
        # would make the host, not the GPU, the bottleneck at 8 shards
        shard_views = [[(wg[r * Is:(r + 1) * Is], wu[r * Is:(r + 1) * Is], wd[:, r * Is:(r + 1) * Is]) for r in range(S)]
                       for (wg, wu, wd) in W]

        def views(k, shard_views=shard_views):
            return shard_views[k % len(shard_views)]

        def fwd_s(k):
            return dgf.tree_combine([dgf.ffn_fwd(x, *v) for v in views(k)])

        def step_s(k):
            ys, Gs, Us = [], [], []
            for v in views(k):
                y, g, u = dgf.ffn_fwd(x, *v, training=True)
                r = dgf.ffn_bwd(dy, x, g, u, *v, lanes=True)
                ys.append(y); Gs.append(r["G"]); Us.append(r["U"])
            G, U = dgf.tree_combine(Gs), dgf.tree_combine(Us)
            return dgf.tree_combine(ys), dgf.tree_combine([G, U])

        wg, wu, wd = W[0]
        y_full, g, u = dgf.ffn_fwd(x, wg, wu, wd, training=True)
        dx_full = dgf.ffn_bwd(dy, x, g, u, wg, wu, wd)["dX"]
        y_s, dx_s = step_s(0)
        same = bool((inputs.bits(fwd_s(0)) == inputs.bits(y_full)).all()
                    and (inputs.bits(y_s) == inputs.bits(y_full)).all()
                    and (inputs.bits(dx_s) == inputs.bits(dx_full)).all())
        for k in range(args.warmup):
            fwd_s(k)
            step_s(k)
        f = stats_entry(sample_us(fwd_s, args.steps, args.samples), fwd_bytes(x.shape[0]))
        t = stats_entry(sample_us(step_s, args.steps, args.samples), step_bytes(x.shape[0]))

        # one rank's share: shard 0's forward and step alone (what each of S GPUs would compute)
        def fwd_0(k):
            return dgf.ffn_fwd(x, *views(k)[0])

        def step_0(k):
            v = views(k)[0]
            y, g, u = dgf.ffn_fwd(x, *v, training=True)
            return dgf.ffn_bwd(dy, x, g, u, *v, lanes=True)

        for k in range(args.warmup):
            fwd_0(k)
            step_0(k)
        f0 = stats_entry(sample_us(fwd_0, args.steps, args.samples))
        t0 = stats_entry(sample_us(step_0, args.steps, args.samples))
        out[str(S)] = {"forward": f, "fwd_bwd": t, "bitwise_equal_to_unsharded": same,
                       "forward_overhead_us": round(f["us"] - fwd_us, 2),
                       "fwd_bwd_overhead_us": round(t["us"] - step_us, 2),
                       "one_shard_forward": f0, "one_shard_fwd_bwd": t0}
        print(f"[bench] I-shards S={S}: all shards forward {f['us']:.1f} us (+{f['us'] - fwd_us:.1f}), fwd+bwd "
              f"{t['us']:.1f} us (+{t['us'] - step_us:.1f}); one shard {f0['us']:.1f} / {t0['us']:.1f} us; "
              f"bitwise {'equal' if same else 'DIFFERENT'}", file=sys.stderr, flush=True)
    out["note"] = ("all shards of one GPU run one after the other on one stream, then the combines: the overhead "
                   "is their extra launches and smaller grids, not a multi-GPU figure; one_shard_* is one "
                   "rank's own compute at I/S (no exchange)")
    return out


def one_rank(args) -> dict:
    """Shard 0 of the I-sharded M=32 forward and training step at --shards
    shards (W_gate and W_up rows, W_down columns of the first I / S): the
    forward alone (--warmup calls, then --samples regions of --steps), then
    the forward with g and u saved followed by the backward with its dX lanes
    kept, timed the same way, over --copies resident weight copies."""
    import torch
    from deterministic_gated_ffn_amd import binding as dgf
    from deterministic_gated_ffn_amd import inputs

    M, S = 32, args.shards
    w0 = tuple(t.cuda() for t in inputs.ffn_weights())
    W = [w0] + [tuple(t.clone() for t in w0) for _ in range(args.copies - 1)]
    Is = w0[0].shape[0] // S
    views = [(wg[:Is], wu[:Is], wd[:, :Is]) for (wg, wu, wd) in W]
    x_c, dy_c = inputs.activations(M)
    x, dy = x_c.cuda(), dy_c.cuda()
    torch.cuda.synchronize()

    def fwd(k):
        return dgf.ffn_fwd(x, *views[k % len(views)])

    def step(k):
        v = views[k % len(views)]
        y, g, u = dgf.ffn_fwd(x, *v, training=True)
        return dgf.ffn_bwd(dy, x, g, u, *v, lanes=True)

    for k in range(args.warmup):
        fwd(k)
    f = stats_entry(sample_us(fwd, args.steps, args.samples))
    for k in range(args.warmup):
        step(k)
    t = stats_entry(sample_us(step, args.steps, args.samples))
    print(f"[bench] one rank of {S} I-shards (I = {Is}): forward {f['us']:.1f} us, fwd+bwd {t['us']:.1f} us",
          file=sys.stderr, flush=True)
    return {"shards": S, "I_shard": Is, "M": M, "forward": f, "fwd_bwd": t}


def ordinal(b):
    """BF16 bit patterns as integers in value order (+0 and -0 both 0), so that
    the difference of two is their distance in ulps."""
    import numpy as np
    b = np.asarray(b, np.uint16).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)


def cpu_baseline(M: int, gpu: dict) -> tuple[dict, dict]:
    """The CPU oracle on a bounded sample of the same step: the full M=32
    forward, the full dA and dX, and 1/16 of the dW rows (scaled by 16).
    Also compares that sample with the same elements of the step's outputs on
    the GPU (`gpu`: BF16 bits of y, g, u, dX, dW_gate, dW_up, dW_down)."""
    import numpy as np

    import oracle
    from deterministic_gated_ffn_amd import inputs

    os.environ.setdefault("OMP_NUM_THREADS", str(len(os.sched_getaffinity(0))))
    cores = int(os.environ["OMP_NUM_THREADS"])
    oracle.lib()
    wg, wu, wd = (inputs.bits(t) for t in inputs.ffn_weights())
    x, dy = (inputs.bits(t) for t in inputs.activations(M))
    t0 = time.perf_counter()
    o = oracle.ffn_fwd(x, wg, wu, wd)
    t_fwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    da = oracle.gemm_tree(dy, wd, "NN")
    dg, du, a = oracle.act_bwd(da, o["g"], o["u"])
    G = oracle.gemm_tree(dg, wg, "NN")
    U = oracle.gemm_tree(du, wu, "NN")
    dx = oracle.tree_combine([G, U]).reshape(M, H)
    t_dx = time.perf_counter() - t0
    frac = 16
    t0 = time.perf_counter()
    dwg = oracle.gemm_tree(np.ascontiguousarray(dg[:, :I // frac]), x, "TN")
    dwu = oracle.gemm_tree(np.ascontiguousarray(du[:, :I // frac]), x, "TN")
    dwd = oracle.gemm_tree(np.ascontiguousarray(dy[:, :H // frac]), a, "TN")
    t_dw = (time.perf_counter() - t0) * frac
    total = t_fwd + t_dx + t_dw
    baseline = {"value": round(step_bytes(M) / total / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"C oracle (OpenMP, {os.environ.get('OMP_NUM_THREADS')} threads) on the M=32 training step: "
                          f"full forward ({t_fwd:.1f} s), full dA/dsilu/dX ({t_dx:.1f} s), dW on 1/{frac} of the rows "
                          f"scaled x{frac} ({t_dw:.1f} s)",
                "seconds_per_step": round(total, 2), "cpu": platform.processor() or platform.machine(),
                "os_cpu_count": os.cpu_count()}

    # the GPU step's outputs against the oracle on the same elements: exact BF16 matches and ulp distances
    pairs = {"y": (gpu["y"], o["y"]), "g": (gpu["g"], o["g"]), "u": (gpu["u"], o["u"]), "dX": (gpu["dX"], dx),
             "dW_gate": (gpu["dW_gate"][:I // frac], dwg), "dW_up": (gpu["dW_up"][:I // frac], dwu),
             "dW_down": (gpu["dW_down"][:H // frac], dwd)}
    per, n_all, bad_all, ulp_all = {}, 0, 0, 0
    for k, (got, ref) in pairs.items():
        got, ref = np.asarray(got, np.uint16), np.asarray(ref, np.uint16).reshape(np.shape(got))
        bad = int((got != ref).sum())
        ulp = int(np.abs(ordinal(got) - ordinal(ref)).max()) if got.size else 0
        per[k] = {"elements": int(got.size), "mismatches": bad, "max_ulp": ulp}
        n_all, bad_all, ulp_all = n_all + got.size, bad_all + bad, max(ulp_all, ulp)
    # the same GPU outputs against the float64 brute-force FFN (no intermediate rounding)
    from oracle import fp64
    f = fp64.ffn_fwd(x, wg, wu, wd)
    fb = fp64.ffn_bwd(dy, x, wg, wu, wd)
    rel = {"y": fp64.rel_l2(gpu["y"], f["y"]), "g": fp64.rel_l2(gpu["g"], f["g"]), "u": fp64.rel_l2(gpu["u"], f["u"]),
           "dX": fp64.rel_l2(gpu["dX"], fb["dX"]),
           "dW_gate": fp64.rel_l2(gpu["dW_gate"][:I // frac], fb["dW_gate"][:I // frac]),
           "dW_up": fp64.rel_l2(gpu["dW_up"][:I // frac], fb["dW_up"][:I // frac]),
           "dW_down": fp64.rel_l2(gpu["dW_down"][:H // frac], fb["dW_down"][:H // frac])}
    del f, fb
    parity = {"vs": "oracle", "elements": int(n_all), "mismatches": bad_all,
              "rel_l2_vs_fp64": {k: float(f"{v:.3e}") for k, v in rel.items()},
              "rel_l2_vs_fp64_max": float(f"{max(rel.values()):.3e}"), "rel_l2_bar": 1e-2,
              "exact_match_fraction": round(1 - bad_all / n_all, 9) if n_all else None, "max_ulp": ulp_all,
              "outputs": per,
              "sample": f"the M=32 training step on weight copy 0: y, g, u and dX in full, the first 1/{frac} "
                        "of the rows of dW_gate, dW_up and dW_down"}
    return baseline, parity


if __name__ == "__main__":
    main()
