"""Benchmark: fused GEMM + bias + activation on one MI355X.

A step is one execute of the planned fused kernel over the workload's
inputs, which are resident in HBM before timing starts.  Default workload:
the pages' H200 benchmark shape, A 65536x16384 times B 16384x8192, bf16,
bias over rows + ReLU (RELU_BIAS), bf16 output.

Prints ONE JSON line with the throughput (TFLOP/s for MFMA-bound workloads,
GB/s for the batch-16 Linear), the roofline of the dominant kernel (kernel
duration from HIP events on the launch stream), the unfused two-kernel pair
timed in the same run, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "e4m3": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = ["tile_kernel.h", "smallm_kernel.hip", "ge_device.h", "ge_params.h"]


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="C5a")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-unfused", action="store_true")
    p.add_argument("--rotate", type=int, default=None,
                   help="copies of the operands cycled through (defeats the 256 MiB MALL "
                        "for HBM-bound workloads); default 16 for the batch-16 Linear, else 1")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead: run a plain device copy of MIB MiB (counter calibration)")
    return p.parse_args()


def kernel_src_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "activation_epilogue_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, launches_bytes_alg: float):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path)).get(workload)
    except Exception:
        return None
    if not t or t.get("kernel_src_hash") != kernel_src_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def copy_calibration(mib: int, steps: int):
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": steps}))


def cpu_baseline(w, inp, seconds: float, unit: str):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole rows of D (all of K) through its GEMM, bias and activation passes,
    repeated on further rows until about `seconds` of CPU time is spent."""
    import numpy as np
    import torch

    import oracle
    import synth

    def raw(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.float32:
            return t.numpy()
        if t.dtype == torch.float8_e4m3fn:
            return t.view(torch.uint8).numpy()
        return t.view(torch.int16).numpy().view(np.uint16)

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    Bc = raw(inp.B)
    bias = raw(inp.bias).reshape(-1)
    sa = float(inp.scale_a.item()) if inp.scale_a is not None else 1.0
    sb = float(inp.scale_b.item()) if inp.scale_b is not None else 1.0
    rows = max(1, min(w.m, threads))
    done, t_total = 0, 0.0
    while done < w.m and t_total < seconds:
        rows = min(rows, w.m - done)
        A_rows = raw(inp.A[done:done + rows])
        t0 = time.perf_counter()
        C = oracle.gemm(A_rows, w.in_dtype, Bc, w.in_dtype, w.op_b, sa, sb)
        b = bias[done:done + rows] if w.axis == "row" else bias
        P = oracle.bias_pass(C, b, w.out_dtype, w.axis)
        oracle.act_pass(P, w.epilog)
        dt = time.perf_counter() - t0
        t_total += dt
        done += rows
        if dt < seconds / 4:
            rows *= 2
    es, eo = synth.ELEM_SIZE[w.in_dtype], synth.ELEM_SIZE[w.out_dtype]
    flops = 2.0 * done * w.n * w.k
    nbytes = done * w.k * es + w.k * w.n * es + done * w.n * eo
    value = flops / t_total / 1e12 if unit == "TFLOP/s" else nbytes / t_total / 1e9
    return {"value": round(value, 6), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{done} of {w.m} rows of D ({done}x{w.n} outputs, full K={w.k}) through the "
                      f"oracle's fp64 GEMM, bias and activation passes in {t_total:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the op shards by rows of A or columns of B with no exchange step; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(args.steps, 1))
        return

    import synth
    from activation_epilogue_02_amd import binding as B

    if not os.path.exists(B.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    w = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    hbm_bound = w.m <= 16
    rot = args.rotate if args.rotate is not None else (16 if hbm_bound else 1)

    inp = synth.make_inputs(w, device="cuda")
    copies = [inp]
    for r in range(1, rot):
        copies.append(synth.make_inputs(w, device="cuda", seed=w.seed + 100 * r))
    bias = [c.bias.reshape(-1).contiguous() for c in copies]

    t0 = time.perf_counter()
    g = B.GemmEpilog(w.m, w.n, w.k, w.in_dtype, w.out_dtype, w.op_b)
    g.plan(w.epilog, w.axis)
    plan_us = (time.perf_counter() - t0) * 1e6
    desc = g.describe()
    outs = [g.alloc_outputs(dev) for _ in range(rot)]

    stream = torch.cuda.current_stream()

    def step(i, h=g, outputs=outs):
        c = copies[i % rot]
        D, aux, ws = outputs[i % rot]
        B.gemm_epilog_execute(h.h, c.A, c.B, bias[i % rot], D, aux, c.scale_a, c.scale_b, ws,
                              None if ws is None else ws.numel(), stream.cuda_stream)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            fn(i)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        durs = [a.elapsed_time(b) for a, b in ev]
        return wall, durs

    wall, durs = timed(step)
    ms_per_step = wall * 1e3 / args.steps
    kern_ms = sum(durs) / len(durs)

    unfused = None
    if not args.no_unfused and w.epilog != "none":
        gu = B.GemmEpilog(w.m, w.n, w.k, w.in_dtype, w.out_dtype, w.op_b)
        gu.plan(w.epilog, w.axis, unfused=1)
        outs_u = [gu.alloc_outputs(dev) for _ in range(rot)]
        wall_u, durs_u = timed(lambda i: step(i, gu, outs_u))
        # interleave once more with the fused kernel to be fair to clocks
        wall2, durs2 = timed(step)
        kern_ms = min(kern_ms, sum(durs2) / len(durs2))
        ms_per_step = min(ms_per_step, wall2 * 1e3 / args.steps)
        ku = sum(durs_u) / len(durs_u)
        unfused = {"ms_per_step": round(wall_u * 1e3 / args.steps, 4), "kernel_pair_ms": round(ku, 4),
                   "fused_speedup": round(ku / kern_ms, 4), "plan": gu.describe()}
        del outs_u
        gu.free()

    alg_bytes = w.algorithmic_bytes()
    if hbm_bound:
        value = alg_bytes / (ms_per_step / 1e3) / 1e9
        metric_unit = "GB/s"
        achieved = alg_bytes / (kern_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        value = w.flops / (ms_per_step / 1e3) / 1e12
        metric_unit = "TFLOP/s"
        achieved = w.flops / (kern_ms / 1e3) / 1e12
        peak = PEAK_TFLOPS[w.in_dtype]
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    roof["traffic"] = traffic_for(args.workload, alg_bytes)
    roof["kernel_ms"] = round(kern_ms, 4)
    roof["algorithmic_bytes_per_launch"] = alg_bytes
    roof["flops_per_launch"] = w.flops

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, args.cpu_seconds, metric_unit)

    out = {
        "metric": "fused GEMM+bias+act TFLOP/s and % MFMA peak; HBM GB/s at batch 16",
        "value": round(value, 3),
        "unit": metric_unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "data": "synthetic (seeded; see DESIGN.md input recipe)",
        "config": {"workload": w.name, "m": w.m, "n": w.n, "k": w.k, "epilog": w.epilog,
                   "bias_axis": w.axis, "op_b": w.op_b, "out_dtype": w.out_dtype,
                   "operand_copies": rot, "plan": desc, "plan_us": round(plan_us, 1)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "unfused": unfused,
        "gpu": torch.cuda.get_device_name(0),
        "torch": torch.__version__,
        "hip": torch.version.hip,
    }
    print(json.dumps(out), flush=True)
    g.free()


if __name__ == "__main__":
    main()
