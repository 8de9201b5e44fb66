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

PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "e4m3": 5000.0, "mxf8": 5000.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "activation_epilogue_02_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# HBM-traffic counters: FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each
# scaled by what it reads for a plain device copy of known size
COPY_MIB = 1024


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="C5a")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-unfused", action="store_true")
    p.add_argument("--no-small-m", action="store_true",
                   help="skip the nested batch-16 Linear record of the default run")
    p.add_argument("--rotate", type=int, default=None,
                   help="copies of the operands cycled through (defeats the 256 MiB MALL "
                        "for HBM-bound workloads); default 16 for the batch-16 Linear, else 1")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--group-m", type=int, default=0,
                   help="tile rows per group of the launch order (0 = the planner's choice)")
    p.add_argument("--tile", type=int, default=0,
                   help="force a tile id of the planner (0 = its own choice)")
    p.add_argument("--autotune", action="store_true",
                   help="let gemm_epilog_autotune pick the kernel on the workload's buffers before timing")
    p.add_argument("--no-graph", action="store_true",
                   help="launch each step from Python instead of replaying the K steps as one "
                        "captured HIP graph (then host launch latency shows in the timings)")
    p.add_argument("--split-k", type=int, default=0,
                   help="force the K split of the small-m path (0 = the planner's choice)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="instead: run a plain device copy of MIB MiB (counter calibration)")
    p.add_argument("--digest", default=None, metavar="DIR",
                   help="instead: summarise the rocprofv3 runs under DIR for --workload into "
                        "profiles/ (no GPU needed)")
    return p.parse_args()


def kernel_src_hash() -> str:
    """Hash of every kernel and launch source: counters taken on other
    sources do not describe the kernel being timed."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str):
    """HBM bytes per launch of the dominant kernel, from the committed
    rocprofv3 counter runs, if they were taken on the current kernel sources;
    else None."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        t = json.load(open(path)).get(workload)
    except (OSError, ValueError):
        return None
    if not t or t.get("kernel_src_hash") != kernel_src_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# ---- profile digest (host only) ------------------------------------------------------
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -d {d}/prof_{wll}_trace -o run --output-format csv "
             "-- python3 bench.py --workload {wl} --steps {steps} --warmup 2 --no-cpu-baseline --no-small-m",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -d {d}/prof_{wll}_fetch -o run --output-format csv "
             "-- python3 bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline --no-unfused "
             "--no-graph --no-small-m",
    "write": "rocprofv3 --pmc WRITE_SIZE -d {d}/prof_{wll}_write -o run --output-format csv "
             "-- python3 bench.py --workload {wl} --steps 3 --warmup 1 --no-cpu-baseline --no-unfused "
             "--no-graph --no-small-m",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE -d {d}/prof_copy_fetch -o run --output-format csv "
                  "-- python3 bench.py --copy-calibration 1024 --steps 3",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE -d {d}/prof_copy_write -o run --output-format csv "
                  "-- python3 bench.py --copy-calibration 1024 --steps 3",
}

def _dominant(stats):
    """The fused kernel: the library kernel (ge::ge_*, not the unfused pair's
    elementwise pass or the counter clear) with the most GPU time."""
    cands = [r for r in stats if "ge::ge_" in r["Name"] and "ge_ew_kernel" not in r["Name"]
             and "ge_clear" not in r["Name"] and "ge_bgrad_reduce" not in r["Name"]
             and "ge_sum_kernel" not in r["Name"]]
    if not cands:
        raise SystemExit("digest: no fused library kernel in the kernel stats")
    return max(cands, key=lambda r: float(r["TotalDurationNs"]))


def _csv(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _counter_avg(dirpath, name_part, counter):
    rows = [r for r in _csv(os.path.join(dirpath, "run_counter_collection.csv"))
            if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not rows:
        raise SystemExit(f"digest: no {counter} rows for {name_part} in {dirpath}")
    vals = [float(r["Counter_Value"]) for r in rows]
    return sum(vals) / len(vals), len(vals), rows[0]["Kernel_Name"]


def _last_json(path):
    line = None
    with open(path) as fh:
        for ln in fh:
            if ln.startswith("{"):
                line = ln
    return json.loads(line) if line else None


def digest(d: str, wl: str):
    """Turn the rocprofv3 CSVs of one workload (kernel trace + stats, a
    FETCH_SIZE and a WRITE_SIZE pass) and of the copy calibration into a
    short text summary under profiles/ and the traffic figure bench.py
    reports.  The kernel-source hash comes from the profiled run's own bench
    line, so the figure is dropped once the kernel changes."""
    import synth
    w = synth.WORKLOADS[wl]
    stats = _csv(os.path.join(d, f"prof_{wl.lower()}_trace", "run_kernel_stats.csv"))
    run = _last_json(os.path.join(d, f"prof_{wl.lower()}_trace.log"))
    if run is None:
        raise SystemExit("digest: the traced bench run printed no JSON line")
    k = _dominant(stats)
    part = k["Name"].split("(")[0].replace("void ", "")   # template name with arguments
    avg_ns = float(k["AverageNs"])
    fetch_kib, nf, kname = _counter_avg(os.path.join(d, f"prof_{wl.lower()}_fetch"), part, "FETCH_SIZE")
    write_kib, nw, _ = _counter_avg(os.path.join(d, f"prof_{wl.lower()}_write"), part, "WRITE_SIZE")
    cf, _, _ = _counter_avg(os.path.join(d, "prof_copy_fetch"), "copyBuffer", "FETCH_SIZE")
    cw, _, _ = _counter_avg(os.path.join(d, "prof_copy_write"), "copyBuffer", "WRITE_SIZE")
    copy_kib = COPY_MIB * 1024.0
    f_scale, w_scale = copy_kib / cf, copy_kib / cw
    read_b = fetch_kib * 1024 * f_scale
    write_b = write_kib * 1024 * w_scale
    traffic = read_b + write_b
    alg = w.algorithmic_bytes()
    steps = run.get("steps", 10)
    cmds = {key: c.format(d="gpurun_out", wl=wl, wll=wl.lower(), steps=steps)
            for key, c in PROFILE_COMMANDS.items()}
    name = part.replace("ge::", "").split("<")[0] + "_" + wl
    lines = [
        f"# {part} on {w.name}",
        "",
        f"kernel-source hash: {run.get('kernel_src_hash')}   plan: {run['config']['plan']}",
        "",
        "Commands (run from the repository root on an MI355X, rocprofv3 "
        "output under gpurun_out/):",
        "",
    ] + [f"    {c}" for c in cmds.values()] + [
        "",
        "## Kernel trace statistics (rocprofv3 --stats), kernels above 0.5% of GPU time",
        "",
        "| kernel | calls | average ns | % time |",
        "|---|---|---|---|",
    ] + [f"| {r['Name'][:100]} | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['Percentage']} |"
         for r in stats if float(r["Percentage"]) > 0.5] + [
        "",
        f"Dominant kernel average duration: {avg_ns / 1e3:.3f} us "
        f"(bench.py HIP-event average in the same run: {run['roofline']['kernel_ms'] * 1e3:.3f} us).",
        "",
        "## HBM traffic per launch (rocprofv3 --pmc, one counter per run)",
        "",
        f"- FETCH_SIZE {fetch_kib:.1f} KiB/dispatch (mean of {nf}); the copy of {COPY_MIB} MiB reads "
        f"{cf:.1f} KiB -> scale {f_scale:.4f} -> {read_b / 1e9:.4f} GB read",
        f"- WRITE_SIZE {write_kib:.1f} KiB/dispatch (mean of {nw}); the copy writes {cw:.1f} KiB -> "
        f"scale {w_scale:.4f} -> {write_b / 1e9:.4f} GB written",
        f"- traffic {traffic / 1e9:.4f} GB per launch; algorithmic bytes {alg / 1e9:.4f} GB "
        f"(ratio {traffic / alg:.2f})",
        f"- at the traced average duration: {traffic / (avg_ns * 1e-9) / 1e9:.1f} GB/s of traffic",
        "",
    ]
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, name + ".md"), "w") as fh:
        fh.write("\n".join(lines))
    tpath = os.path.join(PROFILES, "traffic.json")
    table = json.load(open(tpath)) if os.path.exists(tpath) else {}
    table[wl] = {"kernel": kname, "kernel_src_hash": run.get("kernel_src_hash"),
                 "hbm_bytes_per_launch": round(traffic), "read_bytes": round(read_b),
                 "write_bytes": round(write_b), "fetch_scale": round(f_scale, 4),
                 "write_scale": round(w_scale, 4), "avg_kernel_ns": round(avg_ns)}
    with open(tpath, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
    print("\n".join(lines))


def copy_calibration(mib: int, steps: int):
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(steps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4, "launches": steps}))


def cpu_baseline(w, inp, seconds: float, unit: str, aux_in=None):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    whole rows of D (all of K) through its GEMM, bias and activation passes
    (for the backward epilogues: GEMM and DRELU / DGELU pass on the aux
    input's rows), repeated on further rows until about `seconds` of CPU time
    is spent."""
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
        if t.dtype == torch.uint8:
            return t.numpy()
        return t.view(torch.int16).numpy().view(np.uint16)

    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    grad = w.epilog in ("drelu", "dgelu", "drelu_bgrad", "dgelu_bgrad")
    mask_in = w.epilog in ("drelu", "drelu_bgrad")
    if grad:
        aux_c = aux_in.detach().cpu().contiguous()
        aux_c = aux_c.numpy().view(np.uint32) if mask_in else raw(aux_c)
    Bc = raw(inp.B)
    mx = w.in_dtype == "mxf8"
    SBc = raw(inp.mx_b) if mx else None
    bias = raw(inp.bias).reshape(-1)
    sa = float(inp.scale_a.item()) if inp.scale_a is not None else 1.0
    sb = float(inp.scale_b.item()) if inp.scale_b is not None else 1.0
    rows = max(1, min(w.m, threads))
    done, t_total, start = 0, 0.0, 0
    # whole rows of D, cycling through the rows of A (again from row 0 once
    # all are done) until about `seconds` of oracle time has been spent
    while t_total < seconds:
        rows = min(rows, w.m - start)
        A_rows = raw(inp.A[start:start + rows])
        t0 = time.perf_counter()
        if mx:
            C = oracle.gemm_mx(A_rows, "e4m3", raw(inp.mx_a[start:start + rows]), Bc, "e4m3", SBc, w.op_b)
        else:
            C = oracle.gemm(A_rows, w.in_dtype, Bc, w.in_dtype, w.op_b, sa, sb)
        if grad:
            Y = (oracle.drelu_pass(C, aux_c[start:start + rows]) if mask_in
                 else oracle.dgelu_pass(C, aux_c[start:start + rows], w.out_dtype))
            if w.epilog.endswith("_bgrad"):
                oracle.bgrad_pass(Y, w.axis)
        else:
            b = bias[start:start + rows] if w.axis == "row" else bias
            P = oracle.bias_pass(C, b, w.out_dtype, w.axis)
            oracle.act_pass(P, w.epilog)
        dt = time.perf_counter() - t0
        t_total += dt
        done += rows
        start = (start + rows) % w.m
        if dt < seconds / 4:
            rows *= 2
    es, eo = synth.ELEM_SIZE[w.in_dtype], synth.ELEM_SIZE[w.out_dtype]
    flops = 2.0 * done * w.n * w.k
    nbytes = done * w.k * es + w.k * w.n * es + done * w.n * eo
    value = flops / t_total / 1e12 if unit == "TFLOP/s" else nbytes / t_total / 1e9
    return {"value": round(value, 6), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{done} rows of D (of {w.m}; {done}x{w.n} outputs, full K={w.k}, rows taken "
                      f"in order and again from row 0 once all are done) through the oracle's fp64 "
                      f"GEMM and {'DRELU/DGELU' if grad else 'bias and activation'} passes in "
                      f"{t_total:.1f} s"}


def roofline(w, ms_per_step, kern_ms, hbm_bound):
    """(roofline dict, value, unit) of a workload: GB/s of its algorithmic
    bytes against the HBM peak for the batch-16 Linear, else TFLOP/s against
    the dense MFMA peak of its input dtype."""
    alg_bytes = w.algorithmic_bytes()
    if hbm_bound:
        value = alg_bytes / (ms_per_step / 1e3) / 1e9
        achieved = alg_bytes / (kern_ms / 1e3) / 1e9
        return ({"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                 "frac": round(achieved / PEAK_HBM_GBS, 4)}, value, "GB/s")
    value = w.flops / (ms_per_step / 1e3) / 1e12
    achieved = w.flops / (kern_ms / 1e3) / 1e12
    peak = PEAK_TFLOPS[w.in_dtype]
    return ({"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
             "frac": round(achieved / peak, 4)}, value, "TFLOP/s")


def elementwise_bytes(w) -> int:
    """Algorithmic bytes of the unfused pair's second kernel: the stored
    product read back and D written (D's dtype), the bias, and the aux (mask
    written or read, or the pre-activation written or read)."""
    eo = synth_elem(w.out_dtype)
    nb = (w.m if w.axis == "row" else w.n) * eo if w.epilog not in ("none", "drelu", "dgelu") else 0
    aux = 0
    if w.epilog in ("relu_aux_bias", "drelu", "drelu_bgrad"):
        aux = w.m * (((w.n + 127) // 128) * 16)
    elif w.epilog in ("gelu_aux_bias", "dgelu", "dgelu_bgrad"):
        aux = w.m * w.n * eo
    return 2 * w.m * w.n * eo + nb + aux


def synth_elem(dt):
    import synth
    return synth.ELEM_SIZE[dt]


def run_workload(w, args, dev, with_unfused=True, tile=0, split_k=0, autotune=False):
    """Plan and time one workload: W eager warm-up steps, then K steps
    between two synchronisations (by default replayed as one captured HIP
    graph), HIP events on the launch stream around them; the unfused pair and
    the product alone (its first kernel) timed in the same process."""
    import torch

    import synth
    from activation_epilogue_02_amd import binding as B

    hbm_bound = w.m <= 16
    rot = args.rotate if args.rotate is not None else (16 if hbm_bound else 1)
    inp = synth.make_inputs(w, device="cuda")
    copies = [inp]
    for r in range(1, rot):
        copies.append(synth.make_inputs(w, device="cuda", seed=w.seed + 100 * r))
    # backward epilogues: an aux input and no bias read; the bias-gradient
    # ones write the gradient to the bias pointer
    grad = w.epilog in ("drelu", "dgelu", "drelu_bgrad", "dgelu_bgrad")
    bgrad = w.epilog.endswith("_bgrad")
    bias = [torch.empty_like(c.bias.reshape(-1)) if bgrad else
            (None if grad else c.bias.reshape(-1).contiguous()) for c in copies]
    aux_in = [synth.make_aux(w, device="cuda", seed=w.seed + 100 * r) if grad else None
              for r in range(rot)]

    t0 = time.perf_counter()
    g = B.GemmEpilog(w.m, w.n, w.k, w.in_dtype, w.out_dtype, w.op_b)
    g.plan(w.epilog, w.axis, tile=tile, split_k=split_k, group_m=getattr(args, 'group_m', 0))
    plan_us = (time.perf_counter() - t0) * 1e6
    outs = [g.alloc_outputs(dev) for _ in range(rot)]
    if autotune:
        D0, aux0, ws0 = outs[0]
        B.gemm_epilog_autotune(g.h, copies[0].A, copies[0].B, bias[0], D0, aux_in[0] if grad else aux0,
                               copies[0].scale_a, copies[0].scale_b, ws0, iters=3,
                               stream=torch.cuda.current_stream().cuda_stream)
        outs = [g.alloc_outputs(dev) for _ in range(rot)]   # the tuned plan's workspace
    desc = g.describe()
    stream = torch.cuda.current_stream()

    def step(i, h=g, outputs=outs, with_aux_in=True):
        c = copies[i % rot]
        D, aux, ws = outputs[i % rot]
        if grad and with_aux_in:
            aux = aux_in[i % rot]
        # the stream current at call time: the capture stream while a graph
        # is being recorded
        if w.in_dtype == "mxf8":
            B.gemm_epilog_execute_mx(h.h, c.A, c.B, c.mx_a, c.mx_b, bias[i % rot] if with_aux_in else None,
                                     D, aux, c.scale_a, c.scale_b, ws, None if ws is None else ws.numel(),
                                     torch.cuda.current_stream().cuda_stream)
            return
        B.gemm_epilog_execute(h.h, c.A, c.B, bias[i % rot] if with_aux_in else None, D, aux,
                              c.scale_a, c.scale_b, ws, None if ws is None else ws.numel(),
                              torch.cuda.current_stream().cuda_stream)

    def timed(fn):
        """W eager warm-up steps, then exactly K timed steps between two
        synchronisations.  By default the K steps are captured once as a HIP
        graph (replayed once untimed, to load it) and the timed region is one
        replay: the kernels then run back to back instead of waiting for
        Python to launch each one.  Returns (wall seconds, [mean ms per step
        from HIP events on the launch stream])."""
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.no_graph:
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
            return wall, [a.elapsed_time(b) for a, b in ev]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        return wall, [e0.elapsed_time(e1) / args.steps]

    # the timed run: K steps between two synchronisations; the HIP events
    # on the launch stream give the kernel's own average duration
    wall, durs = timed(step)
    ms_per_step = wall * 1e3 / args.steps
    kern_ms = sum(durs) / len(durs)

    unfused = None
    if with_unfused and w.epilog != "none":
        gu = B.GemmEpilog(w.m, w.n, w.k, w.in_dtype, w.out_dtype, w.op_b)
        gu.plan(w.epilog, w.axis, unfused=1, tile=tile, split_k=split_k, group_m=getattr(args, 'group_m', 0))
        outs_u = [gu.alloc_outputs(dev) for _ in range(rot)]
        wall_u, durs_u = timed(lambda i: step(i, gu, outs_u))
        # the pair's first kernel alone: the product with no epilogue
        gp = B.GemmEpilog(w.m, w.n, w.k, w.in_dtype, w.out_dtype, w.op_b)
        gp.plan("none", w.axis, tile=tile, split_k=split_k, group_m=getattr(args, 'group_m', 0))
        outs_p = [gp.alloc_outputs(dev) for _ in range(rot)]
        _, durs_p = timed(lambda i: step(i, gp, outs_p, with_aux_in=False))
        # the fused kernel once more after the pair, so that the comparison
        # brackets the pair in time (clocks and temperature drift)
        _, durs2 = timed(step)
        kf = 0.5 * (kern_ms + sum(durs2) / len(durs2))
        ku = sum(durs_u) / len(durs_u)
        kp = sum(durs_p) / len(durs_p)
        ew_ms = ku - kp
        ew_b = elementwise_bytes(w)
        unfused = {"ms_per_step": round(wall_u * 1e3 / args.steps, 4), "kernel_pair_ms": round(ku, 4),
                   "fused_kernel_ms": round(kf, 4), "fused_speedup": round(ku / kf, 4),
                   "product_only_ms": round(kp, 4),
                   "elementwise_ms": round(ew_ms, 4),
                   "elementwise_GBs": round(ew_b / (ew_ms * 1e-3) / 1e9, 1) if ew_ms > 0 else None,
                   "elementwise_hbm_frac": round(ew_b / (ew_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                   if ew_ms > 0 else None,
                   "plan": gu.describe()}
        del outs_u, outs_p
        gu.free()
        gp.free()
    g.free()
    return {"ms_per_step": ms_per_step, "kern_ms": kern_ms, "hbm_bound": hbm_bound, "desc": desc,
            "plan_us": plan_us, "rot": rot, "unfused": unfused, "inp": inp, "aux_in0": aux_in[0]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the op shards by rows of A or columns of B with no exchange step; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    if args.digest:
        digest(args.digest, args.workload)
        return
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
    res = run_workload(w, args, dev, with_unfused=not args.no_unfused, tile=args.tile, split_k=args.split_k,
                       autotune=args.autotune)
    ms_per_step, kern_ms, hbm_bound = res["ms_per_step"], res["kern_ms"], res["hbm_bound"]
    roof, value, metric_unit = roofline(w, ms_per_step, kern_ms, hbm_bound)
    roof["traffic"] = traffic_for(args.workload)
    roof["kernel_ms"] = round(kern_ms, 4)
    roof["algorithmic_bytes_per_launch"] = w.algorithmic_bytes()
    roof["flops_per_launch"] = w.flops

    # the HBM half of the metric: the batch-16 Linear, timed in the same run
    # (kernel duration from HIP events, 16 rotating operand copies)
    small_m = None
    if args.workload != "C3" and not args.no_small_m:
        w3 = synth.WORKLOADS["C3"]
        r3 = run_workload(w3, args, dev, with_unfused=not args.no_unfused)
        roof3, _, _ = roofline(w3, r3["ms_per_step"], r3["kern_ms"], True)
        small_m = {"workload": w3.name, "kernel_us": round(r3["kern_ms"] * 1e3, 3),
                   "achieved_GBs": roof3["achieved"], "peak_GBs": PEAK_HBM_GBS, "hbm_frac": roof3["frac"],
                   "us_per_step": round(r3["ms_per_step"] * 1e3, 3), "plan": r3["desc"],
                   "operand_copies": r3["rot"], "unfused": r3["unfused"],
                   "traffic": traffic_for("C3")}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, res["inp"], args.cpu_seconds, metric_unit, res["aux_in0"])

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
        "timing": "eager launches, HIP events per step" if args.no_graph else
                  "K steps replayed as one captured HIP graph, HIP events around the replay",
        "config": {"workload": w.name, "m": w.m, "n": w.n, "k": w.k, "epilog": w.epilog,
                   "bias_axis": w.axis, "op_b": w.op_b, "out_dtype": w.out_dtype,
                   "operand_copies": res["rot"], "plan": res["desc"], "plan_us": round(res["plan_us"], 1),
                   "autotuned": bool(args.autotune)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "unfused": res["unfused"],
        "small_m": small_m,
        "gpu": torch.cuda.get_device_name(0),
        "torch": torch.__version__,
        "hip": torch.version.hip,
        "kernel_src_hash": kernel_src_hash(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
