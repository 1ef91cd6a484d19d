#!/usr/bin/env python3
"""Benchmark of the FP8 block-scaled NT GEMM on one MI355X.

A step is one pass over every shape of a workload, each shape one call of the library
on inputs already resident in HBM.  The default run measures the four GEMM workloads of
the flashmla.org/zh page's tables in turn and prints one JSON line whose headline is
the contiguous grouped workload (MoE prefill: {4x8192, 8x4096, 8 random} rows x
(N,K) in {(4096,7168),(7168,2048)}, the largest single-GPU configuration, bound by the
matrix cores) in FLOP/s; the dense decode (HBM-bound), dense prefill and masked grouped
workloads ride along under "workloads", each with its own step rate and the roofline of
its dominant kernel.  --workload picks one workload alone (also "quant", "small").

Each roofline is the dominant (longest) kernel's algorithmic bytes or FLOPs per launch
over its mean launch time, measured with HIP events recorded on the launch stream around
back-to-back launches that rotate over copies of the operands (so none finds its inputs
left in the Infinity Cache), against 8 TB/s or 5.0 PFLOP/s dense FP8.  The line also
carries the GPU clock sampled while the headline's dominant kernel ran, the pages' own
GB/s convention, and the CPU oracle timed on this host on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0         # MI355X dense FP8 MFMA (no sparsity)
PEAK_SCLK_MHZ = 2400.0           # the engine clock the MFMA peak is quoted at


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all",
                    choices=["all", "decode", "prefill", "contiguous", "masked", "small", "quant"])
    ap.add_argument("--shapes", default="", help="comma-separated subset of shape indices")
    ap.add_argument("--formats", default="e4m3xe4m3",
                    choices=["e4m3xe4m3", "e5m2xe5m2", "e4m3xe5m2", "e5m2xe4m3"],
                    help="operand formats A x B (the workloads are quantised to them)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches, not a graph")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip sampling the GPU clock (2 s of back-to-back launches)")
    ap.add_argument("--cpu-budget-s", type=float, default=30.0)
    ap.add_argument("--detail", default="", help="write per-shape details to this JSON file")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain device-to-device copy of MIB MiB (a kernel of "
                         "known traffic, to scale HBM byte counters under a profiler)")
    return ap.parse_args()


def workload_cases(name):
    from moe_grouped_gemm_lhs_amd import inputs as I
    return {"decode": I.decode_cases, "prefill": I.prefill_cases,
            "contiguous": I.contiguous_cases, "masked": I.masked_cases,
            "small": I.small_case}[name]()


# fp8 block quantisation: (block shape, rows, K) of bf16 inputs -- the activations of the
# prefill and decode shapes (1x128 per token) and two weight matrices (128x128 blocks)
QUANT_CASES = [("1x128", 4096, 7168), ("1x128", 128, 7168), ("128x128", 7168, 16384),
               ("128x128", 24576, 1536)]

WORKLOAD_TEXT = {
    "quant": "fp8 block quantisation of bf16 inputs: 1x128 for 4096x7168 and 128x7168 "
             "activations, 128x128 for 7168x16384 and 24576x1536 weights",
    "decode": "dense decode FP8 NT GEMM, M in {64,128} x (N,K) in {(2112,7168),(24576,1536),"
              "(32768,512),(7168,16384),(4096,7168),(7168,2048)}, 12 shapes",
    "prefill": "dense prefill FP8 NT GEMM, M=4096 x the six (N,K) pairs, 1% N(0,30) outliers",
    "contiguous": "contiguous grouped FP8 NT GEMM, {4x8192, 8x4096, 8x random multiples of 128}"
                  " rows x (N,K) in {(4096,7168),(7168,2048)}",
    "masked": "masked grouped FP8 NT GEMM, (G,cap) in {(1,1024),(2,512),(4,256)} x "
              "(N,K) in {(4096,7168),(7168,2048)}, masked_m ~ U[0,cap]",
    "small": "dense FP8 NT GEMM 128x256x512",
}


def work_of(p):
    from moe_grouped_gemm_lhs_amd import accounting as acc
    if p.kind == "dense":
        return acc.dense_work(p.M, p.N, p.K)
    if p.kind == "contiguous":
        return acc.contiguous_work(p.sizes, p.N, p.K)
    return acc.masked_work(p.masked_m, p.M, p.N, p.K)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU component).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from moe_grouped_gemm_lhs_amd import binding as dg
    from moe_grouped_gemm_lhs_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dg.load_library()

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {n} bytes done", file=sys.stderr, flush=True)
        del src, dst
    if args.workload == "quant":
        return bench_quant(args, torch, np, dg, I, dev)

    names = [args.workload] if args.workload != "all" else ["contiguous", "decode", "prefill",
                                                             "masked"]
    head = names[0]
    results = {}
    for name in names:
        print(f"[bench] workload {name}", file=sys.stderr, flush=True)
        results[name] = measure(name, args, torch, np, dg, I, dev, headline=name == head)
        torch.cuda.empty_cache()
    r = results[head]
    fmt_note = "" if args.formats == "e4m3xe4m3" else f", operands {args.formats}"
    line = {
        "metric": "FP8 TFLOPS and HBM GB/s (as % of MI355X peak) per M,N,K / group shape",
        "value": r["value"], "unit": r["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3" if args.formats == "e4m3xe4m3" else "fp8" + args.formats,
        "data": "synthetic (seeded N(0,1), 1x128 / 128x128 e4m3fn block quantisation)",
        "config": {"workload": WORKLOAD_TEXT[head] + fmt_note, "shapes": r["shapes"],
                   "parallelism": "single GPU", "step": r["step"]},
        "tflops": r["tflops"], "gbs": r["gbs"], "pages_gbs": r["pages_gbs"],
        "roofline": r["roofline"],
        "sclk_mhz": r.get("sclk_mhz"),
        "cpu_baseline": r.get("cpu_baseline"),
        "per_shape": r["per_shape"],
    }
    if len(names) > 1:
        line["workloads"] = {
            n: {k: results[n][k] for k in ("value", "unit", "ms_per_step", "tflops", "gbs",
                                            "pages_gbs", "roofline", "per_shape")}
            | {"workload": WORKLOAD_TEXT[n]}
            for n in names[1:]}
    for key in ("masked_decode_latency_us", "masked_step_latency_us"):
        if key in r:
            line[key] = r[key]
        elif len(names) > 1 and key in results.get("masked", {}):
            line["workloads"]["masked"][key] = results["masked"][key]
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump(dict(line=line, detail={n: results[n]["detail"] for n in names}), f,
                      indent=1)
    print(json.dumps(line), flush=True)


HBM_BOUND = {"decode", "masked", "small"}


def measure(name, args, torch, np, dg, I, dev, headline=False):
    """One workload: its step rate (a HIP graph of all its calls, replayed K times), each
    call's duration (events around eager launches), the dominant call's launch time over
    back-to-back launches, and, for the headline workload, the GPU clock while that call
    runs and the CPU oracle on a sample."""
    cases = workload_cases(name)
    a_fmt, b_fmt = args.formats.split("x")
    if (a_fmt, b_fmt) != ("e4m3", "e4m3"):
        cases = I.with_formats(cases, a_fmt, b_fmt)
    if args.shapes and args.workload != "all":
        keep = [int(v) for v in args.shapes.split(",")]
        cases = [cases[i] for i in keep]

    # ---- inputs: generated on the host, made resident in HBM before timing
    t0 = time.time()
    problems, calls = [], []
    # one workspace, zero filled once, shared by every call in stream order
    ws_need = 0
    for case in cases:
        kind_id = {"dense": 0, "contiguous": 1, "masked": 2}[case["kind"]]
        rows = case.get("M") or case.get("cap") or sum(case.get("sizes", [0]))
        ws_need = max(ws_need, dg.dg_workspace_bytes(kind_id, rows, case["N"], case["K"],
                                                     case.get("G", len(case.get("sizes", [1])))))
    ws = torch.zeros(max(ws_need, 16), dtype=torch.uint8, device=dev)
    for case in cases:
        p = I.make(case)
        fm = dict(a_format=p.a_fmt, b_format=p.b_fmt)
        nkb, nnb = p.K // 128, -(-p.N // 128)
        A = torch.from_numpy(p.A).to(dev)
        sA = torch.from_numpy(p.sA).to(dev)
        B = torch.from_numpy(p.B).to(dev)
        sB = torch.from_numpy(p.sB).to(dev)
        mm = None
        if p.kind == "dense":
            B, sB = B.view(p.N, p.K), sB.view(nnb, nkb)
            C = torch.empty((p.M, p.N), dtype=torch.bfloat16, device=dev)
            ops = [A, sA, B, sB, C]
            def make(A, sA, B, sB, C, fm=fm):
                return lambda: dg.dg_gemm_fp8_nt(A, sA, B, sB, C, workspace=ws, **fm)
        elif p.kind == "contiguous":
            B, sB = B.view(p.G, p.N, p.K), sB.view(p.G, nnb, nkb)
            gi = torch.from_numpy(p.group_idx).to(dev)
            C = torch.empty((p.rows, p.N), dtype=torch.bfloat16, device=dev)
            ops = [A, sA, B, sB, gi, C]
            def make(A, sA, B, sB, gi, C, fm=fm):
                return lambda: dg.dg_grouped_gemm_fp8_contiguous(A, sA, B, sB, gi, C,
                                                                 workspace=ws, **fm)
        else:
            A, sA = A.view(p.G, p.M, p.K), sA.view(p.G, p.M, nkb)
            B, sB = B.view(p.G, p.N, p.K), sB.view(p.G, nnb, nkb)
            mm = torch.from_numpy(p.masked_m).to(dev)
            C = torch.empty((p.G, p.M, p.N), dtype=torch.bfloat16, device=dev)
            ops = [A, sA, B, sB, mm, C]
            def make(A, sA, B, sB, mm, C, fm=fm):
                return lambda: dg.dg_grouped_gemm_fp8_masked(A, sA, B, sB, mm, C,
                                                             workspace=ws, **fm)
        fn = make(*ops)
        # the same call over fresh copies of every operand (for timing without cache reuse)
        clone = (lambda make=make, ops=ops: make(*[t.clone() for t in ops]))
        flops, nbytes = work_of(p)
        kind_id = {"dense": 0, "contiguous": 1, "masked": 2}[p.kind]
        inst = dg.dg_instance_name(kind_id, p.M if p.kind != "contiguous" else p.rows, p.N, p.K, p.G)
        problems.append(p)
        calls.append(dict(name=I.case_name(case), fn=fn, clone=clone, flops=flops,
                          bytes=nbytes, pages=pages_bytes_of(p), instance=inst, masked_m=mm))
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    print(f"[bench] {name}: {len(calls)} shapes resident in HBM ({gen_s:.1f} s to generate)",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        for c in calls:
            c["fn"]()
    torch.cuda.synchronize()

    # ---- the step as one HIP graph (the calls read their routing from device memory and
    # never synchronise, so a captured step replays exactly); eager launches otherwise
    graph = None
    if not args.no_graph:
        try:
            cap = torch.cuda.Stream(dev)
            cap.wait_stream(stream)
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=cap):
                for c in calls:
                    c["fn"]()
            torch.cuda.synchronize()
            for _ in range(max(1, args.warmup)):
                graph.replay()
            torch.cuda.synchronize()
        except Exception as e:  # pragma: no cover - fall back to eager steps
            print(f"[bench] graph capture unavailable ({e}); timing eager steps", file=sys.stderr)
            graph = None

    def one_step():
        if graph is not None:
            graph.replay()
        else:
            for c in calls:
                c["fn"]()

    # ---- timed region 1: K whole steps (the job's throughput)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    wall_s = t_end - t_start
    ms_per_step = wall_s * 1e3 / args.steps

    # ---- timed region 2: K eager steps with HIP events around every launch, recorded on
    # the stream the kernels run on (per-shape durations; the roofline's kernel time)
    # Each step's launches are queued behind a short device-side spin, so that the host
    # runs ahead and the events bracket the kernels alone, not the host's launch latency.
    spin = _spin_cycles_for(torch, stream, 40e-6 * len(calls) + 50e-6)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in calls] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s_ in range(args.steps):
        torch.cuda._sleep(spin)
        for i, c in enumerate(calls):
            ev[s_][i][0].record(stream)
            c["fn"]()
            ev[s_][i][1].record(stream)
    torch.cuda.synchronize()

    per = []
    for i, c in enumerate(calls):
        times = [ev[s_][i][0].elapsed_time(ev[s_][i][1]) for s_ in range(args.steps)]
        us = 1e3 * float(np.mean(times))
        per.append(dict(name=c["name"], instance=c["instance"], us=round(us, 3),
                        us_median=round(1e3 * float(np.median(times)), 3),
                        tflops=round(c["flops"] / us / 1e6, 2),
                        gbs=round(c["bytes"] / us / 1e3, 1)))
    total_flops = sum(c["flops"] for c in calls)
    total_bytes = sum(c["bytes"] for c in calls)
    total_pages = sum(c["pages"] for c in calls)
    step_s = ms_per_step / 1e3
    hbm_bound = name in HBM_BOUND
    if hbm_bound:
        value, unit = total_bytes / step_s / 1e9, "GB/s"
    else:
        value, unit = total_flops / step_s / 1e12, "TFLOP/s"

    # dominant kernel: the shape with the largest share of the step
    dom = max(range(len(calls)), key=lambda i: per[i]["us"])
    d = per[dom]
    # ---- timed region 3: its launch duration without the per-launch event overhead
    launch_us = _batch_launch_us(torch, stream, calls[dom], args.steps, d["us"])
    if hbm_bound:
        achieved = calls[dom]["bytes"] / (launch_us * 1e-6) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=None)
    else:
        achieved = calls[dom]["flops"] / (launch_us * 1e-6) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 1), peak=FP8_PEAK_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / FP8_PEAK_TFLOPS, 4), traffic=None)
    roof["kernel"] = f"{d['instance']} on {d['name']}"
    roof["launch_us"] = round(launch_us, 3)
    roof["launch_us_event_pair"] = d["us"]
    roof["traffic"] = _profiled_traffic(d["instance"], d["name"])

    out = {"value": round(value, 2), "unit": unit, "ms_per_step": round(ms_per_step, 4),
           "shapes": len(calls),
           "step": "one HIP graph of all shapes" if graph is not None else "eager launches",
           "tflops": round(total_flops / step_s / 1e12, 2),
           "gbs": round(total_bytes / step_s / 1e9, 1),
           "pages_gbs": round(total_pages / step_s / 1e9, 1),
           "roofline": roof,
           "per_shape": [[q["name"], q["us"], q["tflops"], q["gbs"]] for q in per],
           "detail": per}
    if name == "masked":
        out["masked_decode_latency_us"] = masked_graph_latency(torch, np, dev, problems, calls,
                                                               args.steps)
        out["masked_step_latency_us"] = masked_step_latency(torch, np, dev, problems, calls,
                                                            args.steps)
    if headline:
        out["sclk_mhz"] = None if args.no_sclk else sclk_while_running(torch, calls[dom], 2.0)
        if not hbm_bound and out["sclk_mhz"]:
            # the same fraction against the MFMA peak at the clock the GPU held meanwhile
            peak_held = FP8_PEAK_TFLOPS * out["sclk_mhz"]["median"] / PEAK_SCLK_MHZ
            roof["frac_at_sclk"] = round(achieved / peak_held, 4)
        if not args.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(problems, calls, args.cpu_budget_s, hbm_bound)
    return out


def pages_bytes_of(p):
    """The pages' GB/s convention for one call: FP8 A and B plus BF16 C, scales ignored,
    every row (every capacity row in the masked layout) counted."""
    from moe_grouped_gemm_lhs_amd import accounting as acc
    if p.kind == "dense":
        return acc.pages_bytes(1, p.M, p.N, p.K)
    if p.kind == "contiguous":
        return acc.pages_bytes(1, p.rows, p.N, p.K) + (p.G - 1) * p.N * p.K
    return acc.pages_bytes(p.G, p.M, p.N, p.K)


def sclk_while_running(torch, call, seconds=2.0):
    """The GPU clock reported by rocm-smi, sampled every ~0.25 s while the call runs back
    to back for about `seconds` (best effort: None when rocm-smi is unavailable)."""
    import re
    import shutil
    import subprocess
    import threading
    smi = shutil.which("rocm-smi")
    if smi is None:
        return None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    call["fn"]()
    e1.record()
    torch.cuda.synchronize()
    n = max(1, int(seconds / max(e0.elapsed_time(e1) * 1e-3, 1e-6)))
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            try:
                out = subprocess.run([smi, "--showclocks", "--json"], capture_output=True,
                                     text=True, timeout=10).stdout
                m = re.search(r'"sclk clock speed:":\s*"\((\d+)Mhz\)"', out)
                if m:
                    samples.append(int(m.group(1)))
            except Exception:
                return
            stop.wait(0.25)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    for _ in range(n):
        call["fn"]()
    torch.cuda.synchronize()
    stop.set()
    th.join(timeout=15)
    if not samples:
        return None
    samples.sort()
    return {"median": samples[len(samples) // 2], "min": samples[0], "max": samples[-1],
            "samples": len(samples),
            "source": "rocm-smi --showclocks while the dominant kernel ran back to back"}


def masked_graph_latency(torch, np, dev, problems, calls, steps):
    """Launch-inclusive latency of one masked call per decode step with fresh counts: each
    step writes new masked_m values (a small device copy from a table of seeded draws)
    and then runs the call, either eagerly or by replaying a HIP graph captured once.
    Per case: [name, eager us/step, graph us/step], wall clock over `steps` steps."""
    out = []
    for p, c in zip(problems, calls):
        mm = c["masked_m"]
        saved = mm.clone()
        draws = np.random.default_rng(p.seed + 1000).integers(0, p.M + 1, (16, p.G))
        table = torch.from_numpy(draws.astype(np.int32)).to(dev)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.graph(graph, stream=side):
            c["fn"]()
        torch.cuda.synchronize()
        res = [c["name"]]
        for use_graph in (False, True):
            for i in range(3):
                mm.copy_(table[i % 16])
                graph.replay() if use_graph else c["fn"]()
            torch.cuda.synchronize()
            t = time.perf_counter()
            for i in range(steps):
                mm.copy_(table[i % 16])
                graph.replay() if use_graph else c["fn"]()
            torch.cuda.synchronize()
            res.append(round((time.perf_counter() - t) * 1e6 / steps, 2))
        mm.copy_(saved)
        out.append(res)
    torch.cuda.synchronize()
    return out


def masked_step_latency(torch, np, dev, problems, calls, steps):
    """A decode step as a serving loop runs it: fresh masked_m for every call of the
    workload (device copies from a table of seeded draws), all the calls, then a host
    synchronisation (the host needs the step's results before the next).  The calls run
    either as eager launches or as one replay of a HIP graph that holds all of them.
    Returns {"eager": us/step, "graph": us/step, "calls": n}, wall clock over `steps`."""
    mms = [c["masked_m"] for c in calls]
    saved = [m.clone() for m in mms]
    tables = [torch.from_numpy(np.random.default_rng(p.seed + 2000).integers(
        0, p.M + 1, (16, p.G)).astype(np.int32)).to(dev) for p in problems]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.graph(graph, stream=side):
        for c in calls:
            c["fn"]()
    torch.cuda.synchronize()
    res = {"calls": len(calls)}
    for use_graph in (False, True):
        def step(i):
            for m, t in zip(mms, tables):
                m.copy_(t[i % 16])
            if use_graph:
                graph.replay()
            else:
                for c in calls:
                    c["fn"]()
            torch.cuda.synchronize()
        for i in range(3):
            step(i)
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        res["graph" if use_graph else "eager"] = round((time.perf_counter() - t0) * 1e6 / steps, 1)
    for m, v in zip(mms, saved):
        m.copy_(v)
    torch.cuda.synchronize()
    return res


def bench_quant(args, torch, np, dg, I, dev):
    """The quantisation workload: each shape one call on a resident bf16 input; value is
    algorithmic bytes (2 read + 1 written per element, plus the fp32 scales) per second."""
    fmt = args.formats.split("x")[0]
    cases = QUANT_CASES
    if args.shapes:
        cases = [cases[int(i)] for i in args.shapes.split(",")]
    calls = []
    for i, (kind, rows, K) in enumerate(cases):
        X = torch.from_numpy(I.normal_matrix(90 + i, 1, rows, K)).to(dev).to(torch.bfloat16)
        Q = torch.empty((rows, K), dtype=torch.uint8, device=dev)
        srows = rows if kind == "1x128" else -(-rows // 128)
        S = torch.empty((srows, K // 128), dtype=torch.float32, device=dev)
        f = dg.dg_quantize_fp8_1x128 if kind == "1x128" else dg.dg_quantize_fp8_128x128
        nbytes = rows * K * 3 + S.numel() * 4
        make = (lambda X, Q, S, f=f: (lambda: f(X, fmt, Q, S)))
        clone = (lambda make=make, X=X, Q=Q, S=S:
                 make(X.clone(), torch.empty_like(Q), torch.empty_like(S)))
        calls.append(dict(name=f"quant_{kind}_{rows}x{K}", fn=make(X, Q, S), clone=clone,
                          bytes=nbytes, instance=f"quant_{kind}", X=X, kind=kind))
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        for c in calls:
            c["fn"]()
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    with torch.cuda.graph(graph, stream=cap):
        for c in calls:
            c["fn"]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / args.steps
    spin = _spin_cycles_for(torch, stream, 40e-6 * len(calls) + 50e-6)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in calls] for _ in range(args.steps)]
    for s_ in range(args.steps):
        torch.cuda._sleep(spin)
        for i, c in enumerate(calls):
            ev[s_][i][0].record(stream)
            c["fn"]()
            ev[s_][i][1].record(stream)
    torch.cuda.synchronize()
    per = []
    for i, c in enumerate(calls):
        us = 1e3 * float(np.mean([ev[s_][i][0].elapsed_time(ev[s_][i][1])
                                  for s_ in range(args.steps)]))
        per.append((c["name"], round(us, 3), round(c["bytes"] / us / 1e3, 1)))
    total = sum(c["bytes"] for c in calls)
    dom = max(range(len(calls)), key=lambda i: per[i][1])
    launch_us = _batch_launch_us(torch, stream, calls[dom], args.steps, per[dom][1])
    achieved = calls[dom]["bytes"] / (launch_us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        # a bounded sample: the leading rows of the first shape, about a second of work
        c = calls[0]
        x = c["X"][:256].cpu().view(torch.int16).numpy().view(np.uint16)
        t = time.perf_counter()
        reps = 0
        while time.perf_counter() - t < max(1.0, min(args.cpu_budget_s, 10.0)):
            oracle.quantize_1x128(x, fmt)
            reps += 1
        dt = time.perf_counter() - t
        cpu = {"value": round(reps * x.size * 3 / dt / 1e9, 4), "unit": "GB/s",
               "cores": oracle.threads(), "kind": "oracle",
               "sample": f"{reps} x 1x128 quantisation of 256x{x.shape[1]} bf16 rows "
                         f"({dt:.1f} s of oracle time)"}
    line = {
        "metric": "FP8 TFLOPS and HBM GB/s (as % of MI355X peak) per M,N,K / group shape",
        "value": round(total / step_s / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"bf16->fp8{fmt}", "data": "synthetic (seeded N(0,1) bf16)",
        "config": {"workload": WORKLOAD_TEXT["quant"], "shapes": len(calls),
                   "parallelism": "single GPU", "step": "one HIP graph of all shapes"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": f"{calls[dom]['instance']} on {calls[dom]['name']}",
                     "launch_us": round(launch_us, 3), "launch_us_event_pair": per[dom][1]},
        "cpu_baseline": cpu,
        "per_shape": [list(x) for x in per],
    }
    print(json.dumps(line), flush=True)


_ROOT = os.path.dirname(os.path.abspath(__file__))
_KERNEL_SOURCES = ["moe_grouped_gemm_lhs_amd/csrc/dg_kernels.hip",
                   "moe_grouped_gemm_lhs_amd/csrc/dg_internal.h",
                   "moe_grouped_gemm_lhs_amd/csrc/dg_host.cpp"]
_TRAFFIC_FILES = {
    ("dense_128x128_stream_4w", "dense_128x7168x16384"):
        "profiles/decode_dense_128x128_stream_4w_hbm_traffic.txt",
    ("dense_256x224", "dense_4096x7168x16384"): "profiles/prefill_dense_256x224_hbm_traffic.txt",
    ("contig_256x256", "contig_8xrand_4096x7168"):
        "profiles/contiguous_contig_256x256_8xrand_hbm_traffic.txt",
    ("contig_256x256", "contig_4x8192_4096x7168"):
        "profiles/contiguous_contig_256x256_4x8192_hbm_traffic.txt",
    ("masked_128x128", "masked_4x256_4096x7168"): "profiles/masked_masked_128x128_hbm_traffic.txt",
}


def _profiled_traffic(instance, shape):
    """HBM bytes per launch of this kernel on this shape from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a copy of known size), or None
    when there is none or the kernel sources changed since it was taken."""
    import hashlib
    rel = _TRAFFIC_FILES.get((instance, shape))
    if rel is None or not os.path.exists(os.path.join(_ROOT, rel)):
        return None
    fields = {}
    for line in open(os.path.join(_ROOT, rel)):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for src in _KERNEL_SOURCES:
        with open(os.path.join(_ROOT, src), "rb") as f:
            h.update(f.read())
    if fields.get("kernel_sources_sha256") != h.hexdigest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


MALL_BYTES = 256 << 20           # MI355X Infinity Cache (memory-side, in front of HBM)


def rotation_copies(nbytes):
    """Operand sets a timed call rotates over: enough that the other sets' bytes between
    two uses of one set exceed twice the Infinity Cache (at most 16 sets)."""
    return min(16, -(-2 * MALL_BYTES // max(nbytes, 1)) + 1)


def _batch_launch_us(torch, stream, call, n, est_us):
    """Mean duration of one launch of a call: n back-to-back launches queued behind a
    device-side spin (so the host's launch latency is hidden), one pair of HIP events
    recorded on the launch stream around all of them; the gaps between consecutive
    launches are included, the per-launch event overhead is not.  The launches rotate
    over copies of the call's operands, enough that twice the Infinity Cache's capacity
    is touched between two reads of the same bytes, so no launch finds its inputs left
    in that cache by an earlier one."""
    r = rotation_copies(call["bytes"])
    fns = [call["fn"]] + [call["clone"]() for _ in range(r - 1)]
    spin = _spin_cycles_for(torch, stream, 1.5 * n * est_us * 1e-6 + 50e-6)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(spin)
    e0.record(stream)
    for i in range(n):
        fns[i % r]()
    e1.record(stream)
    torch.cuda.synchronize()
    del fns
    return 1e3 * e0.elapsed_time(e1) / n


def _spin_cycles_for(torch, stream, seconds):
    """Cycle count for torch.cuda._sleep that keeps the device busy for about `seconds`."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    probe = 1 << 20
    torch.cuda._sleep(probe)            # first call loads the spin kernel
    torch.cuda.synchronize()
    e0.record(stream)
    torch.cuda._sleep(probe)
    e1.record(stream)
    torch.cuda.synchronize()
    per_cycle_s = max(e0.elapsed_time(e1) * 1e-3 / probe, 1e-12)
    return int(min(seconds / per_cycle_s, 1 << 40))


def cpu_baseline(problems, calls, budget_s, hbm_bound, min_s=10.0):
    """Time the CPU oracle on a bounded sample of the workload: whole shapes in order,
    repeated until at least min_s of oracle time has been spent, and the leading rows of
    a shape when a whole one would overrun budget_s; throughput is scaled to the
    metric's unit from the work actually done (a shape's bytes in proportion to the rows
    done, so a partial shape does not count all of B)."""
    import oracle

    done_s, done_flops, done_bytes = 0.0, 0, 0.0
    parts = {}
    passes = 0
    while done_s < min_s and done_s < budget_s:
        passes += 1
        for p, c in zip(problems, calls):
            if done_s >= budget_s:
                break
            if p.kind != "dense":
                rows = p.rows if p.kind == "contiguous" else p.G * p.M
            else:
                rows = p.M
            # estimate from one small slice first: never overrun the budget by much
            r_probe = min(rows, max(1, oracle.threads()))
            t = time.perf_counter()
            _oracle_rows(p, r_probe)
            dt = time.perf_counter() - t
            per_row = dt / r_probe
            r = int(min(rows, max(r_probe, (budget_s - done_s - dt) / max(per_row, 1e-9))))
            if r > r_probe:
                t = time.perf_counter()
                _oracle_rows(p, r)
                dt = time.perf_counter() - t
            else:
                r = r_probe
            done_s += dt
            done_flops += c["flops"] * r // max(rows, 1) if p.kind != "masked" else \
                2 * r * p.N * p.K
            done_bytes += c["bytes"] * r / max(rows, 1)
            parts[c["name"]] = f"{c['name']}:{r}/{rows} rows"
    if hbm_bound:
        value, unit = done_bytes / done_s / 1e9, "GB/s"
    else:
        value, unit = done_flops / done_s / 1e12, "TFLOP/s"
    return {"value": round(value, 5), "unit": unit, "cores": len(os.sched_getaffinity(0)),
            "threads": oracle.threads(), "cpu": _cpu_model(), "kind": "oracle",
            "sample": f"{passes} pass(es) over " + "; ".join(parts.values())
                      + f" ({done_s:.1f} s of oracle time)",
            "tflops": round(done_flops / done_s / 1e12, 5)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_rows(p, r):
    import oracle
    nnb = -(-p.N // 128)
    fm = dict(a_fmt=p.a_fmt, b_fmt=p.b_fmt)
    if p.kind == "dense":
        return oracle.gemm_fp8_nt(p.A[:r], p.sA[:r], p.B, p.sB, **fm)
    if p.kind == "contiguous":
        return oracle.grouped_contiguous(p.A[:r], p.sA[:r], p.B, p.sB, p.group_idx[:r], p.G,
                                         **fm)
    return oracle.gemm_fp8_nt(p.A[:r], p.sA[:r], p.B[:p.N], p.sB[:nnb], **fm)


if __name__ == "__main__":
    main()
