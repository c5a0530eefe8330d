#!/usr/bin/env python3
"""Muon-step benchmark on one MI355X.

A step is one full Muon step (momentum, Newton-Schulz orthogonalisation,
weight update) over every matrix of the workload, one library call per
same-shape group.  The default workload is the Qwen2.5-7B-shaped layer set
(q, o 3584x3584; k, v 3584x512; gate, up, down 3584x18944) with Gram
Newton-Schulz (one restart after iteration 2, T = 5); the standard variant
is timed beside it.  Inputs are seeded and synthetic (synth/inputs.py) and
already resident in HBM when the timed region starts.

Prints one JSON line.  ``value`` is the algorithmic (symmetric-aware)
Newton-Schulz TFLOP/s of the whole step; the roofline block reports the
dominant kernel from HIP events recorded around each launch on the launch
stream; the cpu_baseline block times the fp64 oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_16BIT_TFLOPS = 2516.6  # MI355X dense bf16/fp16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_F32_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
METRIC = "NS orthogonalization TFLOP/s (% bf16 MFMA peak) + Muon steps/s per layer batch"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen2.5-7b")
    ap.add_argument("--variant", default="gram", choices=["gram", "standard"])
    ap.add_argument("--compute", default=None, help="operand type override: bf16, f16 or f32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-variant", action="store_true", help="skip timing the other NS variant")
    ap.add_argument("--no-low-bit", action="store_true",
                    help="skip timing the step with the low-bit (4-bit grid / 8-bit subspace) momentum state")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the compact timing of the other workloads (default run only)")
    ap.add_argument("--no-parity", action="store_true",
                    help="skip the relative error against the fp64 oracle (one matrix per group) and the "
                         "256x512 comparison with the SVD polar factor")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the register-only MFMA ceiling probe (profiling runs)")
    ap.add_argument("--one-stream", action="store_true",
                    help="issue every group on one stream (default: one stream per group)")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("MFMA_DIR", "BENCH_JSON"),
                    help="write the MFMA counter summary (--pmc MfmaUtil MfmaFlopsF16) of every GEMM kernel, "
                         "with the algorithmic FLOPs from the same run's bench.py line, to --out and exit")
    ap.add_argument("--traffic-run", metavar="TRACE_JSON",
                    help="one serial step per group with the library's launch trace on (no timing), the "
                         "trace's per-launch algorithmic bytes written to TRACE_JSON; run under rocprofv3 --pmc "
                         "for --summarize-traffic")
    ap.add_argument("--summarize-traffic", nargs=3, metavar=("READ_DIR", "WRITE_DIR", "TRACE_JSON"),
                    help="HBM-side bytes per kernel from two rocprofv3 --pmc passes over --traffic-run (L2-to-"
                         "memory read requests by size, write requests by size) against the trace's algorithmic "
                         "bytes; writes --out and exits")
    ap.add_argument("--summarize-stats", metavar="STATS_DIR",
                    help="write the rocprofv3 --kernel-trace --stats table to --out and exit")
    ap.add_argument("--out", default=None, help="output file of the --summarize-* modes")
    ap.add_argument("--command", default="", help="the profiled command, recorded by the --summarize-* modes")
    return ap.parse_args()


TRACED_STEPS_MAX = 30  # steps of the serial, per-launch traced pass
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "matrix_orthogonalizing_optimizer_step_amd", "csrc")


def _code_tokens(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed
    (string and character literals kept as written)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest() -> str:
    """sha256 over the code of the HIP sources (comments and layout left out):
    a traffic figure holds only for the code it was taken on."""
    import hashlib

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + _code_tokens(f.read()).encode())
    return h.hexdigest()


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"hbm_traffic_{workload}.txt")


def read_traffic(kernel: str, workload: str):
    """Bytes moved between L2 and memory per launch of `kernel` from the
    committed counter summary, or None when there is none or the sources
    changed since it was taken."""
    path = traffic_file(workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    key = f"traffic_bytes_per_launch[{kernel}]"
    if fields.get("source_sha256") != source_digest() or key not in fields:
        return None
    return float(fields[key])


def _csv_rows(d: str, suffix: str):
    import csv
    import glob

    rows = []
    for path in glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


READ_COUNTERS = ("TCC_EA0_RDREQ", "TCC_EA0_RDREQ_32B", "TCC_EA0_RDREQ_64B", "TCC_EA0_RDREQ_128B")
WRITE_COUNTERS = ("TCC_EA0_WRREQ", "TCC_EA0_WRREQ_64B")


def _short_kernel(name: str) -> str:
    """'void muon::(anonymous namespace)::norm_kernel<1>(muon::NormArgs)' -> 'norm_kernel<1>'."""
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    return name.split("(")[0].split("::")[-1].strip()


def _dispatch_counters(d: str):
    """Per dispatch of the library's kernels (in dispatch order): (short
    kernel name, {counter: value summed over instances})."""
    per = {}
    for r in _csv_rows(d, "counter_collection.csv"):
        if "muon::" not in r["Kernel_Name"]:
            continue
        key = int(r["Dispatch_Id"])
        ent = per.setdefault(key, [_short_kernel(r["Kernel_Name"]), {}])
        ent[1][r["Counter_Name"]] = ent[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def summarize_traffic(args):
    """Bytes moved between the L2 and memory per kernel, from the raw request
    counters: reads = 32 n32 + 64 n64 + 128 n128 (requests by size), writes =
    64 n64 + 32 (n - n64).  The library's launches of --traffic-run are
    matched one by one, in order, with their dispatches, so every kernel's
    counter bytes stand beside the algorithmic bytes of the same launches.
    Writes are attributed to the dispatch during which the write-back L2
    evicts them, so per kernel they are approximate; their sum is not."""
    with open(args.summarize_traffic[2]) as f:
        trace = json.load(f)
    names = {t["kernel"] for t in trace["launches"]}
    n = len(trace["launches"])

    def split(d):
        """The first n dispatches of traced kernels, then every later dispatch
        of the library (the untraced low-bit step)."""
        allx = _dispatch_counters(d)
        matched, i = [], 0
        while i < len(allx) and len(matched) < n:
            if allx[i][0] in names:
                matched.append(allx[i])
            i += 1
        return matched, allx[i:]

    rd, rd_rest = split(args.summarize_traffic[0])
    wr, wr_rest = split(args.summarize_traffic[1])
    if not (len(rd) == len(wr) == n) or [x[0] for x in rd_rest] != [x[0] for x in wr_rest]:
        raise SystemExit(f"dispatch counts differ: read pass {len(rd)}, write pass {len(wr)}, trace {n}")
    tab = {}
    for (kr, cr), (kw, cw), t in zip(rd, wr, trace["launches"]):
        if not (kr == kw == t["kernel"]):
            raise SystemExit(f"dispatch order differs: {kr} / {kw} / {t['kernel']}")
        e = tab.setdefault(kr, dict(n=0, alg=0.0, rd=0.0, wr=0.0, req=0.0, req_split=0.0))
        n32, n64, n128 = (cr.get(c, 0.0) for c in READ_COUNTERS[1:])
        e["n"] += 1
        e["alg"] += t["bytes"]
        e["rd"] += 32 * n32 + 64 * n64 + 128 * n128
        e["req"] += cr.get("TCC_EA0_RDREQ", 0.0)
        e["req_split"] += n32 + n64 + n128
        e["wr"] += 64 * cw.get("TCC_EA0_WRREQ_64B", 0.0) + 32 * (cw.get("TCC_EA0_WRREQ", 0.0) -
                                                                 cw.get("TCC_EA0_WRREQ_64B", 0.0))
    lines = [f"workload: {trace['workload']}",
             f"command: {args.command}",
             f"source_sha256: {source_digest()}",
             "reads = 32 TCC_EA0_RDREQ_32B + 64 TCC_EA0_RDREQ_64B + 128 TCC_EA0_RDREQ_128B; "
             "writes = 64 TCC_EA0_WRREQ_64B + 32 (TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B)",
             "per launch, MB (1e6 bytes); algorithmic = the library's count (operands once, outputs once)",
             f"{'kernel':34s} {'launches':>8s} {'alg_MB':>10s} {'read_MB':>10s} {'write_MB':>10s} "
             f"{'(r+w)/alg':>9s} {'req_by_size/req':>15s}"]
    tot = dict(alg=0.0, rd=0.0, wr=0.0)
    for k in sorted(tab, key=lambda k: -tab[k]["alg"]):
        e = tab[k]
        for x in tot:
            tot[x] += e[x]
        lines.append(f"{k:34s} {e['n']:8d} {e['alg'] / e['n'] / 1e6:10.1f} {e['rd'] / e['n'] / 1e6:10.1f} "
                     f"{e['wr'] / e['n'] / 1e6:10.1f} {(e['rd'] + e['wr']) / e['alg']:9.3f} "
                     f"{e['req_split'] / max(e['req'], 1.0):15.4f}")
        lines.append(f"traffic_bytes_per_launch[{k}]: {(e['rd'] + e['wr']) / e['n']:.0f}")
    lines.append(f"all kernels: algorithmic {tot['alg'] / 1e9:.3f} GB, read {tot['rd'] / 1e9:.3f} GB, "
                 f"write {tot['wr'] / 1e9:.3f} GB")
    if rd_rest:
        lines.append("the step with the low-bit momentum state (k = rank / 16), per kernel: dispatches, read MB "
                     "and write MB per dispatch (no algorithmic count: not traced)")
        other = {}
        for (k, cr), (_, cw) in zip(rd_rest, wr_rest):
            e = other.setdefault(k, [0, 0.0, 0.0])
            e[0] += 1
            e[1] += 32 * cr.get("TCC_EA0_RDREQ_32B", 0.0) + 64 * cr.get("TCC_EA0_RDREQ_64B", 0.0) + \
                128 * cr.get("TCC_EA0_RDREQ_128B", 0.0)
            e[2] += 64 * cw.get("TCC_EA0_WRREQ_64B", 0.0) + 32 * (cw.get("TCC_EA0_WRREQ", 0.0) -
                                                                 cw.get("TCC_EA0_WRREQ_64B", 0.0))
        for k in sorted(other, key=lambda k: -(other[k][1] + other[k][2])):
            c, r_, w_ = other[k]
            lines.append(f"  {k:34s} {c:8d} {r_ / c / 1e6:10.1f} {w_ / c / 1e6:10.1f}")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_stats(args):
    """The rocprofv3 --kernel-trace --stats table, one line per kernel."""
    rows = _csv_rows(args.summarize_stats, "kernel_stats.csv")
    rows.sort(key=lambda r: -float(r["Percentage"]))
    out = [f"command: {args.command}", f"source_sha256: {source_digest()}",
           f"{'kernel':44s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows:
        out.append(f"{_short_kernel(r['Name']):44s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                   f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}")
    with open(args.out, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def summarize_mfma(args):
    """Per GEMM kernel: MFMA FLOPs counted by the hardware (MfmaFlopsF16) and
    the MFMA busy fraction of all SIMDs during the dispatch (MfmaUtil), against
    the algorithmic FLOPs per launch the bench.py line of the same run reports."""
    rows = _csv_rows(args.summarize_mfma[0], "counter_collection.csv")
    with open(args.summarize_mfma[1]) as f:
        line = json.loads(f.read().strip().splitlines()[-1])
    per = {}
    for r in rows:
        name = r["Kernel_Name"]
        if "gemm_nt_mfma" not in name:
            continue
        short = name.replace("void ", "").split("(muon::")[0].replace("muon::", "")
        d = per.setdefault(short, {"MfmaFlopsF16": [], "MfmaUtil": []})
        if r["Counter_Name"] in d:
            dur = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
            d[r["Counter_Name"]].append((float(r["Counter_Value"]), dur))
    out = [f"command: {args.command}", f"source_sha256: {source_digest()}",
           "mfma_busy_pct: MFMA-busy share of all SIMD cycles during the dispatches, weighted by dispatch time",
           "kernel                          dispatches  hw_mfma_gflop  alg_gflop  hw/alg  mfma_busy_pct"]
    for k in sorted(per):
        d = per[k]
        if not d["MfmaFlopsF16"]:
            continue
        hw = sum(v for v, _ in d["MfmaFlopsF16"]) / len(d["MfmaFlopsF16"])
        tot = sum(t for _, t in d["MfmaUtil"])
        util = sum(v * t for v, t in d["MfmaUtil"]) / tot if tot > 0 else float("nan")
        kb = line["kernels"].get(k)
        alg = kb["tflops"] * 1e12 * kb["avg_launch_ms"] / 1e3 if kb and kb["tflops"] else float("nan")
        out.append(f"{k:32s} {len(d['MfmaFlopsF16']):10d} {hw / 1e9:14.1f} {alg / 1e9:10.1f} {hw / alg:7.3f} "
                   f"{util:14.1f}")
    with open(args.out, "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out))


def mfma_ceiling(mu, dev, rounds=12500, reps=3):
    """The 16-bit MFMA rate this device sustains on register operands alone,
    per operand type (muon_mfma_ceiling: two blocks per compute unit, every
    wave issuing MFMAs back to back on hashed data), median of `reps`
    launches of ~15-20 ms after one warm-up launch.  Under a full MFMA load
    the power the data draw sets the clock, so this is what any product of
    that operand type can approach."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = 2 * cus
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    out = {}
    for dt in ("f16", "bf16"):
        mu.mfma_ceiling(blocks, rounds, sink, dt)
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            flops = mu.mfma_ceiling(blocks, rounds, sink, dt)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        tflops = flops / (ms / 1e3) / 1e12
        log(f"[bench] register-only MFMA ceiling ({dt}): {tflops:.0f} TFLOP/s ({ms:.2f} ms per launch)")
        out[dt] = {"tflops": tflops, "frac_of_dense_peak": tflops / PEAK_16BIT_TFLOPS,
                   "implied_clock_ghz": tflops * 1e3 / (cus * 4096.0), "ms_per_launch": ms}
    out["blocks"] = blocks
    out["note"] = ("v_mfma_f32_32x32x16 back to back on register operands with hashed values, no memory traffic; "
                   "the power the operand data draw, not the nominal 2.4 GHz, sets the clock under this load")
    return out


def main():
    args = parse()
    if args.summarize_mfma:
        summarize_mfma(args)
        return
    if args.summarize_traffic:
        summarize_traffic(args)
        return
    if args.summarize_stats:
        summarize_stats(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the step shards by "
              "matrix ownership across GPUs, which this build does not run)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import matrix_orthogonalizing_optimizer_step_amd as mu
    from synth import inputs as syn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = syn.WORKLOADS[args.workload]
    log(f"[bench] workload {wl.key}: {wl.matrices} matrices, {wl.elements / 1e6:.1f}M elements")

    # ---------------------------------------------------------------- inputs
    groups = []
    for gi, g in enumerate(wl.groups):
        Ws, Ms, Gs = syn.group_inputs(wl, gi)
        groups.append(dict(g=g, W=[w.to(dev) for w in Ws], M=[m.to(dev) for m in Ms], G=[x.to(dev) for x in Gs]))
        log(f"[bench] group {g.name}: {g.count} x {g.rows}x{g.cols} uploaded")
    torch.cuda.synchronize()

    def cfg_for(variant):
        return mu.NSConfig(compute=args.compute)

    def flops_for(variant, symmetric_aware=True):
        return sum(x["g"].count * mu.ns_flops(x["g"].rows, x["g"].cols, variant, cfg_for(variant), symmetric_aware)
                   for x in groups)

    # The groups are independent: each gets its own stream (default priority)
    # and workspace so their launches overlap; the step ends when all are done.
    main = torch.cuda.current_stream()
    total_ws = 0
    for x in groups:
        nb = max(mu.workspace_size(x["g"].count, x["g"].rows, x["g"].cols, v, cfg_for(v)) for v in ("gram", "standard"))
        x["ws"] = torch.empty(nb, dtype=torch.uint8, device=dev)
        x["stream"] = main if args.one_stream else torch.cuda.Stream(device=dev)
        total_ws += nb
    if args.one_stream:
        shared = max(groups, key=lambda x: x["ws"].numel())["ws"]
        for x in groups:
            x["ws"] = shared
    log(f"[bench] workspace {total_ws / 2**30:.2f} GiB, {'one stream' if args.one_stream else 'one stream per group'}")

    def step(variant, serial=False, orth_only=False, base=None):
        main = base or torch.cuda.current_stream()
        serial = serial or args.one_stream
        if not serial:
            ev = torch.cuda.Event()
            ev.record(main)
        for x in groups:
            if not serial:
                x["stream"].wait_event(ev)
            s = main if serial else x["stream"]
            if orth_only:  # the orthogonalisation alone, M -> O
                f = mu.gram_ns_orthogonalize if variant == "gram" else mu.ns_orthogonalize
                f(x["M"], x["O"], cfg_for(variant), workspace=x["ws"], stream=s)
            else:
                mu.muon_step(x["W"], x["M"], x["G"], 0.95, 0.02, 0.0, variant, cfg_for(variant), workspace=x["ws"],
                             stream=s)
        if not serial:
            for x in groups:
                done = torch.cuda.Event()
                done.record(x["stream"])
                main.wait_event(done)

    def timed(variant, steps, warmup, orth_only=False):
        """Mean seconds per step over `steps` (host clock, synchronised on both
        sides) and the per-step durations from events on the main stream."""
        for _ in range(warmup):
            step(variant, orth_only=orth_only)
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t0 = time.perf_counter()
        evs[0].record(main)
        for i in range(steps):
            step(variant, orth_only=orth_only)
            evs[i + 1].record(main)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
        return sec, per

    def timed_graph(variant, steps):
        """Capture one step (every group's stream joined into the capture) in a
        HIP graph and time `steps` replays."""
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # warm-up off the capture: caches the pointer arrays
            step(variant, base=side)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(variant, base=torch.cuda.current_stream())
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        del g
        return sec

    def summary(variant, sec):
        alg = flops_for(variant, True)
        dense = flops_for(variant, False)
        return {
            "ms_per_step": sec * 1e3,
            "tflops_algorithmic": alg / sec / 1e12,
            "pct_of_16bit_peak": 100.0 * alg / sec / 1e12 / PEAK_16BIT_TFLOPS,
            "tflops_dense_equivalent": dense / sec / 1e12,
            "steps_per_s": 1.0 / sec,
            "matrices_per_s": wl.matrices / sec,
            "algorithmic_flops_per_step": alg,
        }

    if args.traffic_run:  # one serial step, traced, for the counter passes
        mu.trace_enable(True)
        step(args.variant, serial=True)
        torch.cuda.synchronize()
        recs = mu.trace_collect()
        mu.trace_enable(False)
        with open(args.traffic_run, "w") as f:
            json.dump({"workload": wl.key, "variant": args.variant,
                       "launches": [{"kernel": r["kernel"], "role": r["role"], "bytes": r["bytes"]} for r in recs]},
                      f)
        log(f"[bench] traffic run: {len(recs)} launches traced to {args.traffic_run}")
        if not args.no_low_bit:  # then the step with the low-bit state (k = rank / 16), untraced
            for gi, x in enumerate(groups):
                g = x["g"]
                k = max(1, min(g.rows, g.cols) // 16)
                R0 = [syn.random_matrix(100 + gi * 64 + i, g.cols, k).to(dev) for i in range(g.count)]
                st = mu.GraspState(g.count, g.rows, g.cols, k, dev, R_init=R0)
                gws = torch.empty(mu.grasp_workspace_size(g.count, g.rows, g.cols, k, args.variant, cfg_for(args.variant)),
                                  dtype=torch.uint8, device=dev)
                torch.cuda.synchronize()
                mu.grasp_step(x["W"], st, x["G"], 0.95, 0.02, 0.0, args.variant, cfg_for(args.variant), workspace=gws)
                torch.cuda.synchronize()
                del st, gws
            log("[bench] traffic run: low-bit state step done")
        return

    results = {}
    variants = [args.variant] + ([] if args.no_other_variant else [v for v in ("gram", "standard") if v != args.variant])
    for x in groups:  # outputs of the orthogonalisation-alone timing
        x["O"] = [torch.empty(x["g"].rows, x["g"].cols, dtype=torch.float32, device=dev) for _ in range(x["g"].count)]
    for v in variants:
        sec, per = timed(v, args.steps, args.warmup)
        results[v] = summary(v, sec)
        results[v]["ms_per_step_p10_p50_p90"] = [float(np.percentile(per, q)) for q in (10, 50, 90)]
        osec, _ = timed(v, args.steps, args.warmup, orth_only=True)
        results[v]["orthogonalization_only"] = {
            "ms_per_step": osec * 1e3, "tflops_algorithmic": flops_for(v, True) / osec / 1e12,
            "note": "ns_orthogonalize / gram_ns_orthogonalize of every group's momentum (no momentum update, "
                    "no weight update)"}
        log(f"[bench] {v}: {sec * 1e3:.3f} ms/step, {results[v]['tflops_algorithmic']:.1f} TFLOP/s; "
            f"orthogonalisation alone {osec * 1e3:.3f} ms")
        if args.graph:
            gsec = timed_graph(v, args.steps)
            results[v]["hip_graph"] = {"ms_per_step": gsec * 1e3, "tflops_algorithmic": flops_for(v, True) / gsec / 1e12,
                                       "note": "the whole step captured once (all streams) and replayed"}
            log(f"[bench] {v}: HIP graph replay {gsec * 1e3:.3f} ms/step")

    # ------------------------------------------------ per-kernel durations (HIP events)
    # The traced steps run the groups back to back on one stream so that each
    # launch's event pair measures that kernel alone on the GPU.
    traced_steps = min(args.steps, TRACED_STEPS_MAX)
    mu.trace_enable(True)
    t0 = time.perf_counter()
    for _ in range(traced_steps):
        step(args.variant, serial=True)
    torch.cuda.synchronize()
    traced_sec = (time.perf_counter() - t0) / traced_steps
    recs = mu.trace_collect()
    mu.trace_enable(False)
    kern = {}
    for r in recs:
        k = kern.setdefault(r["kernel"], dict(ms=0.0, flops=0.0, bytes=0.0, launches=0))
        k["ms"] += r["ms"]
        k["flops"] += r["flops"]
        k["bytes"] += r["bytes"]
        k["launches"] += 1
    roles = {}
    for r in recs:
        key = f'{r["kernel"]}:{r["role"]}'
        k = roles.setdefault(key, dict(ms=0.0, flops=0.0, launches=0))
        k["ms"] += r["ms"] / traced_steps
        k["flops"] += r["flops"] / traced_steps
        k["launches"] += 1
    dom_name, dom = max(kern.items(), key=lambda kv: kv[1]["ms"])
    avg_ms = dom["ms"] / dom["launches"]
    is_mfma = dom["flops"] > 0
    if is_mfma:
        achieved = dom["flops"] / (dom["ms"] / 1e3) / 1e12
        peak = PEAK_F32_TFLOPS if dom_name.endswith("f64acc") else PEAK_16BIT_TFLOPS
        roofline = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                    "traffic": read_traffic(dom_name, wl.key), "kernel": dom_name,
                    "launches_per_step": dom["launches"] // traced_steps,
                    "avg_launch_ms": avg_ms, "flops_per_launch": dom["flops"] / dom["launches"],
                    "algorithmic_bytes_per_launch": dom["bytes"] / dom["launches"]}
    else:
        achieved = dom["bytes"] / (dom["ms"] / 1e3) / 1e9
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS, "traffic": read_traffic(dom_name, wl.key), "kernel": dom_name,
                    "avg_launch_ms": avg_ms}
    kernels = {k: {"ms_per_step": v["ms"] / traced_steps, "launches_per_step": v["launches"] // traced_steps,
                   "avg_launch_ms": v["ms"] / v["launches"],
                   "tflops": v["flops"] / (v["ms"] / 1e3) / 1e12 if v["flops"] else None,
                   "gbs": v["bytes"] / (v["ms"] / 1e3) / 1e9} for k, v in kern.items()}
    role_tab = {k: {"ms_per_step": v["ms"], "tflops": v["flops"] / (v["ms"] / 1e3) / 1e12 if v["flops"] else None}
                for k, v in sorted(roles.items(), key=lambda kv: -kv[1]["ms"])}

    ceiling = None if args.no_ceiling else mfma_ceiling(mu, dev)
    if ceiling is not None and is_mfma and not dom_name.endswith("f64acc"):
        # gemm_nt_mfma<OP, ...>: OP 1 = bf16 operands, 2 = fp16
        dom_dt = "bf16" if dom_name.startswith("gemm_nt_mfma<1") else "f16"
        roofline["practical_ceiling_tflops"] = ceiling[dom_dt]["tflops"]
        roofline["practical_ceiling_dtype"] = dom_dt
        roofline["frac_of_practical_ceiling"] = achieved / ceiling[dom_dt]["tflops"]
    for name, v in results.items():
        dt = args.compute if args.compute in ("f16", "bf16") else ("f16" if name == "gram" else "bf16")
        if ceiling is not None and dt in ceiling:
            v["frac_of_practical_ceiling"] = v["tflops_algorithmic"] / ceiling[dt]["tflops"]

    low_bit = None if args.no_low_bit else time_low_bit_state(args, groups, wl, mu, syn, cfg_for, flops_for, dev)

    # ------------------------------------------------ precision against the fp64 oracle
    parity = None
    if not args.no_parity:
        parity = {"groups": group_parity(wl, variants, cfg_for, mu, syn, dev),
                  "single_256x512_vs_svd_polar": polar_distance(mu, syn, dev)}

    # ------------------------------------------------ the other workloads (compact)
    others = None
    if not args.no_other_workloads and args.workload == "qwen2.5-7b" and not args.one_stream:
        for x in groups:  # free the headline workload's buffers first
            for key in ("W", "M", "G", "O", "ws"):
                x.pop(key, None)
        torch.cuda.empty_cache()
        others = {k: time_workload(syn.WORKLOADS[k], mu, syn, dev) for k in OTHER_WORKLOADS}

    # ------------------------------------------------ CPU baseline: the fp64 oracle
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.variant, mu, syn)

    primary = results[args.variant]
    compute = args.compute or ("f16" if args.variant == "gram" else "bf16")
    out = {
        "metric": METRIC,
        "value": primary["tflops_algorithmic"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": primary["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": compute,
        "data": "synthetic",
        "config": {
            "workload": f"{wl.key} layer set: " + "; ".join(f"{g.count} x {g.rows}x{g.cols}" for g in wl.groups),
            "variant": args.variant, "T": 5,
            "restart_after_iteration": 2 if args.variant == "gram" else None,
            "matrices": wl.matrices, "w_dtype": wl.w_dtype, "state_dtype": wl.state_dtype,
            "value_counts": "symmetric-aware Newton-Schulz FLOPs of the whole step / step time",
            "streams": 1 if args.one_stream else len(groups),
        },
        "pct_of_16bit_peak": primary["pct_of_16bit_peak"],
        "steps_per_s": primary["steps_per_s"],
        "matrices_per_s": primary["matrices_per_s"],
        "variants": results,
        "roofline": roofline,
        "mfma_ceiling": ceiling,
        "kernels": kernels,
        "roles": role_tab,
        "traced_ms_per_step": traced_sec * 1e3,
        "traced_steps": traced_steps,
        "traced_note": "traced steps run the groups serially on one stream (per-kernel event timing)",
        "cpu_baseline": cpu,
        "parity_vs_oracle": parity,
        "other_workloads": others,
        "low_bit_state": low_bit,
        "pages_context": {
            "gram_ns_optimizer_time_saving": "up to 50% (Kimi K2, hardware not stated)",
            "ns_runtime_reduction": "40-50% (Kimi K2, hardware not stated)",
            "optimizer_share_of_step": "about 1-3% (distributed Muon, BF16, hardware not stated)",
        },
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(out), flush=True)


def time_low_bit_state(args, groups, wl, mu, syn, cfg_for, flops_for, dev):
    """The same step with the momentum kept in the low-bit state
    (muon_grasp_step): k = 0 (4-bit grid code of M_t, no subspace) and k =
    min(rows, cols) / 16 (8-bit top subspace from one warm-started power
    iteration, 4-bit grid residual).  Each group on its own stream as in the
    main step; then one traced serial pass for the per-kernel times of the
    state kernels."""
    import torch
    variant = args.variant
    main = torch.cuda.current_stream()
    out = {}
    for label in ("k0", "rank_over_16", "rank_over_16_aux_stream"):
        aux = label.endswith("aux_stream")
        for gi, x in enumerate(groups):
            g = x["g"]
            k = 0 if label == "k0" else max(1, min(g.rows, g.cols) // 16)
            x["aux"] = torch.cuda.Stream(device=dev) if aux else None
            R0 = [syn.random_matrix(100 + gi * 64 + i, g.cols, k).to(dev) for i in range(g.count)] if k else None
            x["gs"] = mu.GraspState(g.count, g.rows, g.cols, k, dev, R_init=R0)
            x["gws"] = torch.empty(mu.grasp_workspace_size(g.count, g.rows, g.cols, k, variant, cfg_for(variant)),
                                   dtype=torch.uint8, device=dev)

        def gstep(serial=False):
            serial = serial or args.one_stream
            if not serial:
                ev = torch.cuda.Event()
                ev.record(main)
            for x in groups:
                if not serial:
                    x["stream"].wait_event(ev)
                mu.grasp_step(x["W"], x["gs"], x["G"], 0.95, 0.02, 0.0, variant, cfg_for(variant),
                              workspace=x["gws"], stream=main if serial else x["stream"],
                              aux_stream=None if serial else x["aux"])
            if not serial:
                for x in groups:
                    done = torch.cuda.Event()
                    done.record(x["stream"])
                    main.wait_event(done)

        for _ in range(args.warmup):
            gstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            gstep()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / args.steps
        mu.trace_enable(True)
        gstep(serial=True)
        torch.cuda.synchronize()
        recs = mu.trace_collect()
        mu.trace_enable(False)
        kern = {}
        for r in recs:
            kk = kern.setdefault(r["role"], dict(ms=0.0, flops=0.0, bytes=0.0))
            kk["ms"] += r["ms"]
            kk["flops"] += r["flops"]
            kk["bytes"] += r["bytes"]
        state_roles = {k: {"ms": v["ms"],
                           "tflops": v["flops"] / (v["ms"] / 1e3) / 1e12 if v["flops"] else None,
                           "gbs": v["bytes"] / (v["ms"] / 1e3) / 1e9}
                       for k, v in kern.items() if k.startswith("grasp") or k.startswith("grid")}
        out[label] = {
            "ms_per_step": sec * 1e3,
            "ns_tflops_algorithmic": flops_for(variant, True) / sec / 1e12,
            "k": {x["g"].name: x["gs"].k for x in groups},
            "state_bytes": sum(sum(t.numel() * t.element_size() for name in
                                   ("res_codes", "res_row_scales", "res_col_scales", "P_codes", "P_scales", "R_codes",
                                    "R_scales") for t in (getattr(x["gs"], name) or [])) for x in groups),
            "serial_state_kernels": state_roles,
            "serial_state_ms": sum(v["ms"] for v in state_roles.values()),
        }
        log(f"[bench] low-bit state {label}: {sec * 1e3:.3f} ms/step, state kernels (serial) "
            f"{out[label]['serial_state_ms']:.3f} ms")
        for x in groups:
            del x["gs"], x["gws"]
    out["note"] = ("muon_grasp_step on the same workload and variant; M_t is rebuilt from the stored state, "
                   "orthogonalised, and stored again; state_bytes counts codes and scales (fp32 momentum: "
                   f"{4 * wl.elements} bytes); *_aux_stream: the state update of each group on a second stream "
                   "beside its Newton-Schulz (the serial per-kernel pass uses one stream)")
    return out


OTHER_WORKLOADS = ("llama-130m", "llama-1.1b", "moe-64x")
OTHER_WARMUP, OTHER_STEPS = 2, 5


def time_workload(wl, mu, syn, dev):
    """Gram and standard NS steps per second on another workload, compact:
    each group holds one seeded matrix (W, M, G) replicated over its count
    (MFMA timing does not depend on the values), one stream and workspace per
    group as in the headline step, 2 warm-up and 5 timed steps."""
    import torch
    log(f"[bench] workload {wl.key}: {wl.matrices} matrices")
    groups = []
    for gi, g in enumerate(wl.groups):
        Ws, Ms, Gs = syn.group_inputs(wl, gi, count=1)
        rep = lambda t: [t.to(dev) for _ in range(g.count)]  # noqa: E731
        nb = max(mu.workspace_size(g.count, g.rows, g.cols, v) for v in ("gram", "standard"))
        groups.append(dict(g=g, W=rep(Ws[0]), M=rep(Ms[0]), G=rep(Gs[0]), stream=torch.cuda.Stream(device=dev),
                           ws=torch.empty(nb, dtype=torch.uint8, device=dev)))
    torch.cuda.synchronize()
    main = torch.cuda.current_stream()

    def step(variant):
        ev = torch.cuda.Event()
        ev.record(main)
        for x in groups:
            x["stream"].wait_event(ev)
            mu.muon_step(x["W"], x["M"], x["G"], 0.95, 0.02, 0.0, variant, None, workspace=x["ws"], stream=x["stream"])
        for x in groups:
            done = torch.cuda.Event()
            done.record(x["stream"])
            main.wait_event(done)

    out = {"matrices": wl.matrices,
           "groups": "; ".join(f"{g.count} x {g.rows}x{g.cols}" for g in wl.groups)}
    for variant in ("gram", "standard"):
        for _ in range(OTHER_WARMUP):
            step(variant)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(OTHER_STEPS):
            step(variant)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / OTHER_STEPS
        alg = sum(g.count * mu.ns_flops(g.rows, g.cols, variant, None, True) for g in wl.groups)
        out[variant] = {"ms_per_step": sec * 1e3, "tflops_algorithmic": alg / sec / 1e12,
                        "pct_of_16bit_peak": 100.0 * alg / sec / 1e12 / PEAK_16BIT_TFLOPS,
                        "matrices_per_s": wl.matrices / sec, "steps_per_s": 1.0 / sec}
        log(f"[bench]   {variant}: {sec * 1e3:.2f} ms/step, {alg / sec / 1e12:.0f} TFLOP/s")
    del groups
    torch.cuda.empty_cache()
    out["note"] = (f"{OTHER_WARMUP} warm-up and {OTHER_STEPS} timed steps; one seeded matrix per group replicated "
                   "over the group (values do not change MFMA timing)")
    return out


def group_parity(wl, variants, cfg_for, mu, syn, dev):
    """One Muon step on the first matrix of each group (its own seeded
    inputs, a batch of one) against the fp64 oracle: the relative Frobenius
    error of O and whether the stored momentum is bit for bit the oracle's."""
    import numpy as np
    import torch

    from oracle import muon_oracle as orc
    out = {}
    for gi, g in enumerate(wl.groups):
        Ws, Ms, Gs = syn.group_inputs(wl, gi, count=1)
        for v in variants:
            W, M = [Ws[0].to(dev)], [Ms[0].to(dev)]
            O = [torch.empty(g.rows, g.cols, dtype=torch.float32, device=dev)]
            mu.muon_step(W, M, [Gs[0].to(dev)], 0.95, 0.02, 0.0, v, cfg_for(v), O_out=O)
            torch.cuda.synchronize()
            _, Mr, Or = orc.muon_step(syn.to_f64(Ws[0]), syn.to_f64(Ms[0]), syn.to_f64(Gs[0]),
                                      float(np.float32(0.95)), float(np.float32(0.02)), 0.0, v,
                                      state_dtype=wl.state_dtype, w_dtype=wl.w_dtype)
            out[f"{g.name} {g.rows}x{g.cols} {v}"] = {
                "relF_O": float(orc.relative_frobenius(syn.to_f64(O[0]), Or)),
                "momentum_bit_exact": bool(np.array_equal(syn.to_f64(M[0]), Mr))}
    log("[bench] parity: " + ", ".join(f"{k} {v['relF_O']:.2e}" for k, v in out.items()))
    return out


def polar_distance(mu, syn, dev):
    """The 256x512 fp32 configuration (one step, standard NS, T = 5): the
    distance of O from the polar factor U V^T of the stored momentum (fp64
    SVD), beside its exact value sqrt(sum (p_5(x_i) - 1)^2 / n) for the fixed
    quintic p (x_i = sigma_i / (||M|| + eps)) and O's error against the
    oracle.  Newton-Schulz at T = 5 is not the polar factor; the first
    number must match the second up to O's own error."""
    import numpy as np
    import torch

    from oracle import muon_oracle as orc
    wl = syn.WORKLOADS["single-256x512"]
    W0, M0, G0 = syn.matrix_inputs(wl, 0, 256, 512)
    mu32, lr32 = float(np.float32(0.95)), float(np.float32(0.02))
    _, Mr, Or = orc.muon_step(syn.to_f64(W0), syn.to_f64(M0), syn.to_f64(G0), mu32, lr32, 0.0, "standard",
                              state_dtype="f32", w_dtype="f64")
    U, sv, Vt = np.linalg.svd(Mr, full_matrices=False)
    polar = U @ Vt
    x = sv / (np.linalg.norm(Mr) + orc.EPS)
    for _ in range(5):
        a, b, c = orc.QUINTIC
        x = a * x + b * x ** 3 + c * x ** 5
    exact = float(np.sqrt(np.sum((x - 1.0) ** 2) / x.size))
    out = {"exact_distance_of_ns_from_polar": exact,
           "oracle_distance_from_polar": float(orc.relative_frobenius(Or, polar))}
    for compute in ("f32", "bf16"):
        W, M = [W0.to(dev)], [M0.to(dev)]
        O = [torch.empty(256, 512, dtype=torch.float32, device=dev)]
        mu.muon_step(W, M, [G0.to(dev)], 0.95, 0.02, 0.0, "standard", mu.NSConfig(compute=compute), O_out=O)
        torch.cuda.synchronize()
        Og = syn.to_f64(O[0])
        out[compute] = {"distance_from_polar": float(orc.relative_frobenius(Og, polar)),
                        "relF_vs_oracle": float(orc.relative_frobenius(Og, Or))}
    log(f"[bench] 256x512 vs SVD polar: exact {exact:.4f}, f32 {out['f32']['distance_from_polar']:.4f}, "
        f"bf16 {out['bf16']['distance_from_polar']:.4f}")
    return out


CPU_SAMPLE_SECONDS = 10.0


def cpu_baseline(wl, variant, mu, syn):
    """Time the fp64 oracle on one matrix per group (the first matrix of each)."""
    import numpy as np

    from oracle import muon_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    inputs = []
    for gi, g in enumerate(wl.groups):
        Ws, Ms, Gs = syn.group_inputs(wl, gi, count=1)
        inputs.append((g, [syn.to_f64(x[0]) for x in (Ws, Ms, Gs)]))
    flops, passes = 0.0, 0
    t0 = time.perf_counter()
    # whole passes over the sample until about 10 s of CPU work (at most 4)
    while passes < 4 and (passes == 0 or time.perf_counter() - t0 < CPU_SAMPLE_SECONDS):
        for g, (W, M, G) in inputs:
            orc.muon_step(W, M, G, float(np.float32(0.95)), float(np.float32(0.02)), 0.0, variant,
                          state_dtype=wl.state_dtype, w_dtype=wl.w_dtype)
            flops += mu.ns_flops(g.rows, g.cols, variant, mu.NSConfig(), True)
        passes += 1
    sec = time.perf_counter() - t0
    names = [f"{g.rows}x{g.cols}" for g, _ in inputs]
    log(f"[bench] cpu oracle: {sec:.1f} s for {passes} pass(es) over {len(names)} matrices")
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} pass(es) of one Muon step ({variant} NS, fp64 numpy) on one matrix of each group: "
                      + ", ".join(names),
            "seconds": sec, "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "single_thread": single_thread_oracle(mu, syn)}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def single_thread_oracle(mu, syn):
    """The oracle's standard-NS step on one 256x512 fp32 matrix with one BLAS
    thread (whole passes, about one second)."""
    import numpy as np

    from oracle import muon_oracle as orc
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        return None
    rows, cols = 256, 512
    W, M, G = (syn.to_f64(syn.random_matrix(90 + i, rows, cols)) for i in range(3))
    flops, passes = mu.ns_flops(rows, cols, "standard", mu.NSConfig(), True), 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        while passes == 0 or (passes < 50 and time.perf_counter() - t0 < 1.0):
            orc.muon_step(W, M, G, float(np.float32(0.95)), float(np.float32(0.02)), 0.0, "standard",
                          state_dtype="f32", w_dtype="f32")
            passes += 1
        sec = time.perf_counter() - t0
    return {"value": flops * passes / sec / 1e12, "unit": "TFLOP/s", "cores": 1,
            "sample": f"{passes} pass(es) of one Muon step (standard NS, fp64 numpy) on one 256x512 matrix"}


if __name__ == "__main__":
    main()
