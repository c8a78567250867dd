#!/usr/bin/env python3
"""MoE layer forward + backward throughput on one MI355X.

One step is the whole hot path over one batch: router logits (linear-router
workloads), top-k routing with device-built metadata, row-wise dispatch, the
grouped SwiGLU expert FFN forward, the weighted combine, and all their
backward passes.  Inputs are seeded synthetic tensors already resident in HBM
when the timed region starts.  Default workload: the largest, T=16384 tokens,
d=4096, E=128 experts, top-4, expert hidden 1536, with MXFP8 expert GEMMs (the
expert weights quantised to MXFP8 inside every step).

Prints one JSON line.  `value` and `ms_per_step` come from K timed steps as a
user runs them, each bracketed by its own event pair (`step_ms`: median, min,
max); the per-kernel times (roofline) come from HIP events the library records
around each of its launches over a second pass of the same K steps (the events
cost a few percent of a step, so they stay out of the first pass).  With the
default workload the same line also carries the same shapes and the same bf16
tensors run with BF16 expert GEMMs (`bf16_same_tensors`, and the MXFP8 / BF16
rate ratio) and the bf16 E=128 workload at d=2048, f=1024 (`bf16_e128`).  The
CPU baseline is the fp64 oracle timed on a bounded token sample of the
headline workload; `cpu_c1_single_core` is the oracle on the tiny fp32 workload
on one thread (median of 10 runs).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

METRIC = "MoE layer fwd+bwd tokens/s and grouped-GEMM TFLOP/s (% of MFMA peak), 1 GPU"
PEAK = {"bf16": 2.5e15, "mxfp8": 5.0e15, "f32": 157.3e12}   # dense MFMA, FLOP/s
HBM_PEAK = 8.0e12                                            # bytes/s


ROOT = os.path.dirname(os.path.abspath(__file__))


def source_digest() -> str:
    """sha256 prefix of the library's HIP sources and C header."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_17_amd", "csrc")
    for f in sorted(x for x in os.listdir(csrc) if x.endswith((".hip", ".hpp"))):
        h.update(f.encode())
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(ROOT, "include", "moe.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def counted_traffic(tag: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary
    (already scaled by the copy calibration), or None when there is no summary for this workload or
    the library sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{tag}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        txt = fh.read()
    m = re.search(r"^source-digest: (\w+)", txt, re.M)
    if not m or m.group(1) != source_digest():
        return None
    for line in txt.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 7 and (cells[0] == kernel or cells[0].startswith(kernel + " ")):
            return float(cells[6]) * 1e6
    return None


def kernel_work(name: str, w, s: int) -> tuple[str, float]:
    """Algorithmic work of one launch: ('mfma', flops) or ('hbm', bytes)."""
    T, d, E, k, f, R = w.T, w.d, w.E, w.k, w.f, w.R
    g = name.split("_")[0]
    flops = {"G1": 4 * R * d * f, "G2": 2 * R * f * d, "G3": 2 * R * d * f, "G4": 2 * R * f * d,
             "G5": 4 * R * f * d, "G6": 4 * R * d * f}
    if g in flops:
        return "mfma", float(flops[g])
    hbm = {
        "dispatch": T * d * s + R * d * s + 4 * R,
        "combine": R * d * s + T * d * s + 8 * R,
        "combine_bwd": T * d * s + 2 * R * d * s + 12 * R,
        "dispatch_bwd": R * d * s + T * d * s + 4 * R,
        "route_select": 4 * T * E + 12 * R,
        "route_topk_bwd": 8 * R + 4 * T * E + 4 * R,
    }
    o = 1 + 1 / 32                              # bytes per MX element: E4M3 code + 1/32 of an E8M0 scale
    rp = 128 * (-(-(-(-R // 32) + E) // 4) + 1)  # padded token axis of the token-axis MX layout
    if w.prec == "mxfp8":
        # the combine backward computes only dgates; X and dY go to their MX layouts through mx_gather
        hbm["combine_bwd"] = T * d * s + R * d * s + 12 * R
        # mx_gather, 4 launches, per-launch average: X and dY = gate x dout [R, d], every expert row read from its
        # token row (plus the permutation, and the gates for dY); dHg and dHu [R, f] read in place; each written
        # in the rows layout and in the token-axis layout
        hbm["mx_gather"] = (2 * (R * d * s + (R + rp) * d * o) + 12 * R + 2 * (R * f * s + (R + rp) * f * o)) / 4
    if name in hbm:
        return "hbm", float(hbm[name])
    if name == "mx_quantize_rows":
        # A [R, f] along f (for G2); per element the source (s bytes) is read and 1 + 1/32 bytes written
        return "hbm", float(R * f * (s + o))
    if name == "mx_quantize_cols":
        # A [R, f] down the tokens of each expert segment, transposed into the padded token axis (for G4)
        return "hbm", float(R * f * s + rp * f * o)
    if name == "mx_quantize_both":
        # one expert weight [E, d, f] per launch (3 per step): read once, written in both layouts
        return "hbm", float(E * d * f * (s + 2 * (1 + 1 / 32)))
    return "other", 0.0


def gemm_bytes(name: str, w, active: int) -> float:
    """Algorithmic HBM bytes of one grouped-GEMM launch: every operand read once and every output written once.
    Operands are bf16 (2 bytes), or for the MXFP8 GEMMs their E4M3 codes plus one E8M0 byte per 32; the saved
    bf16 Hg, Hu read by G3's SwiGLU backward and every output are bf16.  Row-grouped GEMMs read the weights of the
    `active` experts (those with rows); the weight gradients write all E experts' dW."""
    T, d, E, k, f, R = w.T, w.d, w.E, w.k, w.f, w.R
    o = (1 + 1 / 32) if w.prec == "mxfp8" else (4 if w.storage == "f32" else 2)
    b = 4 if w.storage == "f32" else 2
    g = name.split("_")[0]
    return float({
        "G1": R * d * o + 2 * active * d * f * o + 3 * R * f * b,
        "G2": R * f * o + active * f * d * o + R * d * b,
        "G3": R * d * o + active * f * d * o + 2 * R * f * b + 2 * R * f * b,
        "G4": R * f * o + R * d * o + E * f * d * b,
        "G5": 2 * R * f * o + 2 * active * d * f * o + R * d * b,
        "G6": R * d * o + 2 * R * f * o + 2 * E * d * f * b,
    }[g])


def cpu_baseline(w, inp, target_s: float) -> dict:
    """The oracle, untuned, on a bounded token sample of the same workload."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as mo

    def run(n):
        t0 = time.perf_counter()
        mo.layer_forward_backward(inp["x"][:n], inp["w_gate"], inp["w_up"], inp["w_down"], inp["dout"][:n], w.k,
                                  logits=None if "w_router" in inp else inp["logits"][:n],
                                  w_router=inp.get("w_router"))
        return time.perf_counter() - t0

    n0 = min(w.T, 256)
    t0 = run(n0)
    n = int(min(w.T, max(n0, (target_s / max(t0, 1e-3)) * n0)) // 64 * 64) or n0
    t = run(n) if n != n0 else t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": n / t, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {w.T} tokens of the same workload (all {w.E} experts, full d and f), "
                      f"fp64 forward+backward, {t:.1f} s wall",
            "numpy": np.__version__}


def timed_steps(step, steps: int, warmup: int) -> float:
    """ms per layer step over `steps` steps after `warmup` untimed ones."""
    import torch
    for _ in range(warmup):
        step.step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step.step()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def host_info() -> dict:
    """CPU model and the threads this process may use (the oracle's cores)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def smi_sample() -> dict:
    """Clock and power readings of GPU 0 from amd-smi (a short subprocess; its failure is recorded, not fatal)."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"], capture_output=True, text=True,
                           timeout=30)
    except (OSError, subprocess.SubprocessError) as exc:
        return {"error": f"{type(exc).__name__}: {exc}"[:200]}
    if r.returncode != 0:
        return {"error": (r.stderr or r.stdout).strip()[-200:]}
    try:
        data = json.loads(r.stdout)
    except ValueError:
        return {"error": "unparsed output", "head": r.stdout[:200]}
    out = {}

    def walk(node, path):
        if isinstance(node, dict):
            for key, val in node.items():
                walk(val, path + [str(key)])
        elif isinstance(node, list):
            for i, val in enumerate(node):
                walk(val, path + [str(i)])
        else:
            key = "/".join(path)
            low = key.lower()
            if any(t in low for t in ("gfx_0/clk", "mem_0/clk", "socket_power", "power_limit", "gfx_voltage")) \
                    and ("value" in low or low.endswith("clk") or "power" in low):
                out[key] = node
    walk(data, [])
    return out or {"raw_head": r.stdout[:600]}


def run_workload(w, dev_inp, steps: int, warmup: int, mx_per_step: bool = True) -> dict:
    """Time one workload: K steps with an event pair around each (value and the per-step spread), then
    the same K steps with the library's per-launch events (per-kernel durations).  Returns the figures
    and the LayerStep (for the callers' extra measurements)."""
    import statistics

    import torch

    from mixture_experts_layer_17_amd import binding as B
    from mixture_experts_layer_17_amd import layer as L

    step = L.LayerStep(w, dev_inp, mx_weights_per_step=mx_per_step)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    for _ in range(warmup):
        step.step()
    torch.cuda.synchronize()
    print(f"# {w.name}: warm-up done, timing {steps} steps", file=sys.stderr, flush=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for a, b in ev:
        a.record()
        step.step()
        b.record()
    stop.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / steps
    per = [a.elapsed_time(b) for a, b in ev]

    # the same K steps with HIP events around every library launch, recorded on the stream the kernels run
    # on -> per-kernel durations; the events add their own time to this pass only
    B.moe_timing_enable(True)
    step.step()
    torch.cuda.synchronize()
    B.moe_timing_report()  # discard the warm-up records (the event pool is now warm)
    start.record()
    for _ in range(steps):
        step.step()
    stop.record()
    torch.cuda.synchronize()
    ms_instrumented = start.elapsed_time(stop) / steps
    kern = B.moe_timing_report()
    B.moe_timing_enable(False)
    peak_mem = torch.cuda.max_memory_allocated()
    s = 4 if w.storage == "f32" else 2
    per_step_us = {name: 1e3 * ms / steps for name, (n, ms) in kern.items()}
    per_launch_us = {name: 1e3 * ms / n for name, (n, ms) in kern.items()}
    gemm_us = sum(v for kname, v in per_step_us.items() if kname[:2] in ("G1", "G2", "G3", "G4", "G5", "G6"))
    gemm_flops = 18.0 * w.R * w.d * w.f
    gemm_tflops = gemm_flops / (gemm_us * 1e-6) / 1e12 if gemm_us > 0 else None
    memk = {}
    for name in ("dispatch", "combine", "combine_bwd", "dispatch_bwd"):
        if name in per_launch_us:
            _, b = kernel_work(name, w, s)
            memk[name] = round(b / (per_launch_us[name] * 1e-6) / 1e9, 1)
    return {
        "step": step, "ms_per_step": ms_per_step, "per_step_ms": per, "ms_instrumented": ms_instrumented,
        "per_step_us": per_step_us, "per_launch_us": per_launch_us, "gemm_us": gemm_us, "gemm_flops": gemm_flops,
        "gemm_tflops": gemm_tflops, "memk": memk, "peak_mem": peak_mem, "s": s,
        "spread": {"median_ms": statistics.median(per), "min_ms": min(per), "max_ms": max(per)},
    }


def roofline(w, r: dict, active: int) -> dict:
    """The dominant kernel (largest time per step) against its binding roof, with its counted traffic if committed.
    A grouped GEMM is bound by whichever takes longer at peak: its FLOPs on the matrix cores or its algorithmic
    bytes over HBM."""
    per_step_us, per_launch_us = r["per_step_us"], r["per_launch_us"]
    dom = max(per_step_us, key=per_step_us.get)
    bound, work = kernel_work(dom, w, r["s"])
    if bound == "mfma" and w.prec != "f32":
        nbytes = gemm_bytes(dom, w, active)
        if nbytes / HBM_PEAK > work / PEAK[w.prec]:
            bound, work = "hbm", nbytes
    avg_s = per_launch_us[dom] * 1e-6
    tag = f"{w.name.replace('-', '_')}_T{w.T}"
    traffic = counted_traffic(tag, dom)
    if bound == "mfma":
        peak = PEAK[w.prec]
        roof = {"bound": "mfma" if w.prec != "f32" else "alu", "kernel": dom, "achieved": work / avg_s / 1e12,
                "peak": peak / 1e12, "unit": "TFLOP/s", "frac": work / avg_s / peak, "traffic": traffic,
                "work_per_launch": f"{work:.4g} FLOP", "avg_launch_us": per_launch_us[dom]}
    else:
        roof = {"bound": "hbm", "kernel": dom, "achieved": work / avg_s / 1e9, "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": work / avg_s / HBM_PEAK, "traffic": traffic,
                "work_per_launch": f"{work:.4g} B", "avg_launch_us": per_launch_us[dom]}
    roof["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE x2.0 + WRITE_SIZE x1.0, copy-calibrated)"
    roof["traffic_source"] = f"profiles/{tag}_hbm_traffic.md" if traffic is not None else \
        "null: no counter summary taken with the current kernel sources"
    return roof


def gemm_roofs(w, r: dict, active: int) -> dict:
    """Each grouped GEMM against its binding roof (matrix cores or HBM, whichever takes longer at peak)."""
    out = {}
    for name, us in sorted(r["per_launch_us"].items()):
        bound, flops = kernel_work(name, w, r["s"])
        if bound != "mfma" or w.prec == "f32":
            continue
        nbytes = gemm_bytes(name, w, active)
        t_mfma, t_hbm = flops / PEAK[w.prec], nbytes / HBM_PEAK
        out[name] = {"us": round(us, 1), "tflops": round(flops / (us * 1e-6) / 1e12, 1),
                     "frac_mfma": round(t_mfma / (us * 1e-6), 3), "gbps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "frac_hbm": round(t_hbm / (us * 1e-6), 3), "bound": "mfma" if t_mfma >= t_hbm else "hbm",
                     "frac_roof": round(max(t_mfma, t_hbm) / (us * 1e-6), 3)}
    return out


def summary(w, r: dict, active: int) -> dict:
    """Compact figures of one workload for the JSON line."""
    peak = PEAK[w.prec]
    return {
        "workload": f"{w.name}: T={w.T} d={w.d} E={w.E} k={w.k} f={w.f}, {w.prec} expert GEMMs",
        "tokens_per_s": w.T / (r["ms_per_step"] * 1e-3), "ms_per_step": r["ms_per_step"],
        "step_ms": r["spread"],
        "gemm": {"tflops": r["gemm_tflops"], "frac_of_peak": (r["gemm_tflops"] * 1e12 / peak) if r["gemm_tflops"]
                 else None, "peak_tflops": peak / 1e12, "us_per_step": r["gemm_us"]},
        "hbm_kernels_gbps": r["memk"],
        "roofline": roofline(w, r, active),
        "gemm_roofs": gemm_roofs(w, r, active),
        "kernels_us_per_step": {k: round(v, 2) for k, v in sorted(r["per_step_us"].items())},
        "peak_mem_gib": r["peak_mem"] / 2**30,
    }


def c1_single_core(runs: int = 10) -> dict:
    """The oracle on the tiny fp32 workload on one thread: median of `runs` runs."""
    import statistics

    from threadpoolctl import threadpool_limits

    from mixture_experts_layer_17_amd import workloads as wl
    from oracle import moe_oracle as mo

    w = wl.WORKLOADS[1]
    inp = wl.make_inputs(w)
    times = []
    with threadpool_limits(limits=1):
        for _ in range(runs):
            t0 = time.perf_counter()
            mo.layer_forward_backward(inp["x"], inp["w_gate"], inp["w_up"], inp["w_down"], inp["dout"], w.k,
                                      w_router=inp["w_router"])
            times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    return {"workload": f"{w.name}: T={w.T} d={w.d} E={w.E} k={w.k} f={w.f}", "median_s": med,
            "min_s": min(times), "runs": runs, "tokens_per_s": w.T / med, "cores": 1}


def pool_sweep(args) -> int:
    """Expert-pool sweep at a fixed token count: how the layer's throughput moves as the same routed rows
    spread over more, smaller experts (the pages report a small drop from 8 to 128 experts at top-4)."""
    import torch

    from mixture_experts_layer_17_amd import binding as B
    from mixture_experts_layer_17_amd import layer as L
    from mixture_experts_layer_17_amd import workloads as wl

    rows = []
    for E in (8, 16, 32, 64, 128):
        w = wl.scaled(wl.WORKLOADS[3], E=E, name=f"bf16-pool-e{E}")
        print(f"# pool sweep E={E}: generating inputs", file=sys.stderr, flush=True)
        step = L.LayerStep(w, L.to_device(wl.make_inputs(w, seed=args.seed)))
        ms = timed_steps(step, args.steps, args.warmup)
        rs = B.moe_route_stats(step.route["counts"]).cpu().tolist()
        rows.append({"E": E, "tokens_per_s": w.T / (ms * 1e-3), "ms_per_step": ms,
                     "gemm_tflops_est": 18.0 * w.R * w.d * w.f / (ms * 1e-3) / 1e12,
                     "max_rows": rs[0], "min_rows": rs[1], "empty_experts": rs[2]})
        print(f"# E={E}: {rows[-1]['tokens_per_s']:.0f} tokens/s", file=sys.stderr, flush=True)
        del step
        torch.cuda.empty_cache()
    base = rows[0]["tokens_per_s"]
    for r in rows:
        r["vs_e8"] = r["tokens_per_s"] / base
    print(json.dumps({"pool_sweep": rows, "config": "bf16, T=16384, d=2048, k=4, f=1024, N(0,1) router logits, "
                      "whole-layer fwd+bwd tokens/s (gemm_tflops_est: 18 R d f over the whole step)",
                      "steps": args.steps, "warmup": args.warmup}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=5,
                    help="1..5 (default 5: MXFP8, T=16384, d=4096, E=128, top-4, f=1536, the largest)")
    ap.add_argument("--seed", type=int, default=17)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-companions", action="store_true",
                    help="with workload 5: skip the BF16 run on the same tensors and the bf16-e128 workload")
    ap.add_argument("--trace-only", action="store_true",
                    help="only the warm-up and the timed steps (for profiler traces: every launch belongs to a "
                         "step), then a short JSON line")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--pool-sweep", action="store_true",
                    help="only time the bf16 layer at T=16384, d=2048, k=4, f=1024 for E = 8, 16, 32, 64, 128 "
                         "(N(0,1) router logits) and print one JSON line with the sweep")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the MoE layer; the library has no multi-GPU path "
              "(no collectives, no expert sharding), so only --gpus 1 runs.", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return 0

    import dataclasses

    import torch

    from mixture_experts_layer_17_amd import binding as B
    from mixture_experts_layer_17_amd import layer as L
    from mixture_experts_layer_17_amd import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    if args.pool_sweep:
        return pool_sweep(args)
    w = wl.WORKLOADS[args.workload]
    print(f"# workload {w.name} {w.describe()}: generating inputs", file=sys.stderr, flush=True)
    inp = wl.make_inputs(w, seed=args.seed)
    dev_inp = L.to_device(inp)
    if args.trace_only:
        # MXFP8: each step quantises the expert weights once, into both layouts, for its forward and backward
        step = L.LayerStep(w, dev_inp, mx_weights_per_step=True)
        ms = timed_steps(step, args.steps, args.warmup)
        print(json.dumps({"metric": METRIC, "value": w.T / (ms * 1e-3), "unit": "tokens/s",
                          "ms_per_step": ms, "steps": args.steps, "warmup": args.warmup,
                          "workload": w.name, "trace_only": True}), flush=True)
        return 0
    smi_before = smi_sample()
    # the headline workload; MXFP8 steps quantise the expert weights once per step into both layouts
    r = run_workload(w, dev_inp, args.steps, args.warmup, mx_per_step=True)
    step = r["step"]
    rs = B.moe_route_stats(step.route["counts"]).cpu().tolist()  # after the timed region
    head = summary(w, r, w.E - rs[2])
    line = {
        "metric": METRIC,
        "value": w.T / (r["ms_per_step"] * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "mxfp8": "mxfp8"}[w.prec],
        "data": "synthetic: seeded normal activations/logits/upstream grads, random-init weights (std 0.02)",
        "config": {"workload": f"{w.name}: T={w.T} d={w.d} E={w.E} k={w.k} f={w.f}, SwiGLU experts, "
                               f"fwd+bwd incl. routing" + (", expert weights quantised to MXFP8 every step"
                                                          if w.prec == "mxfp8" else ""),
                   "global_batch": w.T, "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "step_ms": head["step_ms"],
        "gemm": head["gemm"],
        "gemm_roofs": head["gemm_roofs"],
        "hbm_kernels_gbps": head["hbm_kernels_gbps"],
        "kernels_us_per_step": head["kernels_us_per_step"],
        "kernel_timing": f"HIP events around every launch over a second pass of the same {args.steps} steps "
                         f"({r['ms_instrumented']:.3f} ms/step with the events; value, ms_per_step and step_ms "
                         f"come from the first pass, one event pair per step)",
        "peak_mem_gib": head["peak_mem_gib"],
        "routing_stats": {"max_rows": rs[0], "min_rows": rs[1], "empty_experts": rs[2], "rows": rs[3],
                          "max_over_mean": rs[0] * w.E / max(rs[3], 1)},
    }
    if w.prec == "mxfp8":
        # the other two ways of handling the weights, same buffers and inputs
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record()
        step.build_weight_cache()
        b1.record()
        torch.cuda.synchronize()
        build_ms = b0.elapsed_time(b1)
        step.mx_per_step = False
        ms_once = timed_steps(step, args.steps, args.warmup)   # cache built above, reused
        cache, step.mx_wcache = step.mx_wcache, None
        ms_pass = timed_steps(step, args.steps, args.warmup)   # forward and backward quantise their own layouts
        step.mx_wcache, step.mx_per_step = cache, True
        line["mx_weights"] = {
            "value": "expert weights quantised at the start of every step into both layouts from one read "
                     "(moe_mx_weight_cache_build, inside the timed step) and used by its forward and backward",
            "build_ms": build_ms,
            "per_pass": {"tokens_per_s": w.T / (ms_pass * 1e-3), "ms_per_step": ms_pass,
                         "note": "forward and backward each quantise the weight layout they use (no cache)"},
            "once": {"tokens_per_s": w.T / (ms_once * 1e-3), "ms_per_step": ms_once,
                     "note": "weights quantised once before the loop and reused (build excluded): the rate of "
                             "micro-batches that share one optimiser step"}}
    del step, r
    torch.cuda.empty_cache()
    if w.prec == "mxfp8" and not args.no_companions:
        # the same shapes and the same bf16 tensors with BF16 expert GEMMs: the MXFP8 / BF16 comparison
        wb = dataclasses.replace(w, name=f"{w.name}-as-bf16", prec="bf16")
        print(f"# {wb.name}: same tensors, BF16 expert GEMMs", file=sys.stderr, flush=True)
        rb = run_workload(wb, dev_inp, args.steps, args.warmup)
        line["bf16_same_tensors"] = summary(wb, rb, w.E - rs[2])
        line["mxfp8_over_bf16"] = line["value"] / line["bf16_same_tensors"]["tokens_per_s"]
        del rb
        torch.cuda.empty_cache()
        w3 = wl.WORKLOADS[3]
        print(f"# workload {w3.name}: generating inputs", file=sys.stderr, flush=True)
        d3 = L.to_device(wl.make_inputs(w3, seed=args.seed))
        r3 = run_workload(w3, d3, args.steps, args.warmup)
        rs3 = B.moe_route_stats(r3["step"].route["counts"]).cpu().tolist()
        line["bf16_e128"] = summary(w3, r3, w3.E - rs3[2])
        del r3, d3
        torch.cuda.empty_cache()
    line["gpu_clocks_power"] = {"before": smi_before, "after": smi_sample()}
    line["host"] = host_info()
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a token sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
        line["cpu_c1_single_core"] = c1_single_core()
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
