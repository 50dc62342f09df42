#!/usr/bin/env python3
"""Benchmark of the lightning-indexer scoring path on one MI355X.

A step is one complete call of the path: the plan (windows + schedule) built
inside the call, then the scoring kernel with its -inf cleanup, on inputs
already resident in device memory.  The default workload is the MXFP8
Q2048 / KV32768, H64 / D128, clean_logits=True call with FP32 weights and
output and rows seeing [0, KV-Q+row) -- the configuration DeepGEMM pull
request 435 times (Performance section) -- on seeded random inputs.

Prints one JSON line.  Alongside the whole-call time it reports the roofline
of the scoring kernel alone (timed with events on the stream it runs on, plan
precomputed) and the fp64 CPU oracle timed on a bounded sample of the same
workload.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0, "mxfp4": 10100.0}
HBM_GBS = 8000.0
METRIC = "µs/call + effective TFLOP/s (visible cells) at H64/D128, MXFP8 Q2048/KV32768"
PAGES_US = {"c4_mxfp8_zero": 412.0, "c4_mxfp4_zero": 407.9}  # GB200, no metadata, all-zero inputs


def device_inputs(wl, dev) -> dict:
    """Raw code buffers of a workload as device tensors."""
    import torch

    def t(a, as_dtype=None):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        elif a.dtype == np.uint32:
            a = a.view(np.int32)
        x = torch.from_numpy(a).to(dev)
        return x.view(as_dtype) if as_dtype is not None else x

    return {"q": t(wl.q), "k": t(wl.k), "q_scale": t(wl.q_scale), "k_scale": t(wl.k_scale),
            "w": t(wl.w, torch.bfloat16 if wl.w_dtype == "bf16" else None),
            "offsets": t(None if wl.offsets is None else np.asarray(wl.offsets, np.int32)),
            "starts": t(None if wl.starts is None else np.asarray(wl.starts, np.int32)),
            "ends": t(None if wl.ends is None else np.asarray(wl.ends, np.int32))}


def call(lib, wl, d, out, plan=None):
    """One scoring call through the C ABI (plan None: built inside the call)."""
    return lib.idx_logits_run(d["q"], d["k"], d["w"], in_dtype=wl.fmt, q_scale=d["q_scale"],
                              k_scale=d["k_scale"], sm_scale=wl.sm_scale, clean_logits=wl.clean, out=out,
                              plan=plan, q_causal_offsets=d["offsets"], row_starts=d["starts"],
                              row_ends=d["ends"], workspace=d.get("workspace"))


def visible_cells(lib, wl, plan) -> int:
    """Visible cells from the windows the library's plan holds."""
    ws, we = lib.idx_logits_plan_windows(plan, wl.B, wl.S_q, wl.S_k)
    return int((we.long() - ws.long()).clamp(min=0).sum().item())


def input_bytes(wl) -> int:
    n = wl.q.nbytes + wl.k.nbytes + wl.w.nbytes
    for a in (wl.q_scale, wl.k_scale):
        if a is not None:
            n += a.nbytes
    return n


def out_bytes(wl, V: int) -> int:
    per = 2 if wl.out_dtype == "bf16" else 4
    return per * (wl.B * wl.S_q * wl.S_k if wl.clean else V)


def cpu_baseline(wl, V: int, target_s: float = 12.0) -> dict:
    """Time the fp64 oracle on whole rows of the workload for about target_s
    seconds and scale to one full call by visible cells."""
    import oracle
    ws, we = oracle.windows(wl)
    vis = np.maximum(we.astype(np.int64) - ws, 0).reshape(-1)
    order = np.random.default_rng(0).permutation(vis.size)
    n, dt = 8, 0.0
    while True:
        rows = order[:n]
        t0 = time.perf_counter()
        _, _, threads = oracle.logits(wl, rows=rows, return_threads=True)
        dt = time.perf_counter() - t0
        if dt >= 0.5 * target_s or n >= vis.size:
            break
        n = min(vis.size, max(n + 1, int(n * target_s / max(dt, 1e-3))))
    v_sample = int(vis[rows].sum())
    us_per_call = dt * (V / max(v_sample, 1)) * 1e6
    return {"value": round(us_per_call, 1), "unit": "µs/call", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(rows)} of {vis.size} rows ({v_sample} visible cells) timed {dt:.1f} s, "
                      f"scaled by visible cells to the full call", "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4_mxfp8",
                    help="named workload (c1, c2, c3, c3_noclean, c4_mxfp8, c4_mxfp4, *_zero, c5, c5_nonaligned)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-zero-variant", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only run a plain device copy of this many bytes `steps` times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import mqa_logits_scoring_amd as lib
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "steps": args.steps}), flush=True)
        return

    def measure(name: str):
        wl = W.make(name)
        d = device_inputs(wl, dev)
        stream = torch.cuda.current_stream(dev)
        odt = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
        outs = [torch.empty((wl.B, wl.S_q, wl.S_k), dtype=odt, device=dev) for _ in range(2)]
        plan = lib.idx_logits_plan(wl.B, wl.S_q, wl.S_k, wl.H, wl.D, q_causal_offsets=d["offsets"],
                                   row_starts=d["starts"], row_ends=d["ends"], device=dev)
        cargs = lib.make_args(d["q"], d["k"], d["w"], outs[0], in_dtype=wl.fmt, q_scale=d["q_scale"],
                             k_scale=d["k_scale"], sm_scale=wl.sm_scale, clean_logits=wl.clean)
        d["workspace"] = torch.empty(lib.idx_logits_workspace_bytes(cargs), dtype=torch.uint8, device=dev)
        V = visible_cells(lib, wl, plan)
        for i in range(args.warmup):
            call(lib, wl, d, outs[i % 2])
        torch.cuda.synchronize()
        # the whole call, plan built inside: exactly `steps` steps
        t0 = time.perf_counter()
        for i in range(args.steps):
            call(lib, wl, d, outs[i % 2])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        us_call = wall / args.steps * 1e6
        # the scoring kernel alone (plan precomputed), events on its stream
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        samples = []
        for rep in range(5):
            ev0.record(stream)
            for i in range(args.steps):
                call(lib, wl, d, outs[i % 2], plan=plan)
            ev1.record(stream)
            ev1.synchronize()
            samples.append(ev0.elapsed_time(ev1) * 1000 / args.steps)
        kern_us = statistics.median(samples)
        return wl, V, us_call, kern_us

    wl, V, us_call, kern_us = measure(args.workload)
    flops = 16384.0 * V
    peak = PEAK_TFLOPS[wl.fmt]
    achieved = flops / (kern_us * 1e-6) / 1e12
    res = {
        "metric": METRIC,
        "value": round(us_call, 2),
        "unit": "µs/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_call / 1000, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.fmt,
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "S_q": wl.S_q, "S_k": wl.S_k, "H": wl.H, "D": wl.D,
                   "in_dtype": wl.fmt, "w_dtype": wl.w_dtype, "out_dtype": wl.out_dtype,
                   "clean_logits": wl.clean, "visible_cells": V, "plan": "built inside each call",
                   "inputs": f"seeded random (seed {wl.seed})"},
        "eff_tflops": round(flops / (us_call * 1e-6) / 1e12, 1),
        "out_gbs": round(out_bytes(wl, V) / (us_call * 1e-6) / 1e9, 1),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "kernel": "score_kernel (plan precomputed)", "kernel_us": round(kern_us, 2),
                     "flop_per_launch": flops, "algorithmic_bytes_per_launch": input_bytes(wl) + out_bytes(wl, V)},
    }
    zero_name = args.workload + "_zero"
    if not args.no_zero_variant and zero_name in W.NAMED:
        zwl, zV, zus, zk = measure(zero_name)
        res["zero_inputs"] = {"workload": zwl.name, "us_per_call": round(zus, 2), "kernel_us": round(zk, 2),
                              "pages_us_gb200": PAGES_US.get(zero_name),
                              "ratio_to_pages": round(zus / PAGES_US[zero_name], 3) if zero_name in PAGES_US else None}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, V)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
