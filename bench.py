#!/usr/bin/env python3
"""Benchmark of the lightning-indexer scoring path on one MI355X.

A step is one complete call of the path on inputs already resident in device
memory: idx_logits_run, which builds the per-call preparation (K in fragment
order, weighted-query pieces) and, without a precomputed plan, the plan
(windows + schedule) in one launch, then runs the scoring kernel with its
-inf cleanup.  The default workload is the MXFP8 Q2048 / KV32768, H64 / D128,
clean_logits=True call with FP32 weights and output and rows seeing
[0, KV-Q+row) -- the configuration DeepGEMM pull request 435 times
(Performance section) -- on seeded random inputs, with its all-zero variant
beside it.

Timing follows that page's protocol, on HIP graphs: every variant is warmed,
then captured as a graph of 5 calls into 5 distinct retained outputs and
replayed 5 times; after a pre-warm that lets the clock settle, each of
`steps` samples replays every variant twice (the second replay is timed with
events on the stream the library launches on, divided by 5), the variants'
order rotating and reversing from sample to sample so that they share one
clock state.  Reported: median / p10 / p90 per variant.  The variants are the
call without a plan ("metadata no", the headline `value`), the call with a
plan built outside timing ("metadata yes"), the scoring kernel alone on a
prepared workspace (the roofline's kernel time), the same for the all-zero
inputs, and for FP8 / MXFP8 the call with exact accumulation.  Every graph's
outputs are checked bitwise against eager calls.

HBM traffic comes from the rocprofv3 FETCH_SIZE / WRITE_SIZE counts kept under
profiles/ (calibrated against a plain copy), and only while the kernel sources
are the ones they were taken on.  The fp64 CPU oracle is timed on a bounded
sample of the same workload.

    python bench.py --write-traffic WORKLOAD FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv COPY_BYTES [COPY_RE]
turns rocprofv3 --pmc counter files into that traffic record (the copy runs
are of `bench.py --copy-bytes COPY_BYTES`; COPY_RE picks its kernel).
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
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
METRIC = "µs/call + effective TFLOP/s (visible cells) at H64/D128, MXFP8 Q2048/KV32768"
# GB200, no metadata, all-zero inputs (DeepGEMM pull request 435, Performance section)
PAGES_US = {"c4_mxfp8_zero": 412.0, "c4_mxfp4_zero": 407.9, "q8k_mxfp8_zero": 3022.2, "q8k_mxfp4_zero": 2968.9}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")
CSRC = os.path.join(ROOT, "mqa_logits_scoring_amd", "csrc")


def kernel_source_hash(fmt: str) -> str:
    """sha256 over the sources of the scoring kernel of one input format,
    with the host code that splits its work into units (fmt "topk": of the
    top-k kernel)."""
    import hashlib
    h = hashlib.sha256()
    files = ("topk.hip", "select_wave.h", "internal.h") if fmt == "topk" else ("score_kernel.h", "score_kernel_gh.h", "internal.h",
                                                              f"score_{fmt}.hip", "api.cpp")
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(workload: str, fmt: str):
    """HBM bytes per launch of the scoring kernel from the stored counter
    record, or None when there is none or the kernel changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256") != kernel_source_hash(fmt):
        return None
    return rec


def _counter_per_dispatch(path: str, counter: str, kernel_re: str) -> float:
    """Mean over matching dispatches of a counter (summed over its instances)
    in a rocprofv3 counter_collection.csv."""
    import csv
    import re
    per = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter or not re.search(kernel_re, r["Kernel_Name"]):
                continue
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"{path}: no {counter} rows for kernels matching {kernel_re!r}")
    return sum(per.values()) / len(per)


def write_traffic(argv) -> None:
    """argv: workload fetch.csv write.csv copy_fetch.csv copy_write.csv copy_bytes [copy_re [topk_k]].
    With topk_k the record is the top-k kernel's (key topk<k>:<workload>)."""
    workload, fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes = argv[:6]
    copy_re = argv[6] if len(argv) > 6 else "copy"
    topk_k = int(argv[7]) if len(argv) > 7 else 0
    import workloads as W
    wl = W.make(workload)
    fmt, workload = wl.fmt, wl.name
    kernel_re = "score_kernel"
    if topk_k:
        fmt, workload, kernel_re = "topk", f"topk{topk_k}:{wl.name}", "topk_rows_kernel|topk_kernel"
    copy_bytes = int(copy_bytes)
    kib = 1024.0
    # the copy kernel reads and writes copy_bytes per dispatch
    f_cal = copy_bytes / (_counter_per_dispatch(cfetch_csv, "FETCH_SIZE", copy_re) * kib)
    w_cal = copy_bytes / (_counter_per_dispatch(cwrite_csv, "WRITE_SIZE", copy_re) * kib)
    fetch = _counter_per_dispatch(fetch_csv, "FETCH_SIZE", kernel_re) * kib * f_cal
    write = _counter_per_dispatch(write_csv, "WRITE_SIZE", kernel_re) * kib * w_cal
    try:
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    except (OSError, ValueError):
        data = {}
    data[workload] = {"fetch_bytes": round(fetch), "write_bytes": round(write), "fetch_calibration": round(f_cal, 4),
                      "write_calibration": round(w_cal, 4), "copy_bytes": copy_bytes,
                      "source_sha256": kernel_source_hash(fmt)}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps({workload: data[workload]}))


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

    d = {"q": t(wl.q), "k": t(wl.k), "q_scale": t(wl.q_scale), "k_scale": t(wl.k_scale),
         "w": t(wl.w, torch.bfloat16 if wl.w_dtype == "bf16" else None),
         "offsets": t(None if wl.offsets is None else np.asarray(wl.offsets, np.int32)),
         "starts": t(None if wl.starts is None else np.asarray(wl.starts, np.int32)),
         "ends": t(None if wl.ends is None else np.asarray(wl.ends, np.int32))}
    if getattr(wl, "thd", None) is not None:
        d["cu_q"] = t(np.asarray(wl.thd["cu_q"], np.int32))
        d["cu_k"] = t(np.asarray(wl.thd["cu_k"], np.int32))
    if getattr(wl, "paged", None) is not None:
        import mqa_logits_scoring_amd as lib
        pg = wl.paged
        d["k_cache"], d["k_scale_cache"] = t(pg["k_cache"]), t(pg["k_scale_cache"])
        d["block_table"] = t(np.asarray(pg["block_table"], np.int32))
        d["ctx"] = t(np.asarray(pg["ctx"], np.int32))
        d["kv"] = lib.make_paged_k(d["k_cache"], d["block_table"], d["ctx"], d["k_scale_cache"])
    return d


def build_plan(lib, wl, d, plan, stream):
    """The call's plan: from causal offsets or explicit windows, or for packed
    variable-length rows from the segment boundaries and the ratio."""
    if getattr(wl, "thd", None) is not None:
        return lib.idx_logits_plan_thd(d["cu_q"], d["cu_k"], wl.thd["ratio"], wl.S_q, wl.S_k, wl.H, wl.D, plan=plan,
                                       stream=stream)
    if getattr(wl, "paged", None) is not None:
        return lib.idx_logits_plan_paged(wl.B, wl.S_q, wl.S_k, d["ctx"], wl.H, wl.D, plan=plan, stream=stream)
    return lib.idx_logits_plan(wl.B, wl.S_q, wl.S_k, wl.H, wl.D, q_causal_offsets=d["offsets"],
                               row_starts=d["starts"], row_ends=d["ends"], plan=plan, stream=stream)


def visible_cells(lib, wl, plan) -> int:
    """Visible cells from the windows the library's plan holds."""
    ws, we = lib.idx_logits_plan_windows(plan, wl.B, wl.S_q, wl.S_k, wl.H, wl.D)
    v = int((we.long() - ws.long()).clamp(min=0).sum().item())
    if v == 0 and bool((ws < 0).any()):
        raise RuntimeError("the plan does not match the workload's dimensions")
    return v


def input_bytes(wl) -> int:
    """Bytes of the inputs a call must read once: for a paged cache, the rows
    inside the requests' (clamped) contexts."""
    n = wl.q.nbytes + wl.w.nbytes + (0 if wl.q_scale is None else wl.q_scale.nbytes)
    if getattr(wl, "paged", None) is not None:
        pg = wl.paged
        rows = int(np.clip(np.asarray(pg["ctx"], np.int64), 0, wl.S_k).sum())
        row_bytes = pg["k_cache"].nbytes // (pg["k_cache"].shape[0] * pg["k_cache"].shape[1])
        scale_bytes = 0 if pg["k_scale_cache"] is None else pg["k_scale_cache"].dtype.itemsize
        return n + rows * (row_bytes + scale_bytes)
    return n + wl.k.nbytes + (0 if wl.k_scale is None else wl.k_scale.nbytes)


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


def measure_peaks(dev, settle_s: float = 0.3) -> dict | None:
    """The matrix-core throughput of every MFMA shape the scoring kernels use
    (libidx_peak.so: independent MFMAs on register operands, pseudo-random or
    zero codes, two waves per SIMD) and a plain 1 GiB device copy, measured
    here.  Each case runs `settle_s` seconds before 10 timed launches, so the
    clock has settled under its own power draw."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "mqa_logits_scoring_amd", "libidx_peak.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.idx_peak_mfma.restype = ctypes.c_int32
    L.idx_peak_mfma.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    L.idx_peak_flop_per_mfma.restype = ctypes.c_double
    L.idx_peak_flop_per_mfma.argtypes = [ctypes.c_int32]
    groups = 512  # two 4-wave workgroups per CU
    out = torch.empty(groups * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    names = {0: "bf16_32x32x16", 1: "fp8_32x32x64", 2: "fp8_16x16x128", 3: "fp4_32x32x64", 4: "fp4_16x16x128"}
    res = {}
    for kind, name in names.items():
        flop1 = L.idx_peak_flop_per_mfma(kind)
        iters = max(1, int(4e12 / (groups * 4 * 8 * flop1)))
        flop = groups * 4 * 8 * iters * flop1
        res[name] = {}
        for zero in (0, 1):
            def go():
                st = L.idx_peak_mfma(kind, groups, iters, zero, out.data_ptr(), stream.cuda_stream)
                if st != 0:
                    raise RuntimeError(f"idx_peak_mfma({kind}) failed with status {st}")
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < settle_s:
                go()
                torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                go()
            e1.record(stream)
            e1.synchronize()
            res[name]["zero" if zero else "random"] = round(10 * flop / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    e1.synchronize()
    copy_gbs = 5 * 2 * n * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    return {"mfma_tflops": res, "copy_gbs": round(copy_gbs, 1),
            "note": "MFMA: independent MFMAs per shape, 2 waves per SIMD, random or zero operands; "
                    "copy: 1 GiB device-to-device, read + write bytes"}


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gpu_clock_state() -> dict:
    """amd-smi's view of GPU 0's clocks and power (best effort: a missing tool
    or an unknown output layout is reported, not raised)."""
    import subprocess
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        # under a profiler the tool's preload would start with the child
        return {"skipped": "running under a profiler"}
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "--clock", "--power", "--json"], capture_output=True,
                           text=True, timeout=30)
        data = json.loads(r.stdout)
    except Exception as e:  # noqa: BLE001 - a diagnostic, never fatal
        return {"error": f"{type(e).__name__}: {e}"[:200]}
    found = {}

    def walk(x, path):
        if isinstance(x, dict):
            for k, v in x.items():
                walk(v, path + [str(k)])
        elif isinstance(x, list):
            for i, v in enumerate(x):
                walk(v, path + [str(i)])
        else:
            key = ".".join(path).lower()
            if (("gfx" in key and "clk" in key) or "power" in key) and len(found) < 24:
                found[".".join(path)] = x
    walk(data, [])
    return found or {"raw": r.stdout[:400]}


class Variant:
    """One timed variant: `launch(i)` enqueues one call into output i of 5 on
    torch's current stream (the graph's capture stream while capturing)."""

    def __init__(self, name, launch, outs, ref_group):
        self.name, self.launch, self.outs, self.ref_group = name, launch, outs, ref_group
        self.graph = None
        self.samples = []


def _pct(xs, q):
    return float(np.percentile(np.asarray(xs, np.float64), q))


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--write-traffic":
        write_traffic(sys.argv[2:])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40, help="timed samples (each replays every variant's graph)")
    ap.add_argument("--warmup", type=int, default=5, help="untimed graph replays of every variant after capture")
    ap.add_argument("--workload", default="c4_mxfp8",
                    help="named workload (c1, c2, c3, c3_noclean, c4_mxfp8, c4_mxfp4, *_zero, c5, c5_nonaligned, "
                         "thd_bf16_r4, paged_mxfp8_decode, screen_h8/h32/h64)")
    ap.add_argument("--prewarm-s", type=float, default=1.0,
                    help="seconds of untimed replays before the samples (lets the GPU clock settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-zero-variant", action="store_true")
    ap.add_argument("--no-exact-variant", action="store_true",
                    help="skip the FP8 / MXFP8 call with exact (fp32) accumulation")
    ap.add_argument("--no-peaks", action="store_true", help="skip the MFMA-shape and copy peak measurement")
    ap.add_argument("--topk", type=int, default=2048,
                    help="also time top-k selection (this k, by column): over the call's scores, and fused with "
                         "the scoring (idx_logits_run_topk); 0 skips both")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure the MFMA throughput per shape and a device copy (libidx_peak.so)")
    ap.add_argument("--eager", action="store_true",
                    help="launch the 5 calls of a sample directly instead of replaying a captured graph "
                         "(for profilers that follow plain kernel launches)")
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

    if args.peaks:
        print(json.dumps(measure_peaks(dev, settle_s=1.0)), flush=True)
        return

    if args.copy_bytes:
        src = torch.ones(args.copy_bytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "steps": args.steps}), flush=True)
        return

    wl = W.make(args.workload)
    paged = getattr(wl, "paged", None) is not None
    thd = getattr(wl, "thd", None) is not None
    odt = torch.bfloat16 if wl.out_dtype == "bf16" else torch.float32
    iv = torch.int16 if odt == torch.bfloat16 else torch.int32
    variants = []
    keep = []  # tensors the graphs read or write

    def add_workload(w, tag, with_plan_variants):
        d = device_inputs(w, dev)
        keep.append(d)
        plan = torch.empty(lib.idx_logits_plan_bytes(w.B, w.S_q, w.S_k, w.H, w.D), dtype=torch.uint8, device=dev)
        build_plan(lib, w, d, plan, None)
        keep.append(plan)

        def outs5():
            o = [torch.empty((w.B, w.S_q, w.S_k), dtype=odt, device=dev) for _ in range(5)]
            keep.extend(o)
            return o

        def args_for(o, accumulate="native"):
            if paged:
                return lib.make_paged_args(d["q"], d["w"], o, w.S_k, in_dtype=w.fmt, q_scale=d["q_scale"],
                                           sm_scale=w.sm_scale, clean_logits=w.clean, accumulate=accumulate)
            return lib.make_args(d["q"], d["k"], d["w"], o, in_dtype=w.fmt, q_scale=d["q_scale"], k_scale=d["k_scale"],
                                 sm_scale=w.sm_scale, clean_logits=w.clean, accumulate=accumulate)

        def call_variant(name, use_plan, accumulate="native"):
            o = outs5()
            a0 = args_for(o[0], accumulate)
            ws = torch.empty(lib.idx_logits_workspace_bytes(a0), dtype=torch.uint8, device=dev)
            keep.append(ws)
            tplan = None
            if thd and not use_plan:  # packed rows build their plan with idx_logits_plan_thd in the call
                tplan = torch.empty_like(plan)
                keep.append(tplan)

            def launch(i):
                if paged:
                    lib.idx_logits_run_paged(d["q"], d["w"], d["kv"], w.S_k, in_dtype=w.fmt, q_scale=d["q_scale"],
                                             sm_scale=w.sm_scale, clean_logits=w.clean, out=o[i], workspace=ws,
                                             plan=plan if use_plan else None, accumulate=accumulate)
                    return
                p = plan if use_plan else (build_plan(lib, w, d, tplan, None) if thd else None)
                lib.idx_logits_run(d["q"], d["k"], d["w"], in_dtype=w.fmt, q_scale=d["q_scale"],
                                   k_scale=d["k_scale"], sm_scale=w.sm_scale, clean_logits=w.clean, out=o[i],
                                   plan=p, q_causal_offsets=d["offsets"], row_starts=d["starts"], row_ends=d["ends"],
                                   workspace=ws, accumulate=accumulate)
            variants.append(Variant(name, launch, o, f"{tag}:{accumulate}"))

        def score_variant(name):
            o = outs5()
            cargs = [args_for(x) for x in o]
            ws = torch.empty(lib.idx_logits_workspace_bytes_planned(cargs[0]), dtype=torch.uint8, device=dev)
            keep.append(ws)
            if paged:
                lib.idx_logits_prepare_paged(cargs[0], d["kv"], ws)
            else:
                lib.idx_logits_prepare(cargs[0], ws)

            def launch(i):
                if paged:
                    lib.idx_logits_score_paged(cargs[i], d["kv"], plan, ws)
                else:
                    lib.idx_logits_score(cargs[i], plan, ws)
            variants.append(Variant(name, launch, o, f"{tag}:native"))

        call_variant(f"{tag}call", False)
        if with_plan_variants:
            call_variant(f"{tag}call_planned", True)
            score_variant(f"{tag}kernel")
        return d, plan

    d, plan = add_workload(wl, "", True)
    zero_name = args.workload + "_zero"
    zwl = None
    if not args.no_zero_variant and zero_name in W.NAMED:
        zwl = W.make(zero_name)
        add_workload(zwl, "zero_", True)
    exact = wl.fmt in ("fp8", "mxfp8") and not args.no_exact_variant
    if exact:
        # the same call with exact accumulation (bf16 matrix core on converted operands)
        dd = d
        o = [torch.empty((wl.B, wl.S_q, wl.S_k), dtype=odt, device=dev) for _ in range(5)]
        keep.extend(o)
        if paged:
            a0 = lib.make_paged_args(dd["q"], dd["w"], o[0], wl.S_k, in_dtype=wl.fmt, q_scale=dd["q_scale"],
                                     sm_scale=wl.sm_scale, clean_logits=wl.clean, accumulate="fp32")
        else:
            a0 = lib.make_args(dd["q"], dd["k"], dd["w"], o[0], in_dtype=wl.fmt, q_scale=dd["q_scale"],
                               k_scale=dd["k_scale"], sm_scale=wl.sm_scale, clean_logits=wl.clean,
                               accumulate="fp32")
        ws_x = torch.empty(lib.idx_logits_workspace_bytes(a0), dtype=torch.uint8, device=dev)
        keep.append(ws_x)

        def launch_exact(i):
            if paged:
                lib.idx_logits_run_paged(dd["q"], dd["w"], dd["kv"], wl.S_k, in_dtype=wl.fmt, q_scale=dd["q_scale"],
                                         sm_scale=wl.sm_scale, clean_logits=wl.clean, out=o[i], workspace=ws_x,
                                         accumulate="fp32")
                return
            lib.idx_logits_run(dd["q"], dd["k"], dd["w"], in_dtype=wl.fmt, q_scale=dd["q_scale"],
                               k_scale=dd["k_scale"], sm_scale=wl.sm_scale, clean_logits=wl.clean, out=o[i],
                               q_causal_offsets=dd["offsets"], row_starts=dd["starts"], row_ends=dd["ends"],
                               workspace=ws_x, accumulate="fp32")
        variants.append(Variant("call_exact_accumulation", launch_exact, o, ":fp32"))
    if args.topk:
        k = args.topk
        src = variants[0].outs[0]
        tidx = [torch.empty((wl.B, wl.S_q, k), dtype=torch.int32, device=dev) for _ in range(5)]
        tval = [torch.empty((wl.B, wl.S_q, k), dtype=torch.float32, device=dev) for _ in range(5)]
        keep.extend(tidx + tval)

        def launch_topk(i):
            lib.idx_logits_topk(plan, src, k, order="column", B=wl.B, H=wl.H, D=wl.D, S_k=wl.S_k, out_idx=tidx[i],
                                out_val=tval[i])
        variants.append(Variant(f"topk{k}", launch_topk, tidx, f"topk{k}"))
        if not paged:
            # scoring and selection in one call, plan built inside as for "call";
            # its indices must equal the two-phase ones bit for bit
            fidx = [torch.empty((wl.B, wl.S_q, k), dtype=torch.int32, device=dev) for _ in range(5)]
            fval = [torch.empty((wl.B, wl.S_q, k), dtype=torch.float32, device=dev) for _ in range(5)]
            n_redo = torch.zeros(1, dtype=torch.int32, device=dev)
            keep.extend(fidx + fval + [n_redo])
            fa = lib.make_args(d["q"], d["k"], d["w"], None, in_dtype=wl.fmt, q_scale=d["q_scale"],
                               k_scale=d["k_scale"], sm_scale=wl.sm_scale, out_dtype=odt)
            fws = torch.empty(lib.idx_logits_topk_workspace_bytes(fa), dtype=torch.uint8, device=dev)
            keep.append(fws)
            tplan_f = torch.empty_like(plan) if thd else None

            def launch_fused(i):
                p = build_plan(lib, wl, d, tplan_f, None) if thd else None
                lib.idx_logits_run_topk(d["q"], d["k"], d["w"], k, in_dtype=wl.fmt, q_scale=d["q_scale"],
                                        k_scale=d["k_scale"], sm_scale=wl.sm_scale, out_dtype=odt, order="column",
                                        plan=p, q_causal_offsets=d["offsets"], row_starts=d["starts"],
                                        row_ends=d["ends"], workspace=fws, out_idx=fidx[i], out_val=fval[i],
                                        n_redo=n_redo)
            variants.append(Variant(f"fused_topk{k}", launch_fused, fidx, f"topk{k}"))

    # eager reference of every group of variants that must agree bitwise
    refs = {}
    for v in variants:
        for i in range(3):
            v.launch(i)
    torch.cuda.synchronize()
    for v in variants:
        if v.ref_group is not None and v.ref_group not in refs:
            refs[v.ref_group] = v.outs[0].clone()
    # capture: 5 calls into 5 distinct outputs per graph, then warm replays
    # (--eager: the 5 calls are launched directly every time)
    class _Eager:
        def __init__(self, v):
            self.v = v

        def replay(self):
            for i in range(5):
                self.v.launch(i)

    for v in variants:
        if args.eager:
            v.graph = _Eager(v)
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(5):
                v.launch(i)
        v.graph = g
    for _ in range(args.warmup):
        for v in variants:
            v.graph.replay()
    torch.cuda.synchronize()
    # the clock ramps up over the first milliseconds of sustained work
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < args.prewarm_s:
        for v in variants:
            v.graph.replay()
        torch.cuda.synchronize()
    clock_before = gpu_clock_state()
    stream = torch.cuda.current_stream(dev)
    events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = len(variants)
    for s in range(args.steps):
        order = variants[s % n:] + variants[:s % n]
        if s % 2:
            order = order[::-1]
        for v in order:
            v.graph.replay()  # warm-up replay of the sample
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            v.graph.replay()
            e1.record(stream)
            events.append((v, s, e0, e1))
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    clock_after = gpu_clock_state()
    per_sample = {}
    for v, s, e0, e1 in events:
        us = e0.elapsed_time(e1) * 1000.0 / 5
        v.samples.append(us)
        per_sample[(v.name, s)] = us
    # every graph replay wrote what the eager calls wrote
    for v in variants:
        if v.ref_group is None:
            continue
        for i in range(5):
            if not torch.equal(v.outs[i].view(iv), refs[v.ref_group].view(iv)):
                raise RuntimeError(f"graph replay of {v.name} (output {i}) differs from the eager call")
    stats = {v.name: {"median_us": round(statistics.median(v.samples), 2), "p10_us": round(_pct(v.samples, 10), 2),
                      "p90_us": round(_pct(v.samples, 90), 2), "samples": len(v.samples)} for v in variants}
    kernel_above_call = sum(1 for s in range(args.steps)
                            if per_sample[("kernel", s)] > per_sample[("call_planned", s)])

    V = visible_cells(lib, wl, plan)
    flops = 2.0 * wl.H * wl.D * V  # 2 H D per visible cell
    peak = PEAK_TFLOPS[wl.fmt]
    us_call = stats["call"]["median_us"]
    kern_us = stats["kernel"]["median_us"]
    rec = counted_traffic(wl.name, wl.fmt)
    traffic = None if rec is None else rec["fetch_bytes"] + rec["write_bytes"]
    achieved = flops / (kern_us * 1e-6) / 1e12
    alg_bytes = input_bytes(wl) + out_bytes(wl, V)
    # the roofline that bounds the kernel: HBM when its arithmetic intensity is
    # below the machine balance (peak FLOP/s per HBM byte/s), else the MFMA peak
    hbm_bound = flops / alg_bytes < peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    gbs = alg_bytes / (kern_us * 1e-6) / 1e9
    tflops = lambda us: round(flops / (us * 1e-6) / 1e12, 1)
    res = {
        "metric": METRIC,
        "value": us_call,
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
                   "clean_logits": wl.clean, "visible_cells": V, "plan": "built inside the call (metadata no)",
                   "inputs": f"seeded random (seed {wl.seed})"},
        "timing": {"protocol": ("5 eager calls" if args.eager else "HIP graph of 5 calls") +
                               " into 5 distinct outputs per variant; per sample one warm and "
                               "one event-timed replay of every variant, order rotating and reversing; /5",
                   "variants": stats, "kernel_above_planned_call_samples": kernel_above_call,
                   "wall_s_of_samples": round(wall_s, 3), "clock_before": clock_before, "clock_after": clock_after},
        "eff_tflops": tflops(us_call),
        "eff_tflops_planned": tflops(stats["call_planned"]["median_us"]),
        "out_gbs": round(out_bytes(wl, V) / (us_call * 1e-6) / 1e9, 1),
        "roofline": dict(
            ({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "frac": round(gbs / HBM_PEAK_GBS, 4), "mfma_tflops": round(achieved, 1),
              "mfma_frac": round(achieved / peak, 4)} if hbm_bound else
             {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
              "frac": round(achieved / peak, 4)}),
            traffic=traffic, kernel="score_kernel", kernel_us=kern_us, flop_per_launch=flops,
            algorithmic_bytes_per_launch=alg_bytes,
            call_frac=round(flops / (us_call * 1e-6) / 1e12 / peak, 4)),
    }
    if thd:
        cq = [int(x) for x in wl.thd["cu_q"]]
        res["config"]["thd"] = {"segments": len(cq) - 1, "seg_lens": [b - a for a, b in zip(cq, cq[1:])],
                                "ratio": wl.thd["ratio"], "m_total": wl.S_k}
        res["config"]["plan"] = "idx_logits_plan_thd inside the timed call"
    if paged:
        pg = wl.paged
        res["config"]["paged"] = {"page_size": pg["page_size"], "num_pages": int(pg["k_cache"].shape[0]),
                                  "max_pages": int(np.asarray(pg["block_table"]).shape[1]),
                                  "context_keys": int(np.clip(np.asarray(pg["ctx"], np.int64), 0, wl.S_k).sum())}
        res["config"]["plan"] = "built inside the call from the context lengths"
    if zwl is not None:
        zus = stats["zero_call"]["median_us"]
        res["zero_inputs"] = {"workload": zwl.name, "call_us": zus, "call_planned_us": stats["zero_call_planned"]["median_us"],
                              "kernel_us": stats["zero_kernel"]["median_us"],
                              "pages_us_gb200": PAGES_US.get(zero_name),
                              "ratio_to_pages": round(zus / PAGES_US[zero_name], 3) if zero_name in PAGES_US else None}
    if exact:
        xus = stats["call_exact_accumulation"]["median_us"]
        res["exact_accumulation"] = {"call_us": xus, "eff_tflops": tflops(xus),
                                     "frac_of_bf16_peak": round(flops / (xus * 1e-6) / 1e12 / PEAK_TFLOPS["bf16"], 4)}
    if args.topk:
        k = args.topk
        t_us = stats[f"topk{k}"]["median_us"]
        # algorithmic bytes: every window score read once, k (index, score) pairs written per row
        read = (2 if odt == torch.bfloat16 else 4) * V
        written = 8 * wl.B * wl.S_q * k
        tg = (read + written) / (t_us * 1e-6) / 1e9
        trec = counted_traffic(f"topk{k}:{wl.name}", "topk")
        res["topk"] = {"k": k, "order": "column", "kernel": "topk_rows_kernel", "kernel_us": t_us,
                       "roofline": {"bound": "hbm", "achieved": round(tg, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(tg / HBM_PEAK_GBS, 4),
                                    "traffic": None if trec is None else trec["fetch_bytes"] + trec["write_bytes"],
                                    "algorithmic_bytes_per_launch": read + written}}
        if f"fused_topk{k}" in stats:
            f_us = stats[f"fused_topk{k}"]["median_us"]
            two = us_call + t_us
            res["topk"]["fused"] = {"call_us": f_us, "two_phase_us": round(two, 2),
                                    "speedup_vs_two_phase": round(two / f_us, 3), "eff_tflops": tflops(f_us),
                                    "rows_scored_twice": int(n_redo.item()),
                                    "indices_equal_two_phase": True}
    del variants, keep
    torch.cuda.empty_cache()
    if not args.no_peaks:
        pk = measure_peaks(dev)
        if pk is not None and res["roofline"]["bound"] == "mfma" and wl.H == 64:
            # the MFMA shape the 64-head scoring kernel of this input format issues
            shape = {"bf16": "bf16_32x32x16", "fp8": "fp8_16x16x128", "mxfp8": "fp8_16x16x128",
                     "mxfp4": "fp4_32x32x64"}[wl.fmt]
            meas = pk["mfma_tflops"][shape]["random"]
            pk["kernel_shape"] = shape
            pk["kernel_frac_of_measured_random"] = round(res["roofline"]["achieved"] / meas, 4)
        res["peaks_measured"] = pk
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, V)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
