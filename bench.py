#!/usr/bin/env python3
"""Benchmark of the fp16 GEMM D = A·Bᵀ on one MI355X.

One step is one tg_gemm_f16 call over the whole workload (the entire hot
path: operand loads, LDS staging, MFMA contraction, epilogue).  Default
workload: the 8192×14336×4096 linear-layer shape with A ~ N(0,1) and
B ~ N(0,1/K), seeded and synthetic, resident in HBM before timing starts.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--all]
                    [--dtype f16|bf16|mxf8]

--dtype bf16 times tg_gemm_bf16 on the same draws; --dtype mxf8 times the
block-scaled FP8 GEMM on the same draws encoded as E4M3 codes with one UE8M0
scale per 32 K elements (peak: the dense fp8 rate): by default
tg_gemm_mxf8_packed, with the scales converted once into the packed layout
(tg_mx_pack_scales) before the timed region, as a caller does for a weight's
fixed scales; --mx-scales rowmajor times tg_gemm_mxf8 on row-major scales.

Prints ONE JSON line on stdout.  Timing: W untimed calls, a device
synchronize, then K calls bracketed by HIP events recorded on the stream the
kernel is launched on (torch's current stream), then a synchronize.  With
--records R the K-call window is timed R times and the median window is
reported (all R in records_ms_per_step); --per-call adds a separate pass of K
calls with an event between consecutive calls and reports their median, min
and quartiles.  Two
operand/output sets alternate between calls so consecutive launches do not
find their operands in the last-level cache from the previous call.

The CPU baseline is the oracle (plain C, fp64) timed on a bounded sample of
the same workload — a prefix of D's rows, all columns, full K — on every
host core this process may use.
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

PEAK_FP16_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA (the block-scaled entry point)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
KERNEL_SOURCES = [os.path.join(ROOT, "dense_fp16_gemm_02_amd", "csrc", f)
                  for f in ("tg_gemm.hip", "tile_layout.hpp")]
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _code_text(src: str) -> str:
    """C++ source with comments, blank lines and indentation removed: what the
    compiler sees, so an edit to a comment or to layout keeps a traffic record."""
    out, i, n = [], 0, len(src)
    quote = None
    while i < n:
        c = src[i]
        if quote:
            out.append(c)
            if c == "\\" and i + 1 < n:
                out.append(src[i + 1])
                i += 2
                continue
            if c == quote:
                quote = None
            i += 1
        elif c in "\"'":
            quote = c
            out.append(c)
            i += 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (line.strip() for line in "".join(out).split("\n"))
    return "\n".join(line for line in lines if line)


def kernel_source_digest() -> str:
    """SHA-256 of the kernel sources' code (comments ignored)."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(_code_text(f.read()).encode())
    return h.hexdigest()


def _pmc_per_dispatch(csv_path: str, counter: str, name_part: str):
    """Mean value of `counter` over the dispatches whose kernel name contains
    `name_part` in a rocprofv3 --pmc counter_collection.csv."""
    import csv
    import collections

    per = collections.defaultdict(float)
    for row in csv.DictReader(open(csv_path)):
        if row["Counter_Name"] == counter and name_part in row["Kernel_Name"]:
            per[row["Dispatch_Id"]] += float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {name_part!r} in {csv_path}")
    vals = list(per.values())
    return sum(vals) / len(vals), len(vals)


def traffic_record(args) -> int:
    """Turn four rocprofv3 --pmc runs (GEMM FETCH_SIZE, GEMM WRITE_SIZE, copy
    FETCH_SIZE, copy WRITE_SIZE) into profiles/<kernel>__<workload>__traffic.json.
    Each GEMM counter is scaled by (known copy bytes / the same counter for
    the copy kernel)."""
    gf, gw, cf, cw = args.traffic_record
    copy_bytes = args.copy_bytes
    kernel, workload = args.traffic_kernel, args.workload
    g_fetch, n1 = _pmc_per_dispatch(gf, "FETCH_SIZE", "gemm_")
    g_write, n2 = _pmc_per_dispatch(gw, "WRITE_SIZE", "gemm_")
    c_fetch, _ = _pmc_per_dispatch(cf, "FETCH_SIZE", "copyBuffer")
    c_write, _ = _pmc_per_dispatch(cw, "WRITE_SIZE", "copyBuffer")
    k_fetch = copy_bytes / c_fetch  # bytes per counter unit (nominally 1024: KiB)
    k_write = copy_bytes / c_write
    rec = {
        "kernel": kernel,
        "workload": workload,
        "kernel_source_sha256": kernel_source_digest(),
        "fetch_counter_per_dispatch": g_fetch,
        "write_counter_per_dispatch": g_write,
        "dispatches": [n1, n2],
        "copy_bytes": copy_bytes,
        "copy_fetch_counter": c_fetch,
        "copy_write_counter": c_write,
        "bytes_per_fetch_unit": k_fetch,
        "bytes_per_write_unit": k_write,
        "hbm_read_bytes_per_launch": g_fetch * k_fetch,
        "hbm_write_bytes_per_launch": g_write * k_write,
        "hbm_bytes_per_launch": g_fetch * k_fetch + g_write * k_write,
    }
    path = os.path.join(PROFILES, f"{kernel}__{workload}__traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))
    return 0


def trace_summary(csv_path: str, name_part: str, window=None) -> dict:
    """Per-dispatch durations of the kernels whose name contains `name_part`
    in a rocprofv3 --kernel-trace kernel_trace.csv, in dispatch order, with
    their mean over the call window [lo, hi) when given (the timed calls of a
    bench run: calls warmup .. warmup+steps-1)."""
    import csv

    rows = [r for r in csv.DictReader(open(csv_path)) if name_part in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    us = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    out = {"kernel": rows[0]["Kernel_Name"] if rows else None, "calls": len(us), "per_call_us": us}
    if us:
        out["mean_us"] = sum(us) / len(us)
    if window and us:
        lo, hi = window
        sel = us[lo:hi]
        out["window"] = [lo, hi]
        out["window_mean_us"] = sum(sel) / len(sel) if sel else None
    return out


def copy_only(nbytes: int, reps: int = 5) -> int:
    """A plain device-to-device copy of `nbytes` (the calibration kernel)."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {nbytes} bytes x {reps}", file=sys.stderr)
    return 0


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary for
    this kernel and workload, or None when there is none or the kernel
    source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}__{workload}__traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def _timed(step, steps: int, warmup: int, records: int, per_call: bool, dev, stream) -> dict:
    """W untimed calls, then `records` windows of K calls, each bracketed by
    two HIP events on the launch stream (a window's mean is one record; the
    default is one window, i.e. exactly K timed calls); with `per_call`, one
    more pass of K calls with an event between consecutive calls for the
    per-call distribution (kept out of the windows: the extra events would
    sit between the launches being timed)."""
    import statistics

    import torch

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize(dev)
    means = []
    t0 = time.perf_counter()
    for r in range(records):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(steps):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize(dev)
        means.append(ev0.elapsed_time(ev1) / steps)
    wall = time.perf_counter() - t0
    out = dict(ms=statistics.median(means), records_ms=means, wall_s=wall, per_call_us=None)
    if per_call:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(stream)
        for i in range(steps):
            step(i)
            evs[i + 1].record(stream)
        torch.cuda.synchronize(dev)
        per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps))
        q = statistics.quantiles(per, n=4) if steps >= 2 else [per[0]] * 3
        out["per_call_us"] = {"median": round(statistics.median(per), 3), "min": round(per[0], 3),
                              "p25": round(q[0], 3), "p75": round(q[2], 3)}
    return out


def time_workload(w, steps: int, warmup: int, rotate: int = 2, vendor: bool = False,
                  dtype: str = "f16", records: int = 1, per_call: bool = False, mx_scales: str = "packed",
                  mx_formats=("e4m3", "e4m3")):
    import numpy as np
    import torch

    import dense_fp16_gemm_02_amd as tg
    import workloads

    dev = torch.device("cuda:0")
    if dtype == "mxf8":
        return _time_mx(w, steps, warmup, rotate, records, per_call, mx_scales, mx_formats)
    a, b = workloads.make_inputs(w, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    A0 = torch.from_numpy(a.view(np.int16)).to(dev).view(tdt)
    B0 = torch.from_numpy(b.view(np.int16)).to(dev).view(tdt)
    sets = []
    for r in range(rotate):
        A = A0 if r == 0 else A0.clone()
        B = B0 if r == 0 else B0.clone()
        D = torch.empty((w.M, w.N), dtype=tdt, device=dev)
        sets.append((A, B, D))
    stream = torch.cuda.current_stream(dev)
    plan = tg.tg_gemm_bf16_plan if dtype == "bf16" else tg.tg_gemm_f16_plan
    call = tg.tg_gemm_bf16 if dtype == "bf16" else tg.tg_gemm_f16
    st, kname, tiles = plan(A0, B0, sets[0][2], w.M, w.N, w.K, w.K, w.K, w.N)
    if st != tg.TG_OK:
        raise RuntimeError(tg.tg_status_string(st))

    def step(i):
        A, B, D = sets[i % rotate]
        if vendor:  # context only: the vendor library on the same inputs
            torch.matmul(A, B.t(), out=D)
            return
        s = call(A, B, D, w.M, w.N, w.K, w.K, w.K, w.N, stream)
        if s != tg.TG_OK:
            raise RuntimeError(f"{call.__name__}: {tg.tg_status_string(s)}")

    t = _timed(step, steps, warmup, records, per_call, dev, stream)
    del sets, A0, B0
    torch.cuda.empty_cache()
    return dict(t, kernel=kname, tiles=tiles, a=a, b=b)


def _time_mx(w, steps: int, warmup: int, rotate: int, records: int = 1, per_call: bool = False,
             scales: str = "packed", formats=("e4m3", "e4m3")):
    """time_workload for the block-scaled FP8 entry points (packed or
    row-major scales; element encodings ``formats`` of A and B: E4M3 on both
    times tg_gemm_mxf8(_packed), any other pair tg_gemm_mx(_packed))."""
    import torch

    import dense_fp16_gemm_02_amd as tg
    import workloads

    if w.K % 32:
        raise RuntimeError(f"{w.name}: K = {w.K} is not whole 32-element scale blocks")
    dev = torch.device("cuda:0")
    qa, sa, qb, sb = workloads.make_mx_inputs(w, *formats)
    fa, fb = (tg.TG_MX_E5M2 if f == "e5m2" else tg.TG_MX_E4M3 for f in formats)
    nb = w.K // 32
    lds = (nb + 3) // 4 * 4  # scale rows padded to whole 4-byte words (the entry point's rule)
    host = [torch.from_numpy(x) for x in (qa, workloads.pad_bytes(sa, lds, 127), qb,
                                          workloads.pad_bytes(sb, lds, 127))]
    sets = []
    for r in range(rotate):
        sets.append(tuple(x.to(dev) for x in host) + (torch.empty((w.M, w.N), dtype=torch.float16, device=dev),))
    stream = torch.cuda.current_stream(dev)
    if scales == "packed":
        packed = []
        for A, SA, B, SB, D in sets:
            PA = torch.empty(tg.tg_mx_packed_bytes(w.M, w.K), dtype=torch.uint8, device=dev)
            PB = torch.empty(tg.tg_mx_packed_bytes(w.N, w.K), dtype=torch.uint8, device=dev)
            for S, rows, P in ((SA, w.M, PA), (SB, w.N, PB)):
                st = tg.tg_mx_pack_scales(S, rows, w.K, lds, P, stream)
                if st != tg.TG_OK:
                    raise RuntimeError(f"tg_mx_pack_scales: {tg.tg_status_string(st)}")
            packed.append((A, PA, B, PB, D))
        sets = packed
        torch.cuda.synchronize(dev)
        if fa == fb == tg.TG_MX_E4M3:
            st, kname, tiles = tg.tg_gemm_mxf8_packed_plan(*sets[0], w.M, w.N, w.K, w.K, w.K, w.N)

            def call(i):
                return tg.tg_gemm_mxf8_packed(*sets[i % rotate], w.M, w.N, w.K, w.K, w.K, w.N, stream)
        else:
            st, kname, tiles = tg.tg_gemm_mx_packed_plan(*sets[0], w.M, w.N, w.K, w.K, w.K, w.N, fa, fb)

            def call(i):
                return tg.tg_gemm_mx_packed(*sets[i % rotate], w.M, w.N, w.K, w.K, w.K, w.N, fa, fb, stream)
    else:
        if fa == fb == tg.TG_MX_E4M3:
            st, kname, tiles = tg.tg_gemm_mxf8_plan(*sets[0], w.M, w.N, w.K, w.K, lds, w.K, lds, w.N)

            def call(i):
                return tg.tg_gemm_mxf8(*sets[i % rotate], w.M, w.N, w.K, w.K, lds, w.K, lds, w.N, stream)
        else:
            st, kname, tiles = tg.tg_gemm_mx_plan(*sets[0], w.M, w.N, w.K, w.K, lds, w.K, lds, w.N, fa, fb)

            def call(i):
                return tg.tg_gemm_mx(*sets[i % rotate], w.M, w.N, w.K, w.K, lds, w.K, lds, w.N, fa, fb, stream)
    if st != tg.TG_OK:
        raise RuntimeError(tg.tg_status_string(st))

    def step(i):
        s = call(i)
        if s != tg.TG_OK:
            raise RuntimeError(f"{kname}: {tg.tg_status_string(s)}")

    t = _timed(step, steps, warmup, records, per_call, dev, stream)
    del sets
    torch.cuda.empty_cache()
    return dict(t, kernel=kname, tiles=tiles, a=(qa, sa), b=(qb, sb))


def cpu_baseline(w, a, b, seconds: float, rows_override=None, fmt: str = "f16", mx_formats=("e4m3", "e4m3")):
    """Time the oracle on the first R rows of D (all N columns, full K)."""
    import numpy as np

    import oracle

    def ref(rows, threads):
        if fmt == "mxf8":
            return oracle.gemm_mx(a[0], a[1], b[0], b[1], w.M, w.N, w.K, rows=rows, nthreads=threads,
                                  a_fmt=mx_formats[0], b_fmt=mx_formats[1])
        return oracle.gemm(a, b, w.M, w.N, w.K, rows=rows, nthreads=threads, fmt=fmt)

    threads = oracle.default_threads()
    if rows_override:
        R = min(rows_override, w.M)
    else:
        probe = min(max(1, threads), w.M)
        t0 = time.perf_counter()
        ref(np.arange(probe), threads)
        per_row = (time.perf_counter() - t0) / probe
        R = int(min(w.M, max(threads, seconds / max(per_row, 1e-9))))
        R = max(threads, (R // threads) * threads) if R >= threads else R
    rows = np.arange(R, dtype=np.int64)
    t0 = time.perf_counter()
    ref(rows, threads)
    t = time.perf_counter() - t0
    flop = 2.0 * R * w.N * w.K
    return {
        "value": flop / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"rows 0..{R - 1} of D ({R} of {w.M} rows, all {w.N} columns, K={w.K}); "
                  f"{t:.2f} s wall",
    }


def mfma_ceiling(w, args) -> int:
    """Time tg_mfma_ceiling (a stream of independent MFMAs on register
    operands, no memory traffic) with the same protocol as the GEMM, for
    each instruction the GEMM kernels use: the operand registers loaded from
    the workload's own A and B (its value distribution: fp16, the same draws
    rounded to bf16, or their block-scaled e4m3 codes), and from zeros (no
    toggling, so no power limit).  Prints one JSON line with TFLOP/s per
    instruction and operand set."""
    import numpy as np
    import torch

    import dense_fp16_gemm_02_amd as tg
    import workloads

    dev = torch.device("cuda:0")

    def upload(x):
        return torch.from_numpy(np.ascontiguousarray(x).reshape(-1).view(np.uint8)).to(dev)

    a, b = workloads.make_inputs(w)
    ops = {"f16": (upload(a), upload(b))}
    del a, b
    a, b = workloads.make_inputs(w, dtype="bf16")
    ops["bf16"] = (upload(a), upload(b))
    del a, b
    qa, _, qb, _ = workloads.make_mx_inputs(w)
    ops["e4m3"] = (upload(qa), upload(qb))
    del qa, qb
    Z = torch.zeros(1 << 17, dtype=torch.uint8, device=dev)
    st, cus, clk_khz, arch = tg.tg_device_info()
    if st != tg.TG_OK:
        raise RuntimeError(tg.tg_status_string(st))
    out = torch.empty(cus * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    iters = args.ceiling_iters
    # (code, name, operand type, bytes per element, flop per wave-iteration, peak)
    shapes = [(tg.TG_MFMA_F16_16X16X32, "mfma_16x16x32_f16", "f16", 2, 1 << 20, PEAK_FP16_TFLOPS),
              (tg.TG_MFMA_F16_32X32X16, "mfma_32x32x16_f16", "f16", 2, 1 << 20, PEAK_FP16_TFLOPS),
              (tg.TG_MFMA_BF16_16X16X32, "mfma_16x16x32_bf16", "bf16", 2, 1 << 20, PEAK_FP16_TFLOPS),
              (tg.TG_MFMA_MXF8_32X32X64, "mfma_scale_32x32x64_e4m3", "e4m3", 1, 1 << 21, PEAK_FP8_TFLOPS)]
    results = {}
    for code, base, kind, esize, per_iter, peak in shapes:
        if args.ceiling_shapes and base not in args.ceiling_shapes.split(","):
            continue
        flop = cus * 4 * iters * float(per_iter)
        for label, (x, y) in (("workload", ops[kind]), ("zeros", (Z, Z))):
            def step(i, x=x, y=y, code=code, esize=esize):
                s = tg.tg_mfma_ceiling(code, x, x.numel() // esize, y, y.numel() // esize, 1, iters, cus, out,
                                       stream)
                if s != tg.TG_OK:
                    raise RuntimeError(f"tg_mfma_ceiling: {tg.tg_status_string(s)}")

            t = _timed(step, args.steps, args.warmup, max(1, args.records), args.per_call, dev, stream)
            tf = flop / (t["ms"] * 1e-3) / 1e12
            name = f"{base}_{label}"
            results[name] = {"ms_per_launch": round(t["ms"], 6), "tflops": round(tf, 1), "peak": peak,
                             "frac_of_peak": round(tf / peak, 4)}
            log(f"{name:40s} {t['ms'] * 1e3:9.2f} us/launch {tf:8.1f} TFLOP/s "
                f"({100 * tf / peak:.1f}% of {peak:.0f})")
    line = {"metric": "TFLOP/s of a matrix-core stream with no memory traffic (tg_mfma_ceiling)",
            "unit": "TFLOP/s", "workload_operands": w.name, "workgroups": cus, "iters": iters,
            "steps": args.steps, "warmup": args.warmup,
            "device": {"arch": arch, "compute_units": cus, "max_sclk_mhz": clk_khz / 1000},
            "results": results}
    print(json.dumps(line), flush=True)
    return 0


def hbm_ceiling(args, nbytes: int = 1 << 30) -> int:
    """Time tg_hbm_read_ceiling (every byte of a buffer read once with
    16-byte loads) with the GEMM's protocol, alternating two 1 GiB buffers so
    the last-level cache (256 MB) cannot serve a call from the previous one;
    for several workgroup counts.  Prints one JSON line with GB/s each."""
    import torch

    import dense_fp16_gemm_02_amd as tg

    dev = torch.device("cuda:0")
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(2)]
    st, cus, clk_khz, arch = tg.tg_device_info()
    if st != tg.TG_OK:
        raise RuntimeError(tg.tg_status_string(st))
    stream = torch.cuda.current_stream(dev)
    results = {}
    for per_cu in (4, 8, 16):
        wg = cus * per_cu
        out = torch.empty(wg * 256, dtype=torch.int32, device=dev)

        def step(i, wg=wg, out=out):
            s = tg.tg_hbm_read_ceiling(bufs[i % 2], nbytes, wg, out, stream)
            if s != tg.TG_OK:
                raise RuntimeError(f"tg_hbm_read_ceiling: {tg.tg_status_string(s)}")

        t = _timed(step, args.steps, args.warmup, max(1, args.records), args.per_call, dev, stream)
        gbs = nbytes / (t["ms"] * 1e-3) / 1e9
        results[f"read_{per_cu}wg_per_cu"] = {"ms_per_launch": round(t["ms"], 6), "gbs": round(gbs, 1),
                                               "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"streaming read, {wg} workgroups: {t['ms'] * 1e3:9.2f} us per GiB  {gbs:8.1f} GB/s "
            f"({100 * gbs / PEAK_HBM_GBS:.1f}% of {PEAK_HBM_GBS:.0f})")
    line = {"metric": "GB/s of a streaming HBM read (tg_hbm_read_ceiling)", "unit": "GB/s", "bytes": nbytes,
            "steps": args.steps, "warmup": args.warmup, "peak": PEAK_HBM_GBS,
            "device": {"arch": arch, "compute_units": cus, "max_sclk_mhz": clk_khz / 1000},
            "results": results}
    print(json.dumps(line), flush=True)
    return 0


def xcd_times(w, args) -> int:
    """W untimed calls of tg_gemm_f16, then K calls through its stamping form
    (tg_gemm_f16_xcd_stamps: the persistent kernel recording each
    workgroup's start, end and XCD), each into its own slice of one stamps
    buffer, with no synchronization between the calls.  Per call, each XCD's
    end is its last workgroup's end, measured from the call's first start on
    the constant 100 MHz clock; the launch ends with the slowest XCD.  Prints
    one JSON line: per-XCD mean ends, the mean span, and the share of the span
    after the mean XCD end (the time one XCD finishing late costs)."""
    import numpy as np
    import torch

    import dense_fp16_gemm_02_amd as tg
    import workloads

    dev = torch.device("cuda:0")
    a, b = workloads.make_inputs(w)
    A0 = torch.from_numpy(a.view(np.int16)).to(dev).view(torch.float16)
    B0 = torch.from_numpy(b.view(np.int16)).to(dev).view(torch.float16)
    sets = [(A0 if r == 0 else A0.clone(), B0 if r == 0 else B0.clone(),
             torch.empty((w.M, w.N), dtype=torch.float16, device=dev)) for r in range(2)]
    stream = torch.cuda.current_stream(dev)
    st, kname, tiles = tg.tg_gemm_f16_plan(A0, B0, sets[0][2], w.M, w.N, w.K, w.K, w.K, w.N)
    if st != tg.TG_OK or not kname.endswith("_pers_dma"):
        print(f"bench.py --xcd-times: {w.name} does not plan to the persistent kernel ({kname})", file=sys.stderr)
        return 2
    _, cus, _, arch = tg.tg_device_info()
    per_call = 3 * max(cus, 8)
    stamps = torch.full((args.steps * per_call,), -1, dtype=torch.int64, device=dev)
    for i in range(args.warmup):
        A, B, D = sets[i % 2]
        if tg.tg_gemm_f16(A, B, D, w.M, w.N, w.K, w.K, w.K, w.N, stream) != tg.TG_OK:
            raise RuntimeError("tg_gemm_f16 failed")
    wgs = set()
    for i in range(args.steps):
        A, B, D = sets[i % 2]
        st, wg = tg.tg_gemm_f16_xcd_stamps(A, B, D, w.M, w.N, w.K, w.K, w.K, w.N,
                                           stamps.data_ptr() + 8 * i * per_call, per_call, stream)
        if st != tg.TG_OK:
            raise RuntimeError(f"tg_gemm_f16_xcd_stamps: {tg.tg_status_string(st)}")
        wgs.add(wg)
    torch.cuda.synchronize(dev)
    if len(wgs) != 1:
        raise RuntimeError(f"workgroup counts differ between calls: {sorted(wgs)}")
    wg = wgs.pop()
    s = stamps.view(args.steps, per_call)[:, :3 * wg].reshape(args.steps, wg, 3).cpu().numpy()
    start, end, xcc = s[:, :, 0], s[:, :, 1], s[:, :, 2]
    if (end < start).any() or (xcc < 0).any() or (xcc >= 8).any():
        raise RuntimeError("stamps out of range")
    t0 = start.min(axis=1, keepdims=True)
    ends_us = (end - t0) / 100.0  # 100 MHz clock
    xcd_end = np.stack([np.where(xcc == x, ends_us, -np.inf).max(axis=1) for x in range(8)], axis=1)
    wg_per_xcd = [int((xcc[0] == x).sum()) for x in range(8)]
    span = xcd_end.max(axis=1)
    mean_end = xcd_end.mean(axis=1)
    late = (span - mean_end) / span
    slowest = np.bincount(xcd_end.argmax(axis=1), minlength=8)
    line = {"metric": "per-XCD end of the persistent fp16 GEMM (tg_gemm_f16_xcd_stamps)", "unit": "us",
            "workload": w.name, "kernel": kname, "tiles": tiles, "workgroups": wg, "workgroups_per_xcd": wg_per_xcd,
            "steps": args.steps, "warmup": args.warmup,
            "xcd_mean_end_us": [round(float(v), 1) for v in xcd_end.mean(axis=0)],
            "mean_span_us": round(float(span.mean()), 1), "mean_xcd_end_us": round(float(mean_end.mean()), 1),
            "late_share": round(float(late.mean()), 4), "slowest_xcd_counts": [int(v) for v in slowest],
            "workgroup_w_on_xcd_w_mod_8": bool(np.all(xcc == np.arange(wg) % 8)),
            "wg_end_spread_within_xcd_us": round(float(np.mean([
                (np.where(xcc == x, ends_us, -np.inf).max(axis=1) - np.where(xcc == x, ends_us, np.inf).min(axis=1)).mean()
                for x in range(8)])), 1),
            "device": {"arch": arch, "compute_units": cus}}
    log(f"{w.name} {kname}: span {line['mean_span_us']} us, mean XCD end {line['mean_xcd_end_us']} us, "
        f"late share {100 * line['late_share']:.1f}%, XCD ends {line['xcd_mean_end_us']}")
    print(json.dumps(line), flush=True)
    return 0


def algorithmic_bytes(w, dtype: str) -> int:
    """Compulsory HBM bytes of one call: A and B read once, D (fp16) written once;
    the block-scaled entry point reads 1-byte codes plus one scale byte per 32 K
    elements of each row."""
    if dtype == "mxf8":
        return (w.M * w.K + w.N * w.K) + 2 * w.M * w.N + (w.M + w.N) * (w.K // 32)
    return w.min_bytes


def run_processes(args) -> int:
    """--processes P: run this benchmark line in P independent processes
    (each its own warm-up and timed calls) and report the median process
    with every process's time beside it.  The CPU baseline, if asked for,
    runs in the last process only."""
    import subprocess
    import statistics

    argv = [a for a in sys.argv[1:]]
    i = argv.index("--processes") if "--processes" in argv else -1
    if i >= 0:
        del argv[i:i + 2]
    argv = [a for a in argv if not a.startswith("--processes=")]
    lines = []
    for p in range(args.processes):
        extra = [] if p == args.processes - 1 else ["--no-cpu-baseline"]
        out = subprocess.run([sys.executable, os.path.abspath(__file__), *argv, *extra],
                             stdout=subprocess.PIPE, text=True)
        if out.returncode != 0:
            return out.returncode
        lines.append(json.loads(out.stdout.strip().splitlines()[-1]))
        log(f"process {p}: {lines[-1]['ms_per_step'] * 1e3:.2f} us per step")
    order = sorted(range(len(lines)), key=lambda k: lines[k]["ms_per_step"])
    line = dict(lines[order[len(order) // 2]])
    line["cpu_baseline"] = lines[-1].get("cpu_baseline")
    line["processes_ms_per_step"] = [round(x["ms_per_step"], 6) for x in lines]
    line["processes"] = args.processes
    log(f"median of {args.processes} processes: {statistics.median(x['ms_per_step'] for x in lines) * 1e3:.2f} us")
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--records", type=int, default=1,
                    help="timed windows of --steps calls; the reported time is their median")
    ap.add_argument("--per-call", action="store_true",
                    help="also time --steps calls one by one (median, min, quartiles)")
    ap.add_argument("--workload", default="linear_8192x14336x4096")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="target length of the oracle sample")
    ap.add_argument("--cpu-rows", type=int, default=None, help="fixed oracle sample size in rows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-cpu-seconds", type=float, default=6.0,
                    help="with --all: length of each workload's oracle sample")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time the matrix-core stream (tg_mfma_ceiling) on the workload's A and B "
                         "and on zeros, for both MFMA shapes; one JSON line")
    ap.add_argument("--xcd-times", action="store_true",
                    help="per-XCD end times of the persistent fp16 kernel on --workload (measurement only)")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="only time a streaming read of HBM (tg_hbm_read_ceiling) over two alternating "
                         "1 GiB buffers; one JSON line")
    ap.add_argument("--ceiling-shapes", default="",
                    help="with --mfma-ceiling: comma-separated subset of mfma_16x16x32_f16, "
                         "mfma_32x32x16_f16, mfma_16x16x32_bf16, mfma_scale_32x32x64_e4m3 (default all)")
    ap.add_argument("--ceiling-iters", type=int, default=1024,
                    help="loop iterations per ceiling launch (2^20 flop per wave each)")
    ap.add_argument("--all", action="store_true",
                    help="also time every workload and print a table on stderr")
    ap.add_argument("--processes", type=int, default=1,
                    help="run the line in P independent processes and report the median process "
                         "(not with --all)")
    ap.add_argument("--mx-scales", choices=["packed", "rowmajor"], default="packed",
                    help="with --dtype mxf8: the scale layout (packed: tg_gemm_mxf8_packed on scales packed once "
                         "before timing; rowmajor: tg_gemm_mxf8)")
    ap.add_argument("--mx-formats", choices=["e4m3,e4m3", "e5m2,e5m2", "e5m2,e4m3", "e4m3,e5m2"],
                    default="e4m3,e4m3",
                    help="with --dtype mxf8: the element encodings of A and B (OCP MX FP8: E4M3 or E5M2; "
                         "anything but E4M3 on both times tg_gemm_mx / tg_gemm_mx_packed)")
    ap.add_argument("--dtype", choices=["f16", "bf16", "mxf8"], default="f16",
                    help="element type (the headline metric is fp16; bf16 and block-scaled FP8 "
                         "are reported alongside)")
    ap.add_argument("--vendor", action="store_true",
                    help="with --all: also time torch.matmul on the same inputs (context); without "
                         "--all: the line times torch.matmul instead of this library (context only, "
                         "config.kernel says so)")
    ap.add_argument("--copy-bytes", type=int, default=None,
                    help="only run a plain device copy of this many bytes (counter calibration)")
    ap.add_argument("--traffic-record", nargs=4, metavar="CSV", default=None,
                    help="GEMM FETCH_SIZE, GEMM WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE "
                         "counter_collection.csv files -> profiles/*__traffic.json")
    ap.add_argument("--traffic-kernel", default=None, help="kernel name for --traffic-record")
    ap.add_argument("--trace-summary", metavar="CSV", default=None,
                    help="print the per-call durations of the GEMM dispatches in a rocprofv3 "
                         "kernel_trace.csv (with --steps/--warmup: the mean over the timed calls)")
    ap.add_argument("--trace-kernel", default="gemm_", help="kernel name part for --trace-summary")
    args = ap.parse_args()

    if args.trace_summary:
        t = trace_summary(args.trace_summary, args.trace_kernel, (args.warmup, args.warmup + args.steps))
        print(json.dumps(t))
        return 0

    if args.traffic_record:
        if not args.copy_bytes or not args.traffic_kernel:
            print("--traffic-record needs --copy-bytes and --traffic-kernel", file=sys.stderr)
            return 2
        return traffic_record(args)

    if args.processes > 1:
        if args.all or args.mfma_ceiling or args.hbm_ceiling or args.xcd_times or args.copy_bytes:
            print("--processes applies to the single benchmark line only", file=sys.stderr)
            return 2
        return run_processes(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this GEMM runs on one GPU; multi-GPU runs are not part of this "
              f"build (asked for --gpus {args.gpus}, WORLD_SIZE={world})", file=sys.stderr)
        return 2

    import torch

    import workloads

    if args.copy_bytes and not args.traffic_record:
        return copy_only(args.copy_bytes)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    w = workloads.BY_NAME[args.workload]
    mx_formats = tuple(args.mx_formats.split(","))
    mx_elem = "E4M3" if mx_formats == ("e4m3", "e4m3") else "×".join(f.upper() for f in mx_formats)

    if args.mfma_ceiling:
        return mfma_ceiling(w, args)
    if args.hbm_ceiling:
        return hbm_ceiling(args)
    if args.xcd_times:
        return xcd_times(w, args)

    if args.all:
        pk = PEAK_FP8_TFLOPS if args.dtype == "mxf8" else PEAK_FP16_TFLOPS
        log(f"{'workload':28s} {'kernel':32s} {'us':>9s} {'TFLOP/s':>9s} {'%peak':>7s} {'GB/s':>8s}")
        for ww in workloads.WORKLOADS:
            if args.dtype == "mxf8" and ww.K % 32:
                log(f"{ww.name:28s} (skipped: K is not whole 32-element scale blocks)")
                continue
            r = time_workload(ww, args.steps, args.warmup, dtype=args.dtype, records=max(1, args.records),
                              per_call=args.per_call, mx_scales=args.mx_scales, mx_formats=mx_formats)
            tf = ww.flop / (r["ms"] * 1e-3) / 1e12
            gbs = algorithmic_bytes(ww, args.dtype) / (r["ms"] * 1e-3) / 1e9
            pc = r["per_call_us"]
            cpu_txt = ""
            if not args.no_cpu_baseline:
                c = cpu_baseline(ww, r["a"], r["b"], min(args.cpu_seconds, args.all_cpu_seconds), None,
                                 args.dtype)
                cpu_txt = f"  oracle {c['value'] * 1e3:.2f} GFLOP/s on {c['cores']} threads ({c['sample']})"
            log(f"{ww.name:28s} {r['kernel']:32s} {r['ms'] * 1e3:9.2f} {tf:9.1f} "
                f"{100 * tf / pk:7.2f} {gbs:8.0f}"
                + (f"  per call: median {pc['median']:.2f} min {pc['min']:.2f} "
                   f"IQR {pc['p25']:.2f}-{pc['p75']:.2f} us" if pc else "") + cpu_txt)
            if args.vendor and args.dtype != "mxf8":
                v = time_workload(ww, args.steps, args.warmup, vendor=True, dtype=args.dtype,
                                  records=max(1, args.records))
                tfv = ww.flop / (v["ms"] * 1e-3) / 1e12
                log(f"{'':28s} {'torch.matmul':32s} {v['ms'] * 1e3:9.2f} {tfv:9.1f} "
                    f"{100 * tfv / PEAK_FP16_TFLOPS:7.2f} {ww.min_bytes / (v['ms'] * 1e-3) / 1e9:8.0f}")

    vendor_line = args.vendor and not args.all and args.dtype != "mxf8"
    r = time_workload(w, args.steps, args.warmup, dtype=args.dtype, records=max(1, args.records),
                      per_call=args.per_call, vendor=vendor_line, mx_scales=args.mx_scales,
                      mx_formats=mx_formats)
    if vendor_line:
        r["kernel"] = "torch.matmul (vendor library; context only)"
    ms = r["ms"]
    tflops = w.flop / (ms * 1e-3) / 1e12
    peak = PEAK_FP8_TFLOPS if args.dtype == "mxf8" else PEAK_FP16_TFLOPS
    log(f"{w.name}: {r['kernel']} tiles={r['tiles']} {ms * 1e3:.2f} us/launch "
        f"{tflops:.1f} TFLOP/s ({100 * tflops / peak:.1f}% of peak)")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, r["a"], r["b"], args.cpu_seconds, args.cpu_rows, args.dtype, mx_formats)
        log(f"cpu baseline: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads; {cpu['sample']}")

    traffic = measured_traffic(r["kernel"], w.name)
    shape = f"{w.M}x{w.N}x{w.K}"
    metric = {
        "f16": f"TFLOP/s fp16 GEMM D=A·B^T at {shape}; % of MFMA dense fp16 peak",
        "bf16": f"TFLOP/s bf16 GEMM D=A·B^T at {shape}; % of MFMA dense bf16 peak",
        "mxf8": f"TFLOP/s block-scaled FP8 GEMM D=(SA·A)·(SB·B)^T ({mx_elem}, UE8M0 per 32 K) at {shape}; "
                f"% of MFMA dense fp8 peak",
    }[args.dtype]
    # a contraction below the ridge point is bounded by HBM, not the matrix cores
    alg_bytes = algorithmic_bytes(w, args.dtype)
    hbm_bound = w.flop / alg_bytes < peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    if hbm_bound:
        gbs = alg_bytes / (ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic}
    else:
        roofline = {"bound": "mfma", "achieved": round(tflops, 3), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(tflops / peak, 4), "traffic": traffic}
    line = {
        "metric": metric,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "kernel": r["kernel"],
                   "tiles": r["tiles"], "pct_of_peak": round(100 * tflops / peak, 2),
                   **({"mx_scales": args.mx_scales} if args.dtype == "mxf8" else {}),
                   **({"mx_formats": args.mx_formats} if args.dtype == "mxf8" and mx_formats != ("e4m3", "e4m3")
                      else {})},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    import dense_fp16_gemm_02_amd as tg
    st, cus, clk_khz, arch = tg.tg_device_info()
    if st == tg.TG_OK:
        # dense matrix-core flop per clock per CU: 4096 for fp16/bf16 (2.5 PFLOP/s
        # = 256 CUs × 4096 × 2.4 GHz), twice that for fp8
        per_clk = 8192 if args.dtype == "mxf8" else 4096
        line["device"] = {"arch": arch, "compute_units": cus, "max_sclk_mhz": clk_khz / 1000,
                          "derived_peak_tflops": round(cus * per_clk * clk_khz * 1e3 / 1e12, 1)}
    if len(r["records_ms"]) > 1:
        line["records_ms_per_step"] = [round(x, 6) for x in r["records_ms"]]
    if r["per_call_us"]:
        line["per_call_us"] = r["per_call_us"]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
