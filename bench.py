#!/usr/bin/env python3
"""Benchmark of the Stream-K GEMM on one MI355X.

One step is one call of the library on one synthetic problem with its inputs
already resident in HBM.  The default workload is the 8192^3 MXFP4 addmm
(E2M1 values with an E8M0 scale per 32 K elements, a bf16 bias along N, bf16
output), the problem on which MXFP4 TFLOP/s and the fraction of the dense FP4
MFMA peak are quoted.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--cap C] [--no-cpu]

The ``roofline`` object uses kernel durations measured here with HIP events on
the launch stream; ``traffic`` comes from the rocprofv3 counter summary kept
under profiles/ and is reported only while the kernel sources are the ones
that summary was taken with (it counts L2-to-fabric bytes, MALL hits
included: an upper bound on HBM bytes).  ``cpu_baseline`` times the CPU oracle
(test infrastructure, never the product path) on the same workload, whole,
repeated for at least ten seconds.  The default run also times the other
synthetic configurations at their default launches (``other_configs``: the
256x256x512 MXFP4 addmm on 5 workgroups, the bf16 addmm at 4096^3, the
16x8192x8192 MXFP4 GEMM over rotating input copies and the fp8 4096^3 GEMM at
grid caps 1, 32, 64, 128 and 256), each with its roofline and a shorter oracle
baseline; ``--no-others`` skips them.

    python bench.py --copy-calibration MIB          # plain device copy (counter reference)
    python bench.py --co-schedule C [--workload W]  # the GEMM on C CUs beside a memory-bound kernel
                                                    # on the other CUs (its own JSON line)
    python bench.py --traffic-summary F W CF CW --copy-calibration MIB
                                                    # rocprofv3 --pmc CSVs -> profiles/traffic_<workload>.json
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MXFP4 Stream-K GEMM TFLOP/s and % of dense FP4 MFMA peak, 1 MI355X"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
# (FP6 runs at the FP4 rate; a product with one E4M3 operand at the fp8 rate)
PEAK_TFLOPS = {"mxfp4": 10100.0, "mxfp6_e2m3": 10100.0, "mxfp6_e3m2": 10100.0, "fp8": 5000.0, "mxfp8": 5000.0,
               "mxfp4_mxfp8": 5000.0, "mxfp8_mxfp4": 5000.0, "bf16": 2500.0}
# bits per element of A and of B
ELEMENT_BITS = {"mxfp4": (4, 4), "mxfp6_e2m3": (6, 6), "mxfp6_e3m2": (6, 6), "mxfp8": (8, 8), "fp8": (8, 8),
                "mxfp4_mxfp8": (4, 8), "mxfp8_mxfp4": (8, 4), "bf16": (16, 16)}
MIXED = {"mxfp4_mxfp8": ("mxfp4", "mxfp8"), "mxfp8_mxfp4": ("mxfp8", "mxfp4")}
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "mxfp4_addmm_8192"


# the sources that decide the forward GEMM kernels and their launch (the
# backward helpers live in a file of their own)
GEMM_SOURCES = ("sk_api.cpp", "sk_common.h", "sk_kernel.h", "sk_kernels.hip", "sk_kernels_mx.hip",
                "sk_kernels_ksplit.hip", "sk_tuning_table.inc")


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "persistent_gemm_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, tag: str, variant: int):
    """HBM bytes per launch from the committed counter summary, if it was taken
    with these kernel sources and the same compiled kernel."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}{tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash() or rec.get("variant") != variant:
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_per_dispatch(csv_dir: str, counter: str, match) -> list:
    """Per-dispatch totals of one rocprofv3 --pmc counter (CSV output) for kernels whose name passes `match`."""
    import csv
    import glob
    per = {}
    for f in sorted(glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter or not match(r["Kernel_Name"]):
                    continue
                key = (f, r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    return list(per.values())


def traffic_summary(args) -> int:
    """HBM bytes per launch of the GEMM kernel from FETCH_SIZE / WRITE_SIZE runs, each
    scaled by what the same counter reads for a plain device copy of known size."""
    fetch_dir, write_dir, copy_fetch_dir, copy_write_dir = args.traffic_summary
    is_gemm = lambda name: "sk_gemm_kernel" in name
    is_copy = lambda name: "copyBuffer" in name   # the HIP runtime's device-to-device copy kernel
    copy_bytes = args.copy_calibration * (1 << 20)
    out = {"workload": args.workload, "source_hash": source_hash(), "copy_bytes": copy_bytes}
    for name, gdir, cdir in (("fetch", fetch_dir, copy_fetch_dir), ("write", write_dir, copy_write_dir)):
        counter = "FETCH_SIZE" if name == "fetch" else "WRITE_SIZE"
        g = _pmc_per_dispatch(gdir, counter, is_gemm)
        c = _pmc_per_dispatch(cdir, counter, is_copy)
        if not g or not c:
            print(f"no {counter} dispatches found (gemm {len(g)}, copy {len(c)})", file=sys.stderr)
            return 1
        g_kib, c_kib = float(np.mean(g)), float(np.mean(c))
        factor = copy_bytes / (c_kib * 1024.0)
        out[name] = {"counter": counter, "gemm_kib_per_dispatch": g_kib, "gemm_dispatches": len(g),
                     "copy_kib_per_dispatch": c_kib, "copy_dispatches": len(c), "scale": factor,
                     "bytes_per_launch": g_kib * 1024.0 * factor}
    out["hbm_bytes_per_launch"] = out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"]
    import persistent_gemm_amd as pg
    from persistent_gemm_amd.inputs import WORKLOADS
    w = WORKLOADS[args.workload]
    out["algorithmic_bytes"] = algorithmic_bytes(w)
    # the kernel the default launch uses (the counters were taken on it)
    out["variant"] = pg.plan(w.dtype, w.M, w.N, w.K, grid_cap=w.grid_cap, policy=pg.AUTO, num_cus=256).variant
    path = os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))
    return 0


def copy_calibration(args) -> int:
    """A plain device-to-device copy of known size (the reference for the HBM byte counters)."""
    import torch
    n = args.copy_calibration * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").random_(0, 256)
    dst = torch.empty_like(src)
    for _ in range(args.warmup + args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": args.warmup + args.steps}), flush=True)
    return 0


def algorithmic_bytes(w) -> int:
    """Each operand, scale, bias and output element once."""
    M, N, K = w.M, w.N, w.K
    if w.op == "backward":
        # reads dC, A, B; writes dA, dB, dbias
        return 2 * (M * N + M * K + N * K) + 2 * (M * K + N * K) + 2 * N
    ba, bb = ELEMENT_BITS[w.dtype]
    b = (M * K * ba + N * K * bb) // 8
    if w.dtype == "fp8":
        b += 8                                  # the two per-tensor fp32 scales
    elif w.dtype != "bf16":
        b += (M + N) * (K // 32)                # E8M0 block scales
    return b + (2 * N if w.bias else 0) + 2 * M * N


def cpu_baseline(w, x, budget_s: float = 10.0) -> dict:
    """The oracle on the whole workload, repeated until budget_s of CPU time has passed."""
    import oracle
    if w.op == "backward":
        run_once = lambda: oracle.bf16_backward(x["dC"], x["A"], x["B"])
        what = "decode, two matrix products and a column sum"
    elif w.dtype in MIXED:
        run_once = lambda: oracle.gemm_mx(*MIXED[w.dtype], x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=w.K)
        what = "decode, one matrix product"
    else:
        run_once = lambda: oracle.gemm(w.dtype, x["A"], x["B"], x["SA"], x["SB"], x["bias"], K=w.K)
        what = "decode, one matrix product"
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: assume BLAS uses the affinity set
        threads = cores
    runs, t0 = 0, time.perf_counter()
    while True:
        run_once()
        runs += 1
        t = time.perf_counter() - t0
        if t >= budget_s:
            break
    flops = float(w.flops) * runs
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "blas_threads": int(threads),
            "kind": "oracle",
            "sample": f"the whole {w.M}x{w.N}x{w.K} problem, {runs} oracle run(s) in {t:.1f} s (fp64 numpy: "
                      f"{what} with {threads} BLAS threads on {cores} cores of the affinity set, bf16 rounding)"}


def co_schedule(args, w, d, tile, policy) -> int:
    """The capped GEMM co-scheduled with other work on one device.

    The GEMM runs on a stream held to CUs [0, C) (its grid is then C
    workgroups) while a memory-bound elementwise loop (out = in + 1 over
    1 GiB of fp32) runs on a stream held to the other CUs.  Each is timed
    alone and both together; the same pair is then run on two unmasked
    streams with the GEMM's grid capped at C workgroups, which caps the count
    but lets its workgroups land on any CU.  Prints one JSON line."""
    import torch

    import persistent_gemm_amd as pg

    n = torch.cuda.get_device_properties(0).multi_processor_count
    g = args.co_schedule
    if not 0 < g < n:
        print(f"--co-schedule needs 0 < C < {n}", file=sys.stderr)
        return 2
    src = torch.ones(256 << 20, device="cuda")
    dst = torch.empty_like(src)
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    def gemm(stream, cap):
        with torch.cuda.stream(stream):
            pg.gemm_ex(w.dtype, d["A"], d["B"], d["SA"], d["SB"], d["bias"], C, grid_cap=cap, policy=policy,
                       tile=tile, variant=args.variant)

    def other(stream):
        with torch.cuda.stream(stream):
            torch.add(src, 1.0, out=dst)

    def alone(fn, stream, k):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    def together(sg, cap, so, ng, no):
        eg = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        eo = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eg[0].record(sg)
        eo[0].record(so)
        # interleaved enqueues, so that both streams have work from the start
        for i in range(max(ng, no)):
            if i < ng:
                gemm(sg, cap)
            if i < no:
                other(so)
        eg[1].record(sg)
        eo[1].record(so)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) * 1e3
        return eg[0].elapsed_time(eg[1]) / ng, eo[0].elapsed_time(eo[1]) / no, wall

    def summary(tg, to, k, no, tgt, tot, wall):
        return {"gemm_ms_alone": round(tg, 5), "other_ms_alone": round(to, 5), "gemm_calls": k, "other_calls": no,
                "gemm_ms_together": round(tgt, 5), "other_ms_together": round(tot, 5),
                "wall_ms_together": round(wall, 3), "speedup_vs_serial": round((k * tg + no * to) / wall, 3)}

    k = max(args.steps, 5)
    sg = pg.cu_masked_stream(range(g))
    so = pg.cu_masked_stream(range(g, n))
    try:
        tg = alone(lambda: gemm(sg, 0), sg, k)
        to = alone(lambda: other(so), so, k)
        no = max(1, round(k * tg / to))
        part = summary(tg, to, k, no, *together(sg, 0, so, k, no))
        pg.check(sg)
    finally:
        pg.destroy_stream(sg)
        pg.destroy_stream(so)
    ug, uo = torch.cuda.Stream(), torch.cuda.Stream()
    tg2 = alone(lambda: gemm(ug, g), ug, k)
    to2 = alone(lambda: other(uo), uo, k)
    capped = summary(tg2, to2, k, no, *together(ug, g, uo, k, no))
    pg.check(ug)
    moved = 2 * src.numel() * 4
    print(json.dumps({
        "metric": "co-scheduled Stream-K GEMM beside a memory-bound kernel, 1 MI355X",
        "workload": args.workload, "dtype": w.dtype, "device_cus": n, "gemm_cus": g, "other_cus": n - g,
        "other_kernel": f"out = in + 1 over fp32 buffers ({moved / 2**30:.1f} GiB moved per call)",
        "gemm_tflops_alone_on_partition": round(w.flops / (tg / 1e3) / 1e12, 3),
        "other_gbs_alone_on_partition": round(moved / (to / 1e3) / 1e9, 1),
        "cu_partition": part, "grid_cap_only": capped}), flush=True)
    return 0


def hold_device(torch, cycles: int) -> None:
    """Queue a spin kernel of about `cycles` GPU clocks on the current stream, so
    the host can enqueue the timed calls before the device reaches them (the
    events around those calls then time the device, not the host).  Without
    torch's spin kernel the calls are simply timed as enqueued."""
    spin = getattr(torch.cuda, "_sleep", None)
    if spin is not None:
        spin(int(cycles))


def vendor(args, w, copies, C, ours) -> int:
    """The vendor library on the same device inputs: torch.addmm (bf16) and
    torch._scaled_mm (fp8 per-tensor, MXFP4 / MXFP8 with E8M0 blocks of 32),
    which torch dispatches to hipBLASLt on gfx950.  Reports its time per call
    (HIP events around the whole timed loop, queue kept full) next to this
    library's, timed the same way, and how many outputs agree bit for bit
    (MXFP4: every partial sum is exact, so they must all agree; the
    vendor's MX call takes no bias here, so both run without one)."""
    import torch
    d0 = copies[0]
    if w.dtype not in ("mxfp4", "mxfp8", "fp8", "bf16"):
        print(f"--vendor: torch has no {w.dtype} product to compare with", file=sys.stderr)
        return 2
    if w.dtype in ("mxfp4", "mxfp8"):
        el = torch.float4_e2m1fn_x2 if w.dtype == "mxfp4" else torch.float8_e4m3fn
        vs = [(c["A"].view(el), c["B"].view(el).t(), c["SA"].view(torch.float8_e8m0fnu),
               c["SB"].view(torch.float8_e8m0fnu)) for c in copies]

        def theirs(i):
            a, b, sa, sb = vs[i % len(vs)]
            return torch._scaled_mm(a, b, sa, sb, out_dtype=torch.bfloat16)

        def ours_nb(i):
            c = copies[i % len(copies)]
            return pg_call(w, c, None, C)
    elif w.dtype == "fp8":
        def theirs(i):
            c = copies[i % len(copies)]
            return torch._scaled_mm(c["A"], c["B"].t(), c["SA"].reshape(()), c["SB"].reshape(()),
                                    out_dtype=torch.bfloat16)
        ours_nb = None
    else:
        def theirs(i):
            c = copies[i % len(copies)]
            return torch.addmm(c["bias"], c["A"], c["B"].t()) if c["bias"] is not None else torch.mm(c["A"], c["B"].t())
        ours_nb = None
    mine = ours_nb or (lambda i: ours(i))

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        hold_device(torch, 20_000_000)   # the queue stays ahead of the host: events time the device
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    t_v, t_o = timed(theirs), timed(mine)
    agree = None
    if ours_nb is not None:
        ref = theirs(0).view(torch.int16)
        torch.cuda.synchronize()
        ours_nb(0)
        torch.cuda.synchronize()
        agree = round(float((C.view(torch.int16) == ref).float().mean()), 6)
    print(json.dumps({
        "metric": f"vendor reference: {w.dtype} GEMM TFLOP/s through torch (hipBLASLt), 1 MI355X",
        "workload": args.workload, "vendor_ms": round(t_v, 5), "vendor_tflops": round(w.flops / t_v / 1e9, 1),
        "ours_ms": round(t_o, 5), "ours_tflops": round(w.flops / t_o / 1e9, 1),
        "bias": bool(w.bias) and ours_nb is None, "outputs_bit_equal": agree,
        "timing": f"HIP events around {args.steps} back-to-back calls after {args.warmup} warm-ups"}), flush=True)
    return 0


def pg_call(w, c, bias, C):
    import persistent_gemm_amd as pg
    return pg.gemm_ex(w.dtype, c["A"], c["B"], c["SA"], c["SB"], bias, C, policy=pg.AUTO)


def device_inputs(torch, w, x, dev) -> dict:
    """Host arrays of one forward workload -> device tensors for the binding."""
    d = {}
    for op, fmt in zip(("A", "B"), MIXED.get(w.dtype, (w.dtype, w.dtype))):
        t = np.ascontiguousarray(x[op])
        if fmt == "bf16":
            d[op] = torch.from_numpy(t.view(np.int16)).view(torch.bfloat16).to(dev)
        elif fmt in ("mxfp8", "fp8"):
            d[op] = torch.from_numpy(t).view(torch.float8_e4m3fn).to(dev)
        else:  # packed E2M1 or FP6 bytes
            d[op] = torch.from_numpy(t).to(dev)
    if w.dtype == "bf16":
        d["SA"] = d["SB"] = None
    elif w.dtype == "fp8":
        d["SA"] = torch.tensor([x["SA"]], dtype=torch.float32, device=dev)
        d["SB"] = torch.tensor([x["SB"]], dtype=torch.float32, device=dev)
    else:
        for k in ("SA", "SB"):
            d[k] = torch.from_numpy(np.ascontiguousarray(x[k])).to(dev)
    d["bias"] = None if x["bias"] is None else torch.from_numpy(x["bias"].view(np.int16)).view(torch.bfloat16).to(dev)
    return d


# Untimed calls after the warm-up steps, until this much wall time has passed: under
# load the device raises its shader clock over the first several milliseconds (a
# 260 us call runs at about 320 us for its first twenty-odd repetitions), so a short
# warm-up would time the ramp instead of the steady state.
SETTLE_MS = 50.0


def time_steps(torch, pg, step, steps: int, warmup: int) -> dict:
    """Wall time per step over `steps` timed steps (after `warmup` steps and the settle
    calls), with nothing but the steps between the two synchronisations; then the device
    time per call: the same steps again between two events on the launch stream, with a
    spin kernel queued first so that the host stays ahead and the calls run back to back;
    then, for information, HIP events around each call of a third pass (events recorded
    between calls lengthen a short call's wall time, so the timed loop has none)."""
    for i in range(warmup):
        step(i)
    pg.check()
    torch.cuda.synchronize()
    t_settle, n_settle = time.perf_counter(), 0
    while (time.perf_counter() - t_settle) * 1e3 < SETTLE_MS:
        step(warmup + n_settle)
        n_settle += 1
        if n_settle % 8 == 0:
            torch.cuda.synchronize()   # keep the queue short: the loop measures device time, not enqueue time
    torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    pg.check()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pg.check()
    # a spin just long enough for the host to enqueue the pass (about 10 us of host time
    # per call), then three untimed calls that bring the clock back to the load's level
    hold_device(torch, 30_000 * (steps + 3))
    for i in range(3):
        step(i)
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record(stream)
    for i in range(steps):
        step(i)
    d1.record(stream)
    torch.cuda.synchronize()
    pg.check()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(stream)
        step(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    pg.check()
    call_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    return {"ms_per_step": wall / steps * 1e3, "call_ms": call_ms, "dev_ms": d0.elapsed_time(d1) / steps,
            "settle": {"calls": n_settle, "ms": round(settle_ms, 1)}}


def roofline_of(w, p, dev_ms: float, call_ms, traffic, cap_scaled: bool) -> dict:
    """The roofline object of one workload: MFMA-bound (FLOP/s against the dtype's dense
    peak, scaled by grid/256 for a capped grid) or, for the 16-row MXFP4 shape,
    HBM-bound (algorithmic bytes/s against 8 TB/s)."""
    s = dev_ms / 1e3
    ab = algorithmic_bytes(w)
    peak = PEAK_TFLOPS[w.dtype] * (p.grid / 256.0 if cap_scaled else 1.0)
    achieved = float(w.flops) / s / 1e12
    r = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
         "frac": round(achieved / peak, 4), "traffic": traffic,
         "traffic_what": ("HBM bytes per launch, upper bound: the L2-to-fabric FETCH_SIZE + WRITE_SIZE counters of "
                          "the kernel (MALL hits included), each scaled by what it reads for a plain copy"),
         "kernel_ms": {"mean": round(dev_ms, 5),
                       "how": "device time per call, back-to-back calls between two HIP events"},
         "call_ms": {"mean": round(float(np.mean(call_ms)), 5), "min": round(float(np.min(call_ms)), 5),
                     "median": round(float(np.median(call_ms)), 5), "max": round(float(np.max(call_ms)), 5),
                     "how": "HIP events around each call of a pass after the timed ones"},
         "algorithmic_bytes": ab, "hbm_gbs_at_algorithmic_bytes": round(ab / s / 1e9, 1)}
    if w.dtype == "mxfp4" and w.M <= 16:
        r.update({"bound": "hbm", "achieved": round(ab / s / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                  "frac": round(ab / s / 1e9 / PEAK_HBM_GBS, 4)})
    return r


def plan_config(pg, p) -> dict:
    return {"tile": f"{p.tile_m}x{p.tile_n}x{p.tile_k}", "threads": p.threads, "variant": p.variant,
            "policy": {pg.HYBRID: "hybrid", pg.PURE_SK: "sk", pg.PURE_DP: "dp"}[p.policy], "grid": p.grid,
            "sk_tiles": p.sk_tiles, "tiles": p.tiles}


# The other synthetic configurations, each timed at its default launch beside the
# headline (the MXFP4 addmm at 8192^3): the 256x256x512 MXFP4 addmm on a grid of
# 5 (latency-bound), the bf16 addmm at 4096^3, the skinny 16x8192x8192 MXFP4
# GEMM (HBM-bound, timed over rotating input copies) and the fp8 4096^3 GEMM at
# each grid cap of its sweep.
OTHER_CONFIGS = ("mxfp4_addmm_256x256x512_g5", "bf16_addmm_4096", "mxfp4_gemm_16x8192x8192",
                 "fp8_gemm_4096_capsweep")


def other_configs(torch, pg, dev, steps: int, warmup: int, cpu: bool) -> list:
    from persistent_gemm_amd.inputs import WORKLOADS, make_inputs
    out = []
    for name in OTHER_CONFIGS:
        w = WORKLOADS[name]
        x = make_inputs(w.dtype, w.M, w.N, w.K, bias=w.bias, seed=w.seed)
        copies = [device_inputs(torch, w, x, dev)]
        for _ in range(1, max(1, w.rotate)):
            copies.append({k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in copies[0].items()})
        C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        tile = tuple(int(v) for v in w.tile.split("x")) if w.tile else None
        caps = w.caps or (w.grid_cap,)
        rec = {"workload": name, "dtype": w.dtype, "M": w.M, "N": w.N, "K": w.K, "bias": w.bias,
               "input_copies": len(copies)}
        runs = []
        for cap in caps:
            p = pg.plan(w.dtype, w.M, w.N, w.K, grid_cap=cap, policy=pg.AUTO, tile=tile)

            def step(i, cap=cap):
                c = copies[i % len(copies)]
                pg.gemm_ex(w.dtype, c["A"], c["B"], c["SA"], c["SB"], c["bias"], C, grid_cap=cap, policy=pg.AUTO,
                           tile=tile)

            # a capped call takes up to 256/cap times longer (about 10 ms at cap 1): fewer repetitions there
            n = max(3, min(steps, steps * p.grid // 256)) if w.caps else steps
            t = time_steps(torch, pg, step, n, min(warmup, n))
            r = {"grid_cap": cap, "steps": n, "settle": t["settle"], "ms_per_step": round(t["ms_per_step"], 5),
                 "value": round(float(w.flops) / (t["ms_per_step"] / 1e3) / 1e12, 3), "unit": "TFLOP/s",
                 "config": plan_config(pg, p),
                 "roofline": roofline_of(w, p, t["dev_ms"], t["call_ms"], None, bool(w.caps))}
            if name == "mxfp4_addmm_256x256x512_g5":
                # 67 MFLOP on 5 workgroups: the call is bound by launch and fixup latency, not by a roofline
                r["roofline"].update({"bound": "latency"})
            runs.append(r)
        if len(runs) == 1:
            rec.update(runs[0])
        else:
            rec["cap_sweep"] = runs
        if cpu:
            rec["cpu_baseline"] = cpu_baseline(w, x, budget_s=3.0)
        out.append(rec)
        del copies, C
        torch.cuda.empty_cache()
    return out


def ceiling(args) -> int:
    """The device's own ceilings for the roofline, from libskprobe.so: MFMA-only rates on the
    whole device with fixed, rotating random and zero operands (FP4, FP6, E4M3, bf16), the
    rotating-operand FP4 rate with direct-to-LDS loads of random bytes interleaved, from an
    L2-sized and a memory-sized span per workgroup, and the cold read of 32 MiB by the
    skinny call's row pattern and by plain loads.  One JSON line."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "persistent_gemm_amd", "libskprobe.so"))
    lib.skp_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_float),
                                  ctypes.POINTER(ctypes.c_double)]
    lib.skp_mfma_dma.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_int,
                                 ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double),
                                 ctypes.POINTER(ctypes.c_double)]
    torch.cuda.set_device(0)
    ms, flop, nbytes = ctypes.c_float(), ctypes.c_double(), ctypes.c_double()
    rows = []
    kinds = [("fp4 scaled 32x32x64", 0, PEAK_TFLOPS["mxfp4"], 80000), ("e4m3 scaled 32x32x64", 1, PEAK_TFLOPS["fp8"], 50000),
             ("bf16 32x32x16", 2, PEAK_TFLOPS["bf16"], 100000),
             ("fp4 scaled 16x16x128", 3, PEAK_TFLOPS["mxfp4"], 160000), ("bf16 16x16x32", 4, PEAK_TFLOPS["bf16"], 200000),
             ("fp6 e2m3 scaled 32x32x64", 5, PEAK_TFLOPS["mxfp6_e2m3"], 80000)]
    for name, kind, peak, iters in kinds:
        for mode, what in ((0, "fixed operands"), (1, "rotating random operands"), (2, "zero operands")):
            if lib.skp_mfma_rate(kind, mode, iters, ctypes.byref(ms), ctypes.byref(flop)) != 0:
                raise RuntimeError("skp_mfma_rate failed")
            tf = flop.value / (ms.value / 1e3) / 1e12
            rows.append({"probe": "mfma only", "mfma": name, "data": what, "ms": round(ms.value, 3),
                         "tflops": round(tf, 1), "frac_of_peak": round(tf / peak, 4)})
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (256 << 20,), dtype=torch.int32, device="cuda")   # 1 GiB of random bytes
    for span, where in ((64 << 10, "64 KiB per workgroup (L2)"), (4 << 20, "4 MiB per workgroup (memory)")):
        for loads in (0, 1, 2, 4):
            if lib.skp_mfma_dma(loads, src.data_ptr(), span, 60000, ctypes.byref(ms), ctypes.byref(flop),
                                ctypes.byref(nbytes)) != 0:
                raise RuntimeError("skp_mfma_dma failed")
            s = ms.value / 1e3
            rows.append({"probe": "fp4 mfma + direct-to-LDS loads", "loads_per_8_mfma": loads, "span": where,
                         "ms": round(ms.value, 3), "tflops": round(flop.value / s / 1e12, 1),
                         "gbs_per_cu_into_lds": round(nbytes.value / s / 1e9 / 256, 1)})
            print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    # the cold read of the skinny call's 32 MiB of B: 15 launches, each on a region none before it read
    lib.skp_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_float)]
    times = (ctypes.c_float * 15)()
    for pattern, what in ((0, "direct-to-LDS rows: 256 workgroups x 32 rows x 4 KiB, 128 B of each row per load"),
                          (1, "plain 16-byte vector loads: 1024 workgroups, contiguous slices")):
        if lib.skp_stream(pattern, src.data_ptr(), 15, times) != 0:
            raise RuntimeError("skp_stream failed")
        us = sorted(t * 1e3 for t in times)
        rows.append({"probe": "cold read of 32 MiB", "pattern": what, "us_median": round(us[7], 2),
                     "us_min": round(us[0], 2), "tbs_at_median": round((32 << 20) / (us[7] * 1e-6) / 1e12, 2),
                     "how": "HIP events around each launch (its dispatch included)"})
        print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
    print(json.dumps({"ceiling": rows, "how": "256 workgroups of 8 waves (2 per SIMD), back-to-back MFMAs into 8 "
                      "accumulators per wave; one timed launch after a shorter warm-up launch"}), flush=True)
    return 0


def trace_calls(args, torch, pg, w, copies, C, cap, policy, tile, p) -> int:
    """The launch's phase trace on `args.trace` calls (after the warm-ups), one JSON line each."""
    buf = torch.zeros(32 * p.grid, dtype=torch.int64, device=C.device)
    for i in range(args.warmup):
        d = copies[i % len(copies)]
        pg.gemm_ex(w.dtype, d["A"], d["B"], d["SA"], d["SB"], d["bias"], C, grid_cap=cap, policy=policy, tile=tile,
                   variant=args.variant)
    pg.check()
    for i in range(args.trace):
        d = copies[(args.warmup + i) % len(copies)]
        buf.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pg.gemm_ex(w.dtype, d["A"], d["B"], d["SA"], d["SB"], d["bias"], C, grid_cap=cap, policy=policy, tile=tile,
                   variant=args.variant, trace=buf)
        e1.record()
        pg.check()
        summ = pg.phase_summary(buf.cpu().numpy(), p.grid, p)
        print(json.dumps({"workload": args.workload, "call": i, "event_us": round(e0.elapsed_time(e1) * 1e3, 2),
                          "config": plan_config(pg, p), "input_copies": len(copies), "phases": summ}), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cap", type=int, default=None, help="grid cap (default: the workload's)")
    ap.add_argument("--tile", default=None, help="tile override, e.g. 256x256")
    ap.add_argument("--policy", default="auto", choices=["auto", "hybrid", "sk", "dp"],
                    help="auto: the measured kernel and policy for the shape (what the plain entry points use)")
    ap.add_argument("--variant", type=int, default=None, help="compiled kernel index (default: automatic)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other configurations (only the named workload is timed)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="rotate over this many input copies (defeats the MALL; default: the workload's)")
    ap.add_argument("--co-schedule", type=int, default=0, metavar="C",
                    help="run the GEMM on C CUs beside a memory-bound kernel on the other CUs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run a plain device copy of MIB MiB instead (counter calibration)")
    ap.add_argument("--vendor", action="store_true",
                    help="time the vendor library (hipBLASLt through torch.addmm / torch._scaled_mm) on the "
                         "same inputs instead (context only; its own JSON line)")
    ap.add_argument("--trace", type=int, default=0, metavar="CALLS",
                    help="instead of timing, run CALLS calls of the launch with the library's phase trace and "
                         "print each call's phase summary (per-workgroup 100 MHz stamps: ramp, streaming, "
                         "fixup waits, epilogues) as one JSON line")
    ap.add_argument("--ceiling", action="store_true",
                    help="instead of the GEMM, run the device-ceiling probes (libskprobe.so): MFMA-only rates by "
                         "operand data and with direct-to-LDS loads interleaved")
    ap.add_argument("--zero-data", action="store_true",
                    help="time the workload with all-zero A and B (same kernel and launch): the power the "
                         "operand bits draw sets the clock; its own JSON line, never the headline")
    ap.add_argument("--traffic-summary", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from rocprofv3 --pmc CSV output (no GPU)")
    args = ap.parse_args()
    if args.traffic_summary:
        if args.copy_calibration <= 0:
            ap.error("--traffic-summary needs --copy-calibration MIB (the copy size of the calibration runs)")
        return traffic_summary(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    if args.copy_calibration > 0:
        return copy_calibration(args)
    if args.ceiling:
        return ceiling(args)

    import torch

    import persistent_gemm_amd as pg
    from persistent_gemm_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    cap = w.grid_cap if args.cap is None else args.cap
    tile = None
    if args.tile:
        tile = tuple(int(v) for v in args.tile.lower().split("x"))
    elif w.tile:
        tile = tuple(int(v) for v in w.tile.split("x"))
    policy = {"auto": pg.AUTO, "hybrid": pg.HYBRID, "sk": pg.PURE_SK, "dp": pg.PURE_DP}[args.policy]

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if w.op == "backward":
        from persistent_gemm_amd.inputs import backward_inputs
        x = backward_inputs(w.M, w.N, w.K, seed=w.seed)
        d = {k: torch.from_numpy(x[k].view(np.int16)).view(torch.bfloat16).to(dev) for k in ("dC", "A", "B")}
        p = pg.plan(w.dtype, w.M, w.K, w.N, grid_cap=cap, policy=policy)   # the dA product's plan

        def step(i):
            pg.gemm_bf16_backward(d["dC"], d["A"], d["B"], grid_cap=cap)
    else:
        if w.dtype in MIXED:
            from persistent_gemm_amd.inputs import mixed_inputs
            x = mixed_inputs(*MIXED[w.dtype], w.M, w.N, w.K, bias=w.bias, seed=w.seed)
        else:
            x = make_inputs(w.dtype, w.M, w.N, w.K, bias=w.bias, seed=w.seed)
        if args.co_schedule:
            return co_schedule(args, w, device_inputs(torch, w, x, dev), tile, policy)

        copies = [device_inputs(torch, w, x, dev)]
        if args.zero_data:
            copies[0]["A"].zero_()
            copies[0]["B"].zero_()
        for i in range(1, max(1, args.rotate or w.rotate)):
            copies.append({k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in copies[0].items()})
        C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        p = pg.plan(w.dtype, w.M, w.N, w.K, grid_cap=cap, policy=policy, tile=tile, variant=args.variant)

        def step(i):
            d = copies[i % len(copies)]
            pg.gemm_ex(w.dtype, d["A"], d["B"], d["SA"], d["SB"], d["bias"], C, grid_cap=cap, policy=policy, tile=tile,
                       variant=args.variant)

        if args.vendor:
            return vendor(args, w, copies, C, step)
        if args.trace:
            return trace_calls(args, torch, pg, w, copies, C, cap, policy, tile, p)

    t = time_steps(torch, pg, step, args.steps, args.warmup)
    ms_per_step = t["ms_per_step"]
    value = float(w.flops) / (ms_per_step / 1e3) / 1e12
    default_launch = (args.cap is None and args.tile is None and policy == pg.AUTO and args.variant is None
                      and not args.zero_data)
    tag = "" if default_launch else "_nondefault"
    traffic = traffic_for(args.workload, tag, p.variant)
    out = {
        "metric": (METRIC if w.dtype == "mxfp4" else
                   f"{w.dtype} Stream-K GEMM backward (dA, dB, dbias) TFLOP/s, 1 MI355X" if w.op == "backward" else
                   f"{w.dtype} Stream-K GEMM TFLOP/s, 1 MI355X"),
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": {**t["settle"], "why": f"untimed calls after the warm-up until {SETTLE_MS:.0f} ms have passed: "
                                         "the device raises its clock over the first milliseconds under load"},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic, A and B all zero (--zero-data)" if args.zero_data else "synthetic",
        "config": {"workload": args.workload, "op": w.op, "M": w.M, "N": w.N, "K": w.K, "bias": w.bias,
                   "input_copies": max(1, args.rotate or w.rotate), **plan_config(pg, p),
                   "policy_requested": args.policy, "parallelism": "stream-k, 1 GPU"},
        "roofline": roofline_of(w, p, t["dev_ms"], t["call_ms"], traffic,
                                args.workload.startswith("fp8_gemm_4096_cap")),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w, x)
    if args.workload == DEFAULT_WORKLOAD and default_launch and not args.no_others:
        del step
        if w.op == "forward":
            del copies, C
        torch.cuda.empty_cache()
        out["other_configs"] = other_configs(torch, pg, dev, args.steps, args.warmup, not args.no_cpu)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
