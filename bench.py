#!/usr/bin/env python3
"""Throughput of the tiled dense GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats R]
                    [--settle-s S] [--flush] [--workload NAME]

A step is one C = A . B^T launch through the C ABI (gemm_bf16_nt) on the
bf16 NT 4096 x 4096 x 8192 workload, inputs already resident in HBM.  The
throughput of a region of K launches is 2 M N K K / t (the pages' TFLOPS
formula, TileLang SM100 README, "Compilation and Usage").  Prints ONE JSON
line on stdout; context goes to stderr.

Timing, in this order, all on one non-default stream:
  1. W untimed launches, then a first timed region of K launches: what a
     short run measures, at whatever clock the chip has just after start
     (reported under timing.first_region);
  2. a settle phase: untimed launches for S seconds (default 2; the count
     and the seconds are in the line).  Under sustained load the board
     holds its power limit and the shader clock settles over about a second;
  3. R timed regions of exactly K back-to-back launches, each between two
     HIP events recorded on the launch stream.  `value` and `ms_per_step`
     are the median region's; min and max are reported beside it.  With one
     kernel per launch and the launches back to back, the median region's
     time per launch is the kernel's mean duration that
     `roofline.achieved` divides the algorithmic flops by (a rocprofv3
     kernel trace of the same command gives the same mean within 1%);
  4. K more launches, each between its own pair of events, for the spread
     of single launches (min, median, max; the events' markers add a few us
     to each, so these are not used for the mean).
Clock probes (the library's tgemm_clock_probe: s_memtime against
s_memrealtime on every CU, paired per CU) bracket the first region, the
settle phase and the set of timed regions, giving the shader clock each XCD
delivered over each.

--graph captures each region's K launches into a HIP graph once and times
its replay, so that host launch costs do not enter the time of short
kernels (the small workloads).

--flush is the cold-cache variant: before every launch a 512 MB buffer is
written, which evicts the inputs from the L2s and the 256 MB Infinity
Cache; each region is followed by the same region of flushes alone, whose
time is subtracted.

--zero-elements is a clock diagnostic: the same launches on inputs whose
elements are all zero (block scales kept).  The kernels run the same
instructions and cycles, but without data-dependent switching the board
stays below its power limit; the clock it then holds, against the one on
the workload's data, shows how much of the time the power limit sets.  Its
line says so under "data" and is not a measurement of the workload.

The line also carries:
  roofline     `traffic` is the HBM bytes per launch from rocprofv3
               FETCH_SIZE/WRITE_SIZE counters, calibrated on a plain copy,
               when a committed measurement matches the current kernel
               source, else null;
  cpu_baseline the CPU oracle (binary64 triple loop, all host threads) timed
               on a bounded sample of the same workload: whole rows of C,
               scaled to TFLOPS.

Two helper modes serve the traffic measurement:
  --copy-calibration       only run a plain device-to-device copy of 1 GiB
                           (torch's copy kernel) a few times, for rocprofv3
                           to count what a copy of known size reads/writes;
  --record-traffic DIR     host only: read the four rocprofv3 --pmc CSVs in
                           DIR (gemm_fetch, gemm_write, copy_fetch,
                           copy_write), scale the GEMM's per-dispatch
                           FETCH_SIZE and WRITE_SIZE by the copy's ratio of
                           known bytes to counted bytes, and write the JSON
                           record bench.py reads plus a short summary.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "mxfp8": 5033.2, "mxfp4": 10066.3, "mxfp6": 10066.3}  # MI355X dense MFMA, 256 CU x 2.4 GHz
METRIC = "TFLOPS (2MNK/t) and % of MFMA peak, bf16 NT GEMM 4096x4096x8192, 1 GPU"
CSRC = os.path.join(ROOT, "dense_tiled_gemm_bf16_amd", "csrc")
KERNEL_SRC = os.path.join(CSRC, "tgemm_kernels.hip")        # the GEMM kernels
QUANT_SRC = os.path.join(CSRC, "tgemm_quant.hip")           # the quantiser


def source_of(kind: str) -> str:
    return QUANT_SRC if kind == "quant_mxfp8" else KERNEL_SRC


def traffic_file(name: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{name}.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(text: str | None = None, src: str = KERNEL_SRC) -> str:
    """SHA-256 prefix of a kernel source's code: comments and blank lines
    removed, so that a change to comments alone keeps a counter record."""
    import re
    if text is None:
        text = open(src).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*", "", ln).rstrip() for ln in text.splitlines()]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from a committed counter run, if it was taken on
    the current kernel source; else None."""
    import workloads
    try:
        rec = json.load(open(traffic_file(name)))
    except (OSError, ValueError):
        return None
    src = source_of(workloads.WORKLOADS[name].kind)
    if rec.get("workload") != name or rec.get("kernel_source_sha256_16") != kernel_source_hash(src=src):
        return None
    return rec.get("hbm_bytes_per_launch")


def device_inputs(w, seed=0):
    import numpy as np
    import torch
    import workloads
    x = workloads.make_inputs(w, seed)
    dev = {}
    for k, v in x.items():
        t = torch.from_numpy(np.ascontiguousarray(v).view(np.int16 if v.dtype == np.uint16 else np.uint8))
        if v.dtype == np.uint16:
            t = t.view(torch.bfloat16 if w.kind == "bf16_nt" else torch.float16)
        dev[k] = t.cuda()
    return x, dev


def launcher(w, dev, out, stream, splitk=None):
    import torch
    import dense_tiled_gemm_bf16_amd as tg
    L = tg.lib()
    s = stream.cuda_stream
    M, N, K = w.M, w.N, w.K
    if splitk is not None:
        # The K-split entry point (16-bit kinds), its workspace allocated here.
        need = L.tgemm_splitk_workspace_bytes(M, N, splitk)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        fn = L.gemm_bf16_splitk if w.kind == "bf16_nt" else L.gemm_f16_splitk
        tb, ldb = (1, K) if w.kind == "bf16_nt" else (0, N)
        args = (0, tb, M, N, K, dev["A"].data_ptr(), K, dev["B"].data_ptr(), ldb, out.data_ptr(), N, splitk,
                ws.data_ptr(), ws.numel(), s)
        dev["_ws"] = ws
    elif w.kind == "bf16_nt":
        args = (M, N, K, dev["A"].data_ptr(), dev["B"].data_ptr(), out.data_ptr(), s)
        fn = L.gemm_bf16_nt
    elif w.kind == "f16_nn":
        args = (M, N, K, dev["A"].data_ptr(), dev["B"].data_ptr(), out.data_ptr(), s)
        fn = L.gemm_f16_nn
    elif w.kind.startswith("mxfp6"):
        fmt = {"mxfp6_e2m3_nt": 0, "mxfp6_e3m2_nt": 1}[w.kind]
        args = (fmt, M, N, K, dev["qA"].data_ptr(), dev["qB"].data_ptr(), dev["sA"].data_ptr(),
                dev["sB"].data_ptr(), out.data_ptr(), s)
        fn = L.gemm_mxfp6_nt
    else:
        args = (M, N, K, dev["qA"].data_ptr(), dev["qB"].data_ptr(), dev["sA"].data_ptr(),
                dev["sB"].data_ptr(), out.data_ptr(), s)
        fn = L.gemm_mxfp4_nt if w.kind == "mxfp4_nt" else L.gemm_mxfp8_nt

    def launch():
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{w.kind}: [{rc}] {tg.last_error()}")
    return launch


def parity_sample(w, x, out):
    """Sampled outputs of the timed launch against the oracle (rtol = atol = 1e-2)."""
    import numpy as np
    import torch
    import oracle
    import workloads
    rows, cols = workloads.sample_positions(w.M, w.N, 64, seed=7)
    got = out.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)[rows, cols]
    if w.kind == "bf16_nt":
        ref = oracle.gemm_bf16_nt_at(x["A"], x["B"], rows, cols)
    elif w.kind == "f16_nn":
        ref = oracle.gemm_f16_nn_at(x["A"], x["B"], rows, cols)
    elif w.kind == "mxfp4_nt":
        ref = oracle.gemm_mxfp4_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols)
    elif w.kind.startswith("mxfp6"):
        ref = oracle.gemm_mxfp6_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols,
                                      workloads.fp6_format(w.kind))
    else:
        ref = oracle.gemm_mxfp8_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols)
    dt = torch.float16 if w.kind == "f16_nn" else torch.bfloat16
    dec = lambda b: torch.from_numpy(b.view(np.int16)).view(dt).double().numpy()
    g, r = dec(got), dec(ref)
    bad = int((~(np.abs(g - r) <= 1e-2 + 1e-2 * np.abs(r))).sum())
    return {"checked": int(rows.size), "outside_tolerance": bad,
            "max_abs_err": float(np.abs(g - r).max())}


def cpu_baseline(w, x, target_s: float):
    """The oracle, as it stands, on whole rows of C; rows chosen so the run
    takes about target_s seconds on all host threads."""
    import numpy as np
    import oracle
    import workloads
    threads = oracle.num_threads()

    def rows_run(r):
        rows = np.repeat(np.arange(r, dtype=np.int64), w.N)
        cols = np.tile(np.arange(w.N, dtype=np.int64), r)
        t0 = time.perf_counter()
        if w.kind == "bf16_nt":
            oracle.gemm_bf16_nt_at(x["A"], x["B"], rows, cols)
        elif w.kind == "f16_nn":
            oracle.gemm_f16_nn_at(x["A"], x["B"], rows, cols)
        elif w.kind == "mxfp4_nt":
            oracle.gemm_mxfp4_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols)
        elif w.kind.startswith("mxfp6"):
            oracle.gemm_mxfp6_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols, workloads.fp6_format(w.kind))
        else:
            oracle.gemm_mxfp8_nt_at(x["qA"], x["qB"], x["sA"], x["sB"], rows, cols)
        return time.perf_counter() - t0

    probe_rows = max(1, threads // w.N + 1)
    t_probe = rows_run(probe_rows)
    per_row = t_probe / probe_rows
    rows = int(max(1, min(w.M, target_s / max(per_row, 1e-9))))
    t = rows_run(rows)
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / t / 1e12, "unit": "TFLOPS", "cores": threads, "kind": "oracle",
            "sample": f"{rows} whole rows of C ({rows}x{w.N} outputs, K={w.K}) of {w.name}, "
                      f"binary64 sequential-k oracle, {t:.1f} s; scaled to 2*rows*N*K/t",
            "seconds": t}


COPY_REPS = 5
COPY_BYTES = 1 << 30


def copy_calibration():
    """A plain copy of known size: reads and writes COPY_BYTES per dispatch."""
    import torch
    torch.cuda.set_device(0)
    n = COPY_BYTES
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copied {n} bytes x {COPY_REPS}")


def _counter_per_dispatch(path: str, counter: str, match):
    import csv
    per = {}
    names = set()
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter or not match(r["Kernel_Name"]):
            continue
        per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
        names.add(r["Kernel_Name"])
    if not per:
        raise SystemExit(f"{path}: no {counter} records for the kernel")
    vals = sorted(per.values())
    return sum(vals) / len(vals), len(vals), sorted(names)


def record_traffic(d: str, name: str):
    """Per-launch HBM bytes of the GEMM from FETCH_SIZE/WRITE_SIZE (KiB per
    dispatch), each scaled by known bytes / counted bytes of a plain copy."""
    import workloads
    w = workloads.WORKLOADS[name]
    quant = w.kind == "quant_mxfp8"
    stem = "quant" if quant else "gemm"
    f = lambda s: os.path.join(d, f"{s}_counter_collection.csv")
    is_kernel = (lambda k: "quantize_mxfp8_kernel" in k) if quant else (lambda k: "gemm_kernel" in k)
    is_copy = lambda k: "copy" in k.lower()
    g_fetch, nd_f, gnames = _counter_per_dispatch(f(stem + "_fetch"), "FETCH_SIZE", is_kernel)
    g_write, nd_w, _ = _counter_per_dispatch(f(stem + "_write"), "WRITE_SIZE", is_kernel)
    c_fetch, _, cnames = _counter_per_dispatch(f("copy_fetch"), "FETCH_SIZE", is_copy)
    c_write, _, _ = _counter_per_dispatch(f("copy_write"), "WRITE_SIZE", is_copy)
    copy_bytes = COPY_BYTES
    kf = copy_bytes / (c_fetch * 1024.0)
    kw = copy_bytes / (c_write * 1024.0)
    fetch_b = g_fetch * 1024.0 * kf
    write_b = g_write * 1024.0 * kw
    if quant:
        alg = quant_bytes(w)
    else:
        per_elem = {"mxfp8_nt": 1.0, "mxfp4_nt": 0.5, "mxfp6_e2m3_nt": 0.75, "mxfp6_e3m2_nt": 0.75}.get(w.kind, 2.0)
        in_bytes = int((w.M + w.N) * w.K * per_elem)
        alg = in_bytes + w.M * w.N * 2
    rec = {"workload": name, "kernel_source_sha256_16": kernel_source_hash(src=source_of(w.kind)),
           "kernel": gnames, "dispatches": [nd_f, nd_w],
           "fetch_kib_per_dispatch": round(g_fetch, 1), "write_kib_per_dispatch": round(g_write, 1),
           "copy_kernel": cnames, "copy_bytes": copy_bytes,
           "copy_fetch_kib": round(c_fetch, 1), "copy_write_kib": round(c_write, 1),
           "fetch_scale": round(kf, 4), "write_scale": round(kw, 4),
           "hbm_read_bytes_per_launch": int(fetch_b), "hbm_write_bytes_per_launch": int(write_b),
           "hbm_bytes_per_launch": int(fetch_b + write_b),
           "algorithmic_bytes_per_launch": alg,
           "traffic_over_algorithmic": round((fetch_b + write_b) / alg, 3)}
    out = os.path.join(d, f"traffic_{name}.json")
    json.dump(rec, open(out, "w"), indent=1)
    print(json.dumps(rec))


def quant_bytes(w) -> int:
    """Algorithmic bytes of one quantiser launch: x read once, q and the
    scales written once."""
    return w.M * w.K * 4 + w.M * w.K + w.M * ((w.K + 127) // 128)


def bench_quantize(args, w):
    """The block-scale quantiser: HBM-bound, reported in GB/s against the
    8 TB/s HBM peak."""
    import numpy as np
    import torch
    import dense_tiled_gemm_bf16_amd as tg
    import oracle
    torch.cuda.set_device(0)
    tg.init()
    import workloads
    x = workloads.make_inputs(w)["X"]
    xd = torch.from_numpy(x).cuda()
    KB = (w.K + 127) // 128
    q = torch.empty((w.M, w.K), dtype=torch.uint8, device="cuda")
    s = torch.empty((w.M, KB), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    L = tg.lib()
    argv = (w.M, w.K, xd.data_ptr(), q.data_ptr(), s.data_ptr(), stream.cuda_stream)

    def launch():
        rc = L.quantize_mxfp8(*argv)
        if rc != 0:
            raise RuntimeError(f"quantize_mxfp8: [{rc}] {tg.last_error()}")

    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            launch()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0.record(stream)
        for _ in range(args.steps):
            launch()
        t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    nbytes = quant_bytes(w)
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"[bench] {w.description}: {ms*1e3:.2f} us/launch, {gbs:.0f} GB/s of {PEAK_HBM_GBS}")
    parity = None
    if not args.no_parity:
        rows = np.arange(0, w.M, max(1, w.M // 64))
        qr, sr = oracle.quantize_mxfp8(x[rows])
        parity = {"rows_checked": int(rows.size),
                  "elements_differing": int((q.cpu().numpy()[rows] != qr).sum()),
                  "scales_differing": int((s.cpu().numpy()[rows] != sr).sum())}
        log(f"[bench] parity sample: {parity}")
    cpu = None
    if args.cpu_seconds > 0:
        # Whole passes over the workload until about cpu_seconds of work.
        threads = oracle.num_threads()
        passes, t = 0, time.perf_counter()
        while passes == 0 or time.perf_counter() - t < args.cpu_seconds:
            oracle.quantize_mxfp8(x)
            passes += 1
        dt = time.perf_counter() - t
        cpu = {"value": round(nbytes * passes / dt / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
               "sample": f"{passes} whole passes of {w.name} through the oracle quantiser, {dt:.1f} s"}
    line = {
        "metric": f"GB/s (algorithmic bytes / t), {w.description}, 1 GPU",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32->fp8e4m3+e8m0", "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "K": w.K},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": measured_traffic(w.name),
                     "kernel_mean_us": round(ms * 1e3, 2), "bytes_per_launch": nbytes},
        "cpu_baseline": cpu, "parity": parity,
    }
    print(json.dumps(line), flush=True)


class ClockProbe:
    """The shader clock delivered between two probes, per XCD: the library's
    clock probe (tgemm_clock_probe) records, on every CU, that CU's
    shader-clock counter and the constant-rate counter; each CU's pair of
    records gives its average clock between the probes, and an XCD's is the
    mean over its CUs (they agree to a few MHz within an XCD)."""

    RECORDS = 256

    def __init__(self):
        import ctypes
        import torch
        self.buf = torch.zeros((2, 4 * self.RECORDS), dtype=torch.int64, device="cuda")
        self.khz = ctypes.c_int(0)

    def sample(self, slot: int, stream) -> None:
        import ctypes
        import dense_tiled_gemm_bf16_amd as tg
        tg.check(tg.lib().tgemm_clock_probe(ctypes.c_void_p(self.buf[slot].data_ptr()), ctypes.byref(self.khz),
                                            ctypes.c_void_p(stream.cuda_stream)))

    def _records(self, slot):
        """{(xcc, se/sh/cu bits): (shader-clock count, constant-rate count)}."""
        b = self.buf[slot].cpu().numpy().reshape(self.RECORDS, 4)
        out = {}
        for rec in b:
            key = (int(rec[0]) >> 32, (int(rec[0]) >> 8) & 0xFF)
            out.setdefault(key, (int(rec[1]), int(rec[2])))
        return out

    def ghz(self) -> dict:
        """{xcd: GHz} between the probes in slots 0 and 1 (after a synchronisation)."""
        rate = self.khz.value * 1e3
        r0, r1 = self._records(0), self._records(1)
        per = {}
        for key, (t0, c0) in r0.items():
            if key in r1 and rate > 0 and r1[key][1] > c0:
                per.setdefault(key[0], []).append((r1[key][0] - t0) / ((r1[key][1] - c0) / rate) / 1e9)
        return {x: sum(v) / len(v) for x, v in sorted(per.items())}


_graphs = {}


def timed_region(launch, stream, steps: int, between=None, graph: bool = False):
    """`steps` launches back to back on `stream` between two HIP events
    recorded on that stream; `between` runs before each launch (inside the
    region: the flush variant subtracts a region of flushes alone).  With
    `graph`, the launches (and flushes) are captured once into a HIP graph
    and the region replays it, so host launch costs do not enter the time.
    Returns (region ms, host wall s)."""
    import torch

    def body():
        for _ in range(steps):
            if between is not None:
                between()
            launch()

    if graph:
        key = (id(launch), id(between), steps)
        if key not in _graphs:
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=stream):
                body()
            torch.cuda.synchronize()
            _graphs[key] = g
        body = _graphs[key].replay
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        body()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1), time.perf_counter() - wall0


def launch_spread(launch, stream, steps: int, between=None):
    """`steps` launches, each between its own pair of HIP events on `stream`
    (`between` outside the pairs).  Returns the per-launch times in us.  Each
    event adds a marker to the stream, so these times include that overhead
    (a few us against the kernel trace); they give the spread, not the mean."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(steps):
            if between is not None:
                between()
            ev[2 * i].record(stream)
            launch()
            ev[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[2 * i].elapsed_time(ev[2 * i + 1]) * 1e3 for i in range(steps)]


def settle(launch, stream, seconds: float, kernel_us: float):
    """Launch in batches of about 20 ms, synchronising after each, until
    `seconds` of host time have passed (no timing).  Returns (launches, s)."""
    import torch
    batch = max(1, int(20e3 / max(kernel_us, 1.0)))
    n, t0 = 0, time.perf_counter()
    while seconds > 0 and time.perf_counter() - t0 < seconds:
        with torch.cuda.stream(stream):
            for _ in range(batch):
                launch()
        torch.cuda.synchronize()
        n += batch
    return n, time.perf_counter() - t0


def _stats(v):
    import statistics
    return {"mean": round(statistics.fmean(v), 3), "median": round(statistics.median(v), 3),
            "min": round(min(v), 3), "max": round(max(v), 3), "n": len(v)}


def _mean_ghz(d):
    return round(sum(d.values()) / len(d), 4) if d else None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000, help="launches per timed region")
    ap.add_argument("--warmup", type=int, default=50, help="untimed launches before the first timed region")
    ap.add_argument("--repeats", type=int, default=5,
                    help="timed regions of --steps launches after the settle phase; value = their median")
    ap.add_argument("--settle-s", type=float, default=2.0,
                    help="seconds of untimed launches between the cold region and the repeats, for the "
                         "power-limited clock to settle (recorded in the line; 0 disables)")
    ap.add_argument("--flush", action="store_true",
                    help="cold-cache variant: write a 512 MB buffer before every launch (outside the "
                         "launch's event pair); value from the per-launch kernel times")
    ap.add_argument("--workload", default="bf16_nt_4096x4096x8192")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU work for the oracle baseline (0 disables it)")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--tile", default="auto",
                    help="output tile TMxTN (e.g. 256x192); default: the library's own choice")
    ap.add_argument("--graph", action="store_true",
                    help="capture each timed region's launches into a HIP graph once and time its replay "
                         "(for kernels shorter than the host's launch cost)")
    ap.add_argument("--splitk", type=int, default=None, metavar="S",
                    help="16-bit workloads: call the K-split entry point with S splits (0: the library "
                         "chooses); default: the plain entry point")
    ap.add_argument("--record-traffic", metavar="DIR")
    ap.add_argument("--zero-elements", action="store_true",
                    help="clock diagnostic: A's and B's elements all zero (block scales kept), so the same "
                         "instruction stream runs without data-dependent switching; not the workload's data")
    args = ap.parse_args()

    if args.record_traffic:
        record_traffic(args.record_traffic, args.workload)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; --gpus must be 1 "
              "(the GEMM has no multi-GPU path to measure)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.repeats < 1:
        print("bench.py: --steps and --repeats must be >= 1, --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_tiled_gemm_bf16_amd as tg
    import workloads

    if args.copy_calibration:
        copy_calibration()
        return

    w = workloads.WORKLOADS[args.workload]
    if w.kind == "quant_mxfp8":
        bench_quantize(args, w)
        return
    prec = {"bf16_nt": "bf16", "f16_nn": "f16", "mxfp8_nt": "mxfp8", "mxfp4_nt": "mxfp4",
            "mxfp6_e2m3_nt": "mxfp6", "mxfp6_e3m2_nt": "mxfp6"}[w.kind]
    torch.cuda.set_device(0)
    tg.init()
    tile = None
    if args.tile != "auto":
        tile = tuple(int(v) for v in args.tile.lower().split("x"))
        tg.set_tile(*tile)
    log(f"[bench] {w.description}: generating inputs")
    x, dev = device_inputs(w)
    if args.zero_elements:
        import numpy as np
        for k in ("A", "B", "qA", "qB"):
            if k in x:
                x[k] = np.zeros_like(x[k])
                dev[k].zero_()
    out_dtype = torch.float16 if w.kind == "f16_nn" else torch.bfloat16
    out = torch.empty((w.M, w.N), dtype=out_dtype, device="cuda")
    stream = torch.cuda.Stream()
    if args.splitk is not None and w.kind not in ("bf16_nt", "f16_nn"):
        print("bench.py: --splitk is for the 16-bit workloads", file=sys.stderr)
        sys.exit(2)
    launch = launcher(w, dev, out, stream, args.splitk)
    probe = ClockProbe()
    noop = lambda: None
    between = None
    if args.flush:
        flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        fills = [0]

        def between():
            fills[0] += 1
            flush_buf.fill_(fills[0] & 255)
    torch.cuda.synchronize()
    peak = PEAK_TFLOPS[prec]
    tfl = lambda us: w.flops / (us / 1e6) / 1e12

    # 1. The untimed warmup launches, then the first timed region: exactly
    #    the launches a short run makes, at whatever clock the chip has then.
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            if between is not None:
                between()
            launch()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        probe.sample(0, stream)
    c_ms, _ = timed_region(launch, stream, args.steps, between, args.graph)
    with torch.cuda.stream(stream):
        probe.sample(1, stream)
    torch.cuda.synchronize()
    c_ghz = probe.ghz()
    if between is not None:
        c_ms -= timed_region(noop, stream, args.steps, between, args.graph)[0]
    cold = {"warmup": args.warmup, "steps": args.steps, "ms_per_step": round(c_ms / args.steps, 5),
            "tflops": round(w.flops * args.steps / (c_ms / 1e3) / 1e12, 2), "clock_ghz": _mean_ghz(c_ghz)}
    log(f"[bench] first region ({args.warmup} warmup + {args.steps} timed launches): {cold['tflops']:.1f} TFLOPS, "
        f"{c_ms / args.steps * 1e3:.1f} us/launch, clock {cold['clock_ghz']} GHz")

    # 2. Untimed launches until the power-limited clock has settled.
    with torch.cuda.stream(stream):
        probe.sample(0, stream)
    n_settle, s_settle = settle(launch if between is None else (lambda: (between(), launch())), stream,
                                args.settle_s, c_ms / args.steps * 1e3)
    with torch.cuda.stream(stream):
        probe.sample(1, stream)
    torch.cuda.synchronize()
    settle_ghz = probe.ghz()
    log(f"[bench] settle: {n_settle} launches in {s_settle:.2f} s, clock {_mean_ghz(settle_ghz)} GHz")

    # 3. The timed regions: `repeats` regions of exactly `steps` launches,
    #    bracketed together by one pair of clock probes.
    regions = []
    with torch.cuda.stream(stream):
        probe.sample(0, stream)
    for r in range(args.repeats):
        ms, wall = timed_region(launch, stream, args.steps, between, args.graph)
        if between is not None:
            # Flush variant: the same region with the flushes alone, right
            # after; the difference is the launches' own time.
            fl_ms, _ = timed_region(noop, stream, args.steps, between, args.graph)
            ms -= fl_ms
        regions.append({"ms": ms, "wall_s": wall, "tflops": w.flops * args.steps / (ms / 1e3) / 1e12})
        log(f"[bench] region {r}: {args.steps} launches in {ms:.3f} ms (wall {wall*1e3:.1f} ms): "
            f"{regions[-1]['tflops']:.1f} TFLOPS, {ms / args.steps * 1e3:.2f} us/launch")
    with torch.cuda.stream(stream):
        probe.sample(1, stream)
    torch.cuda.synchronize()
    rep_ghz = probe.ghz()

    # 4. The spread of single launches (event pair around each).
    spread = _stats(launch_spread(launch, stream, args.steps, between))

    order = sorted(range(len(regions)), key=lambda i: regions[i]["tflops"])
    med = regions[order[len(order) // 2]]
    tflops = med["tflops"]
    ms_per_step = med["ms"] / args.steps
    kernel_us = ms_per_step * 1e3
    achieved = tfl(kernel_us)
    log(f"[bench] median region: {tflops:.1f} TFLOPS = {100*tflops/peak:.1f}% of {peak}; kernel "
        f"{kernel_us:.2f} us -> {achieved:.1f} TFLOP/s = {100*achieved/peak:.1f}%; clock over the regions "
        f"{_mean_ghz(rep_ghz)} GHz; single launches (event pair each) median {spread['median']:.2f} us, "
        f"min {spread['min']:.2f}, max {spread['max']:.2f}")

    parity = None if args.no_parity else parity_sample(w, x, out)
    if parity is not None:
        log(f"[bench] parity sample: {parity}")

    cpu = None
    if args.cpu_seconds > 0:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, x, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']*1e3:.3f} GFLOPS on {cpu['cores']} threads ({cpu['sample']})")
        cpu.pop("seconds", None)

    traffic = None if args.flush else measured_traffic(w.name)
    metric = METRIC if w.name == "bf16_nt_4096x4096x8192" else f"TFLOPS (2MNK/t), {w.description}, 1 GPU"
    if args.flush:
        metric += ", cold cache (512 MB written before each launch, the flushes' own time subtracted)"
    line = {
        "metric": metric,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f16": "f16", "mxfp8": "fp8e4m3+e8m0", "mxfp4": "fp4e2m1+e8m0",
                  "mxfp6": f"fp6{workloads.fp6_format(w.kind) if prec == 'mxfp6' else ''}+e8m0"}[prec],
        "data": "synthetic, A and B elements all zero (clock diagnostic)" if args.zero_elements else "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "layout": "NT" if w.kind != "f16_nn" else "NN",
                   "accumulate": "fp32",
                   "tile": (f"{tile[0]}x{tile[1]}" if tile else "auto") + ", 4 waves, 128-byte K slices",
                   "entry": "gemm_bf16_splitk / gemm_f16_splitk, splits=%d" % args.splitk
                            if args.splitk is not None else "plain",
                   "pct_of_peak": round(100 * tflops / peak, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_mean_us": round(kernel_us, 3), "flops_per_launch": w.flops,
                     "kernel_time_source": "median timed region: two HIP events on the launch stream around "
                                           f"{args.steps} back-to-back launches, one kernel per launch" +
                                           (", less the same region of flushes alone" if args.flush else "")},
        "timing": {
            "repeats": args.repeats,
            "region_tflops": {"median": round(med["tflops"], 2),
                              "min": round(regions[order[0]]["tflops"], 2),
                              "max": round(regions[order[-1]]["tflops"], 2)},
            "single_launch_us": dict(spread, note="an event pair around each launch; the markers add a few us "
                                                  "to each"),
            "clock_ghz": {"timed_regions": _mean_ghz(rep_ghz), "settle": _mean_ghz(settle_ghz),
                          "first_region": _mean_ghz(c_ghz),
                          "per_xcd_timed_regions": {str(k): round(v, 4) for k, v in rep_ghz.items()},
                          "source": "tgemm_clock_probe before and after the first region, the settle phase and "
                                    "the set of timed regions (flushes included, if any): s_memtime against "
                                    "s_memrealtime, paired per CU, mean over each XCD's CUs, then over the XCDs"},
            "settle": {"seconds": round(s_settle, 2), "launches": n_settle,
                       "why": "untimed launches between the first region and the timed regions; under sustained "
                              "load the board holds its power limit and the clock settles over about a second"},
            "first_region": cold,
            "flush": bool(args.flush),
            "graph": bool(args.graph),
        },
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
