#!/usr/bin/env python3
"""Throughput of the tiled dense GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one C = A . B^T launch through the C ABI (gemm_bf16_nt) on the
bf16 NT 4096 x 4096 x 8192 workload, inputs already resident in HBM.
W untimed steps, then K timed steps between two synchronisations; the
throughput is 2 M N K K / t (the pages' TFLOPS formula, TileLang SM100
README, "Compilation and Usage").  Prints ONE JSON line on stdout; context
goes to stderr.

The line carries:
  roofline     the kernel against MI355X's dense bf16 MFMA peak: algorithmic
               flops per launch over the kernel's mean duration, measured
               with HIP events recorded around single launches on the stream
               the kernel runs on; `traffic` is the HBM bytes per launch from
               rocprofv3 FETCH_SIZE/WRITE_SIZE counters when a committed
               measurement matches the current kernel source, else null;
  cpu_baseline the CPU oracle (binary64 triple loop, all host threads) timed
               on a bounded sample of the same workload: whole rows of C,
               scaled to TFLOPS.
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

PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "mxfp8": 5033.2}  # MI355X dense MFMA, 256 CU x 2.4 GHz
METRIC = "TFLOPS (2MNK/t) and % of MFMA peak, bf16 NT GEMM 4096x4096x8192, 1 GPU"
KERNEL_SRC = os.path.join(ROOT, "dense_tiled_gemm_bf16_amd", "csrc", "tgemm_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_bf16_nt_4096x4096x8192.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from a committed counter run, if it was taken on
    the current kernel source; else None."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("workload") != name or rec.get("kernel_source_sha256_16") != kernel_source_hash():
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


def launcher(w, dev, out, stream):
    import dense_tiled_gemm_bf16_amd as tg
    L = tg.lib()
    s = stream.cuda_stream
    M, N, K = w.M, w.N, w.K
    if w.kind == "bf16_nt":
        args = (M, N, K, dev["A"].data_ptr(), dev["B"].data_ptr(), out.data_ptr(), s)
        fn = L.gemm_bf16_nt
    elif w.kind == "f16_nn":
        args = (M, N, K, dev["A"].data_ptr(), dev["B"].data_ptr(), out.data_ptr(), s)
        fn = L.gemm_f16_nn
    else:
        args = (M, N, K, dev["qA"].data_ptr(), dev["qB"].data_ptr(), dev["sA"].data_ptr(),
                dev["sB"].data_ptr(), out.data_ptr(), s)
        fn = L.gemm_mxfp8_nt

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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_nt_4096x4096x8192")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU work for the oracle baseline (0 disables it)")
    ap.add_argument("--no-parity", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this library runs on one GPU; --gpus must be 1 "
              "(the GEMM has no multi-GPU path to measure)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_tiled_gemm_bf16_amd as tg
    import workloads

    w = workloads.WORKLOADS[args.workload]
    prec = {"bf16_nt": "bf16", "f16_nn": "f16", "mxfp8_nt": "mxfp8"}[w.kind]
    torch.cuda.set_device(0)
    tg.init()
    log(f"[bench] {w.description}: generating inputs")
    x, dev = device_inputs(w)
    out_dtype = torch.float16 if w.kind == "f16_nn" else torch.bfloat16
    out = torch.empty((w.M, w.N), dtype=out_dtype, device="cuda")
    stream = torch.cuda.Stream()
    launch = launcher(w, dev, out, stream)
    torch.cuda.synchronize()

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            launch()
    torch.cuda.synchronize()

    # Timed region: K back-to-back launches.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    with torch.cuda.stream(stream):
        t_start.record(stream)
        for _ in range(args.steps):
            launch()
        t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    tflops = w.flops * args.steps / (total_ms / 1e3) / 1e12

    # Kernel duration: event pairs around single launches on the kernel's stream.
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(max(10, min(args.steps, 50)))]
    with torch.cuda.stream(stream):
        for e0, e1 in pairs:
            e0.record(stream)
            launch()
            e1.record(stream)
    torch.cuda.synchronize()
    durs = sorted(e0.elapsed_time(e1) for e0, e1 in pairs)
    kernel_ms = sum(durs) / len(durs)
    achieved = w.flops / (kernel_ms / 1e3) / 1e12
    peak = PEAK_TFLOPS[prec]
    log(f"[bench] {args.steps} steps in {total_ms:.3f} ms (wall {wall*1e3:.1f} ms): "
        f"{ms_per_step*1e3:.1f} us/step, {tflops:.1f} TFLOPS = {100*tflops/peak:.1f}% of {peak}")
    log(f"[bench] kernel mean {kernel_ms*1e3:.1f} us (min {durs[0]*1e3:.1f}, max {durs[-1]*1e3:.1f}) "
        f"-> {achieved:.1f} TFLOPS, {100*achieved/peak:.1f}% of peak")

    parity = None if args.no_parity else parity_sample(w, x, out)
    if parity is not None:
        log(f"[bench] parity sample: {parity}")

    cpu = None
    if args.cpu_seconds > 0:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, x, args.cpu_seconds)
        log(f"[bench] cpu oracle: {cpu['value']*1e3:.3f} GFLOPS on {cpu['cores']} threads ({cpu['sample']})")
        cpu.pop("seconds", None)

    traffic = measured_traffic(w.name)
    line = {
        "metric": METRIC if w.name == "bf16_nt_4096x4096x8192" else f"TFLOPS (2MNK/t), {w.description}, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f16": "f16", "mxfp8": "fp8e4m3+e8m0"}[prec],
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "layout": "NT" if w.kind != "f16_nn" else "NN",
                   "accumulate": "fp32", "tile": "256x256, 4 waves, 128-byte K slices",
                   "pct_of_peak": round(100 * tflops / peak, 2)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel_mean_us": round(kernel_ms * 1e3, 2),
                     "flops_per_launch": w.flops},
        "cpu_baseline": cpu,
        "parity": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
