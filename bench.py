#!/usr/bin/env python3
"""Throughput of the fused Q4_0 dequantize-and-multiply GEMV at one token on
the Llama-3-8B projection shapes, on one MI355X.

One step = one call of qgemv_q4_0 (M = 1) on each of the six shapes
(4096x4096 o_proj, 6144x4096 qkv, 14336x4096 up, 4096x14336 down,
28672x4096 gate_up, 128256x4096 lm_head) [sm8x-bench, the Q4_0 table].
Every shape cycles through at least 1 GiB of distinct weight copies, so each
call streams its weights from HBM and not from the 256 MB last-level cache
[volta-kernel-bakeoff, "Making it fair": cycle enough copies that every call
reads from memory].

value    = algorithmic bytes of all K timed steps / wall time of the K steps
           (inputs resident in HBM; launch gaps included).
roofline = the GEMV kernel's own time, from HIP events recorded by each
           launch (hipExtLaunchKernel), against 8 TB/s; algorithmic bytes per
           call = N*K/32*18 (codes + scales) + 2*K (x) + 4*N (y).
cpu_baseline = the CPU oracle (fp64 C, OpenMP) on a bounded row sample of the
           same shapes, in the same unit.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import seeded_inputs as si  # noqa: E402

PEAK_GBPS = 8000.0
METRIC = "Q4_0 GEMV HBM GB/s and % of 8 TB/s peak at M=1; µs/call per shape"
COPY_BYTES = 1 << 30


def algorithmic_bytes(N: int, K: int, M: int = 1) -> int:
    return N * K // 32 * 18 + 2 * M * K + 4 * M * N


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_workload(qg, torch):
    """Packed weights (library host packer), >= 1 GiB of copies per shape."""
    work = []
    for (N, K) in si.LLAMA3_8B_SHAPES:
        t0 = time.perf_counter()
        w = si.weights(N, K, seed=0)
        packed = qg.qquantize_q4_0(w)
        del w
        nb = packed.size
        copies = max(2, math.ceil(COPY_BYTES / nb))
        buf = torch.empty(copies * nb, dtype=torch.uint8, device="cuda")
        first = torch.from_numpy(packed).to("cuda")
        for c in range(copies):
            buf[c * nb:(c + 1) * nb].copy_(first)
        del first
        x = torch.from_numpy(si.activations(1, K, seed=0)).to("cuda")
        y = torch.empty((1, N), dtype=torch.float32, device="cuda")
        work.append(dict(N=N, K=K, nb=nb, copies=copies, buf=buf, x=x, y=y, next=0,
                         bytes=algorithmic_bytes(N, K)))
        log(f"shape {N}x{K}: {copies} copies x {nb} B ({time.perf_counter() - t0:.1f} s)")
    torch.cuda.synchronize()
    return work


def run_step(qg, work, timer=None):
    for w in work:
        c = w["next"]
        w["next"] = (c + 1) % w["copies"]
        nb = w["nb"]
        if timer is not None:
            timer.arm()
        qg.qgemv_q4_0(w["buf"][c * nb:(c + 1) * nb], w["x"], w["N"], w["K"], w["y"])


def hbm_probe(qg, torch, gib: int = 4, reps: int = 5) -> float:
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    wgs = qg.qg_device_cus() * 8
    sink = torch.empty(wgs, dtype=torch.int32, device="cuda")
    timer = qg.KernelTimer(reps + 1)
    qg.qg_read_probe(buf, sink, wgs)
    for _ in range(reps):
        timer.arm()
        qg.qg_read_probe(buf, sink, wgs)
    torch.cuda.synchronize()
    ms = timer.elapsed_ms()
    timer.close()
    del buf
    return (gib << 30) / (min(ms) * 1e-3) / 1e9


def cpu_baseline(seconds: float) -> dict:
    """The oracle (fp64 C, OpenMP over rows) on a row sample of each shape."""
    import oracle
    o = oracle.get()
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    done_bytes = 0
    elapsed = 0.0
    per_shape = seconds / len(si.LLAMA3_8B_SHAPES)
    sample = []
    for (N, K) in si.LLAMA3_8B_SHAPES:
        rows = min(N, 2048)
        w = si.weights(rows, K, seed=0)   # the first `rows` rows' worth of the same distribution
        p = o.quantize(oracle.Q4_0, w)
        x = si.activations(1, K, seed=0)
        t_shape = 0.0
        reps = 0
        while t_shape < per_shape:
            t0 = time.perf_counter()
            o.gemv(oracle.Q4_0, p, rows, K, x)
            t_shape += time.perf_counter() - t0
            reps += 1
        done_bytes += reps * algorithmic_bytes(rows, K)
        elapsed += t_shape
        sample.append(f"{rows}x{K} x{reps}")
    return {"value": round(done_bytes / elapsed / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "oracle GEMV (fp64, M=1) on the first min(N, 2048) rows of each shape, repeated for "
                      f"{seconds:.0f} s in total: " + ", ".join(sample)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-probe", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the GEMV path runs on a single MI355X (no collectives); "
              "run it with --gpus 1", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import quantized_weight_gemv_amd as qg
    qg.lib()

    work = build_workload(qg, torch)
    step_bytes = sum(w["bytes"] for w in work)

    for _ in range(args.warmup):
        run_step(qg, work)
    torch.cuda.synchronize()

    timer = qg.KernelTimer(args.steps * len(work))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(qg, work, timer)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array(timer.elapsed_ms()).reshape(args.steps, len(work))
    timer.close()

    value = step_bytes * args.steps / wall / 1e9
    kern_us = ms.mean(axis=0) * 1e3
    per_shape = {}
    for w, us, med in zip(work, kern_us, np.median(ms, axis=0) * 1e3):
        gbps = w["bytes"] / (us * 1e-6) / 1e9
        per_shape[f"{w['N']}x{w['K']}"] = {"us_per_call": round(float(us), 3), "us_median": round(float(med), 3),
                                           "GBps": round(gbps, 1), "pct_of_8TBps": round(gbps / PEAK_GBPS * 100, 2),
                                           "algorithmic_bytes": w["bytes"], "copies": w["copies"]}
    kernel_s_per_step = ms.sum(axis=1).mean() * 1e-3
    achieved = step_bytes / kernel_s_per_step / 1e9

    probe = None if args.no_probe else round(hbm_probe(qg, torch), 1)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16*f16->f32",
        "data": "synthetic",
        "config": {"workload": "Q4_0 GEMV, M=1, Llama-3-8B projection shapes N x K = "
                               + ", ".join(f"{n}x{k}" for n, k in si.LLAMA3_8B_SHAPES)
                               + "; weights N(0,0.02) fp32 quantized per 32-block, activations N(0,1) fp16, "
                                 "fp32 out, seed 0; >= 1 GiB of weight copies cycled per shape",
                   "M": 1, "shapes": [f"{n}x{k}" for n, k in si.LLAMA3_8B_SHAPES],
                   "step": "one qgemv_q4_0 call per shape"},
        "pct_of_8TBps": round(value / PEAK_GBPS * 100, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": None,
                     "kernel": "qg::gemv_kernel (Q4_0, M=1)",
                     "note": "algorithmic bytes of the six calls / sum of their kernel times (HIP events "
                             "recorded by each launch)"},
        "per_shape": per_shape,
        "hbm_probe_GBps": probe,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
