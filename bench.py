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
           (inputs resident in HBM; launch gaps included), the K steps
           replayed as one captured HIP graph (eager launch time reported
           beside it; --no-graph times value eagerly).
roofline = the GEMV kernel's own time, from HIP events recorded by each
           launch (hipExtLaunchKernel) over a second pass of K steps, against
           8 TB/s; algorithmic bytes per call = N*K/32*18 (codes + scales) +
           2*K (x) + 4*N (y).
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


def measured_traffic():
    """HBM bytes per step from the committed rocprofv3 counter summary, if it
    was taken on the GEMV sources as they are now; otherwise None."""
    path = os.path.join(ROOT, "profiles", "gemv_q4_0_llama3_8b_m1_traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
        from rocprof_summary import gemv_source_hash
        if d.get("gemv_source_sha256") != gemv_source_hash():
            return None
        return int(d["traffic_bytes_per_step"])
    except (OSError, ValueError, KeyError):
        return None


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
        # one validated call per copy: the timed loop only enqueues kernels
        calls = [qg.PreparedGemv(qg.Q4_0, buf[c * nb:(c + 1) * nb], x, y, N, K) for c in range(copies)]
        work.append(dict(N=N, K=K, nb=nb, copies=copies, buf=buf, x=x, y=y, next=0, calls=calls,
                         bytes=algorithmic_bytes(N, K)))
        log(f"shape {N}x{K}: {copies} copies x {nb} B ({time.perf_counter() - t0:.1f} s)")
    torch.cuda.synchronize()
    return work


def run_step(work, timer=None):
    for w in work:
        c = w["next"]
        w["next"] = (c + 1) % w["copies"]
        if timer is not None:
            timer.arm()
        w["calls"][c]()


def per_shape_graph_us(qg, torch, work, calls_per_shape: int = 64) -> dict:
    """Microseconds per call of each shape launched back to back: one captured
    graph of `calls_per_shape` consecutive calls (cycling the copies), replayed
    once and timed with stream events around the replay.  Unlike per-launch
    events this includes the dispatch gap between calls and nothing else."""
    out = {}
    for w in work:
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            calls = [qg.PreparedGemv(qg.Q4_0, w["buf"][c * w["nb"]:(c + 1) * w["nb"]], w["x"], w["y"], w["N"],
                                     w["K"]) for c in range(w["copies"])]
            with torch.cuda.graph(g, stream=cap):
                for i in range(calls_per_shape):
                    calls[i % w["copies"]]()
        torch.cuda.synchronize()
        g.replay()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        out[f"{w['N']}x{w['K']}"] = s.elapsed_time(e) * 1e3 / calls_per_shape
        del g
    return out


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


# ------------------------------------------------------------------- suite
def _copies(torch, packed: np.ndarray, min_bytes: int = COPY_BYTES):
    nb = packed.size
    copies = max(2, math.ceil(min_bytes / nb))
    buf = torch.empty(copies * nb, dtype=torch.uint8, device="cuda")
    first = torch.from_numpy(packed).to("cuda")
    for c in range(copies):
        buf[c * nb:(c + 1) * nb].copy_(first)
    return buf, nb, copies


def _time_calls(qg, torch, calls, reps: int, warm: int = 5):
    """Median / mean kernel time (us) of `reps` calls, rotating through `calls`,
    from the HIP events each launch records."""
    for i in range(warm):
        calls[i % len(calls)]()
    timer = qg.KernelTimer(reps)
    for i in range(reps):
        timer.arm()
        calls[(i + warm) % len(calls)]()
    ms = np.array(timer.elapsed_ms())
    timer.close()
    return float(np.median(ms) * 1e3), float(ms.mean() * 1e3)


def _time_wall(torch, fns, reps: int, warm: int = 5):
    """Per-call time (us) from torch events around each call on the current
    stream (includes every kernel a call launches and the gaps between them)."""
    for i in range(warm):
        fns[i % len(fns)]()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        ev[i][0].record()
        fns[(i + warm) % len(fns)]()
        ev[i][1].record()
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return float(np.median(ms) * 1e3), float(ms.mean() * 1e3)


def suite(qg, torch, reps: int):
    """Every workload of the library, one JSON record each."""
    out = []
    cus = qg.qg_device_cus()

    def rec(**kw):
        out.append(kw)
        log(json.dumps(kw))

    # GEMV: 2048x2048 seed 0 and the small-batch shapes, both formats, M = 1, 2, 4, 8
    gemv_cases = [(qg.Q4_0, 2048, 2048, 1)]
    for fmt in (qg.Q4_0, qg.Q8_0):
        for (N, K) in si.SMALL_BATCH_SHAPES:
            for M in (1, 2, 4, 8):
                gemv_cases.append((fmt, N, K, M))
    packed_cache = {}
    for fmt, N, K, M in gemv_cases:
        key = (fmt, N, K)
        if key not in packed_cache:
            packed_cache.clear()
            w = si.weights(N, K, seed=0)
            packed_cache[key] = _copies(torch, qg.qquantize_q4_0(w) if fmt == qg.Q4_0 else qg.qquantize_q8_0(w))
        buf, nb, copies = packed_cache[key]
        x = torch.from_numpy(si.activations(M, K, seed=0)).to("cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        calls = [qg.PreparedGemv(fmt, buf[c * nb:(c + 1) * nb], x, y, N, K) for c in range(copies)]
        med, mean = _time_calls(qg, torch, calls, reps)
        b = N * K // 32 * (18 if fmt == qg.Q4_0 else 34) + 2 * M * K + 4 * M * N
        rec(kind="gemv", fmt="q4_0" if fmt == qg.Q4_0 else "q8_0", N=N, K=K, M=M, us_median=round(med, 3),
            us_mean=round(mean, 3), GBps=round(b / med / 1e3, 1), pct_of_8TBps=round(b / med / 1e3 / 80, 2),
            algorithmic_bytes=b, copies=copies)
    packed_cache.clear()

    # MoE: a pool of P experts replicated to >= 1 GiB; fresh distinct indices per call
    for (P, E, N, K) in si.MOE_CONFIGS:
        pw = si.expert_pool(P, N, K, seed=0)
        pool = np.concatenate([qg.qquantize_q4_0(pw[j]) for j in range(P)])
        del pw
        buf, nb, copies = _copies(torch, pool)
        ncalls = 64
        idx = torch.from_numpy(np.stack([si.expert_indices(P, E, seed=0, call=c) for c in range(ncalls)])).cuda()
        x = torch.from_numpy(si.activations(E, K, seed=0)).to("cuda")
        y = torch.empty((E, N), dtype=torch.float32, device="cuda")
        fns = []
        for c in range(max(copies, ncalls)):
            pool_c = buf[(c % copies) * nb:(c % copies + 1) * nb]
            fns.append(lambda pc=pool_c, ic=idx[c % ncalls]: qg.qmoe_gemv_q4_0(pc, P, ic, x, N, K, y))
        med, mean = _time_calls(qg, torch, fns, reps)
        b = E * (N * K // 32 * 18 + 2 * K + 4 * N)
        rec(kind="moe", fmt="q4_0", P=P, E=E, N=N, K=K, us_median=round(med, 3), us_mean=round(mean, 3),
            GBps=round(b / med / 1e3, 1), pct_of_8TBps=round(b / med / 1e3 / 80, 2), algorithmic_bytes=b,
            pool_copies=copies)
        del buf

    # plain 2-bit weights (q2w), beside Q4_0 on the same shapes
    q2_cases = [(N, K, 1) for (N, K) in si.LLAMA3_8B_SHAPES] + \
        [(N, K, M) for (N, K) in si.SMALL_BATCH_SHAPES for M in (1, 2, 4, 8)]
    for (N, K, M) in q2_cases:
        w = si.weights(N, K, seed=0)
        buf, nb, copies = _copies(torch, qg.qquantize_q2w(w))
        x = torch.from_numpy(si.activations(M, K, seed=0)).to("cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        calls = [qg.PreparedGemv(qg.Q2W, buf[c * nb:(c + 1) * nb], x, y, N, K) for c in range(copies)]
        med, mean = _time_calls(qg, torch, calls, reps)
        i8med = None
        if M <= 4:   # the same weights against activations quantized to 8-bit blocks
            c8 = [lambda c=c: qg.qgemv_q2w_q8act(buf[c * nb:(c + 1) * nb], x, N, K, y) for c in range(copies)]
            i8med, _ = _time_calls(qg, torch, c8, reps)
        lutmed = None
        if M == 1 and K <= 4096:   # the same weights through per-pair lookup tables
            cl = [lambda c=c: qg.qgemv_q2w_lut(buf[c * nb:(c + 1) * nb], x, N, K, y) for c in range(copies)]
            lutmed, _ = _time_calls(qg, torch, cl, reps)
        del buf
        buf4, nb4, copies4 = _copies(torch, qg.qquantize_q4_0(w))
        del w
        c4 = [qg.PreparedGemv(qg.Q4_0, buf4[c * nb4:(c + 1) * nb4], x, y, N, K) for c in range(copies4)]
        med4, _ = _time_calls(qg, torch, c4, reps)
        del buf4
        b = N * K // 32 * 10 + 2 * M * K + 4 * M * N
        rec(kind="q2w", fmt="q2w", N=N, K=K, M=M, us_median=round(med, 3), us_mean=round(mean, 3),
            GBps=round(b / med / 1e3, 1), pct_of_8TBps=round(b / med / 1e3 / 80, 2), algorithmic_bytes=b,
            q4_0_us_median=round(med4, 3),
            int8_activations_us_median=None if i8med is None else round(i8med, 3),
            lookup_table_us_median=None if lutmed is None else round(lutmed, 3), copies=copies)

    # activations quantized to 8-bit blocks inside the launch (int8 dot
    # products), beside the fp16-activation GEMV on the same weights
    q8_cases = [(N, K, 1) for (N, K) in si.LLAMA3_8B_SHAPES] + \
        [(N, K, M) for (N, K) in si.SMALL_BATCH_SHAPES for M in (1, 2, 4)]
    for (N, K, M) in q8_cases:
        buf, nb, copies = _copies(torch, qg.qquantize_q4_0(si.weights(N, K, seed=0)))
        x = torch.from_numpy(si.activations(M, K, seed=0)).to("cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        fns = [lambda c=c: qg.qgemv_q4_0_q8act(buf[c * nb:(c + 1) * nb], x, N, K, y) for c in range(copies)]
        med, mean = _time_calls(qg, torch, fns, reps)
        f16 = [qg.PreparedGemv(qg.Q4_0, buf[c * nb:(c + 1) * nb], x, y, N, K) for c in range(copies)]
        fmed, _ = _time_calls(qg, torch, f16, reps)
        b = N * K // 32 * 18 + 2 * M * K + 4 * M * N
        rec(kind="q8act", fmt="q4_0", N=N, K=K, M=M, us_median=round(med, 3), us_mean=round(mean, 3),
            GBps=round(b / med / 1e3, 1), pct_of_8TBps=round(b / med / 1e3 / 80, 2), algorithmic_bytes=b,
            fp16_activations_us_median=round(fmed, 3), copies=copies)
        del buf

    # fp32 activations rounded inside the kernel, beside the same call on
    # activations converted by a separate step (torch's .half()) first
    for (N, K, M) in si.F32IN_CASES:
        buf, nb, copies = _copies(torch, qg.qquantize_q4_0(si.weights(N, K, seed=0)))
        x = torch.from_numpy(si.activations32(M, K, seed=0)).to("cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        fns = [lambda c=c: qg.qgemv_q4_0_f32in(buf[c * nb:(c + 1) * nb], x, N, K, y) for c in range(copies)]
        med, mean = _time_calls(qg, torch, fns, reps)
        wmed, _ = _time_wall(torch, fns, reps)
        two = [lambda c=c: qg.qgemv_q4_0(buf[c * nb:(c + 1) * nb], x.half(), N, K, y) for c in range(copies)]
        smed, _ = _time_wall(torch, two, reps)
        b = N * K // 32 * 18 + 4 * M * K + 4 * M * N
        rec(kind="f32in", fmt="q4_0", N=N, K=K, M=M, us_median=round(med, 3), us_mean=round(mean, 3),
            GBps=round(b / med / 1e3, 1), pct_of_8TBps=round(b / med / 1e3 / 80, 2), algorithmic_bytes=b,
            wall_us_median=round(wmed, 3), separate_conversion_wall_us_median=round(smed, 3), copies=copies)
        del buf

    # gate + up stacked in one 2N-row table with SwiGLU in the epilogue, beside
    # the unfused steps (conversion, one GEMV over the stacked table, silu * up)
    for (N, K) in si.SWIGLU_SHAPES:
        w = np.concatenate([si.weights(N, K, seed=0), si.weights(N, K, seed=1)])
        buf, nb, copies = _copies(torch, qg.qquantize_q4_0(w))
        del w
        for M in si.SWIGLU_TOKENS:
            x = torch.from_numpy(si.activations32(M, K, seed=0)).to("cuda")
            y = torch.empty((M, N), dtype=torch.float32, device="cuda")
            gu = torch.empty((M, 2 * N), dtype=torch.float32, device="cuda")
            fns = [lambda c=c: qg.qgemv_q4_0_swiglu_f32in(buf[c * nb:(c + 1) * nb], x, N, K, y)
                   for c in range(copies)]
            med, mean = _time_calls(qg, torch, fns, reps)
            wmed, _ = _time_wall(torch, fns, reps)

            def unfused(c):
                qg.qgemv_q4_0(buf[c * nb:(c + 1) * nb], x.half(), 2 * N, K, gu)
                torch.mul(torch.nn.functional.silu(gu[:, :N]), gu[:, N:], out=y)
            ufn = [lambda c=c: unfused(c) for c in range(copies)]
            umed, _ = _time_wall(torch, ufn, reps)
            b = 2 * N * K // 32 * 18 + 4 * M * K + 4 * M * N
            rec(kind="swiglu", fmt="q4_0", N=N, K=K, M=M, us_median=round(med, 3), us_mean=round(mean, 3),
                GBps=round(b / med / 1e3, 1), pct_of_8TBps=round(b / med / 1e3 / 80, 2), algorithmic_bytes=b,
                wall_us_median=round(wmed, 3), unfused_wall_us_median=round(umed, 3), copies=copies)
        del buf
        torch.cuda.empty_cache()

    # prefill, and the dense fp16 GEMM on pre-dequantized weights beside it
    for (N, K) in si.PREFILL_SHAPES:
        w = si.weights(N, K, seed=0)
        buf, nb, copies = _copies(torch, qg.qquantize_q4_0(w))
        del w
        w16 = [qg.qdequant_q4_0(buf[c * nb:(c + 1) * nb], N, K, fp16=True).t().contiguous()
               for c in range(max(2, math.ceil(COPY_BYTES / (2 * N * K))))]
        for M in si.PREFILL_TOKENS:
            X = torch.from_numpy(si.activations(M, K, seed=0)).to("cuda")
            Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
            fns = [lambda c=c: qg.qgemm_q4_0_prefill(buf[c * nb:(c + 1) * nb], X, N, K, Y) for c in range(copies)]
            kmed, _ = _time_calls(qg, torch, fns, reps)
            med, mean = _time_wall(torch, fns, reps)
            dense = [lambda c=c: torch.matmul(X, w16[c]) for c in range(len(w16))]
            dmed, _ = _time_wall(torch, dense, reps)
            flops = 2 * M * N * K
            b = N * K // 32 * 18 + 2 * M * K + 4 * M * N
            rec(kind="prefill", fmt="q4_0", N=N, K=K, M=M, us_median=round(med, 3), us_mean=round(mean, 3),
                gemm_kernel_us_median=round(kmed, 3), TFLOPs=round(flops / med / 1e6, 1),
                pct_of_2500TF=round(flops / med / 1e6 / 25, 2), GBps=round(b / med / 1e3, 1),
                dense_fp16_us_median=round(dmed, 3), speedup_vs_dense=round(dmed / med, 3), copies=copies)
        del buf, w16
        torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time value with eager launches instead of a graph")
    ap.add_argument("--no-back-to-back", action="store_true",
                    help="skip the per-shape back-to-back pass (profiler runs: only interleaved steps)")
    ap.add_argument("--suite", default=None, metavar="FILE",
                    help="instead of the headline step, time every workload (GEMV both formats and M = 1..8, "
                         "MoE, prefill with its dense fp16 comparator) and write one JSON record per line to FILE")
    ap.add_argument("--reps", type=int, default=100)
    ap.add_argument("--q2w-calls", type=int, nargs=3, default=None, metavar=("N", "K", "CALLS"),
                    help="for counter passes: CALLS calls of the times-table kernel, then CALLS of the unpacking "
                         "q2w kernel, on one seeded N x K q2w table at one token; prints nothing else")
    ap.add_argument("--prefill-calls", type=int, nargs=4, default=None, metavar=("N", "K", "M", "CALLS"),
                    help="for counter passes: CALLS calls of the Q4_0 prefill on one seeded N x K table and M "
                         "tokens, then CALLS of the dense fp16 GEMM on its dequantized weights; prints nothing else")
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

    if args.q2w_calls:
        N, K, calls = args.q2w_calls
        W = torch.from_numpy(qg.qquantize_q2w(si.weights(N, K, seed=0))).to("cuda")
        x = torch.from_numpy(si.activations(1, K, seed=0)).to("cuda")
        y = torch.empty((1, N), dtype=torch.float32, device="cuda")
        for fn in (qg.qgemv_q2w_lut, qg.qgemv_q2w):
            for _ in range(calls):
                fn(W, x, N, K, y)
        torch.cuda.synchronize()
        return 0

    if args.prefill_calls:
        N, K, M, calls = args.prefill_calls
        W = torch.from_numpy(qg.qquantize_q4_0(si.weights(N, K, seed=0))).to("cuda")
        w16 = qg.qdequant_q4_0(W, N, K, fp16=True).t().contiguous()
        X = torch.from_numpy(si.activations(M, K, seed=0)).to("cuda")
        Y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        for _ in range(calls):
            qg.qgemm_q4_0_prefill(W, X, N, K, Y)
        for _ in range(calls):
            torch.matmul(X, w16)
        torch.cuda.synchronize()
        return 0

    if args.suite:
        recs = suite(qg, torch, args.reps)
        with open(args.suite, "w") as f:
            for r in recs:
                f.write(json.dumps(r) + "\n")
        return 0

    work = build_workload(qg, torch)
    step_bytes = sum(w["bytes"] for w in work)

    for _ in range(args.warmup):
        run_step(work)
    torch.cuda.synchronize()

    # Timed region 1 (value): K steps, captured once into a HIP graph and
    # replayed (the launch-bound loop as a graph; the copy rotation continues
    # exactly as eager launches would, so every call still reads cold copies),
    # bracketed by synchronizations.  The same K steps launched eagerly are
    # timed too and reported beside it.
    def timed_eager():
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            run_step(work)
        torch.cuda.synchronize()
        return time.perf_counter() - t

    eager_wall = timed_eager()
    wall = eager_wall
    graph_used = False
    if not args.no_graph:
        nexts = [w["next"] for w in work]
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            gcalls = [[qg.PreparedGemv(qg.Q4_0, w["buf"][c * w["nb"]:(c + 1) * w["nb"]], w["x"], w["y"], w["N"],
                                       w["K"]) for c in range(w["copies"])] for w in work]
            with torch.cuda.graph(graph, stream=cap):
                for _ in range(args.steps):
                    for w, calls in zip(work, gcalls):
                        c = w["next"]
                        w["next"] = (c + 1) % w["copies"]
                        calls[c]()
        torch.cuda.synchronize()
        for w, n in zip(work, nexts):   # warm the graph on the same copies, then time it
            w["next"] = n
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        graph_used = True

    # Timed region 2 (roofline): the same K steps, every launch recording its
    # own start and end (hipExtLaunchKernel events).  The event path costs
    # several microseconds of host time per launch, so this pass is not the
    # one `value` comes from.
    timer = qg.KernelTimer(args.steps * len(work))
    torch.cuda.synchronize()
    for _ in range(args.steps):
        run_step(work, timer)
    torch.cuda.synchronize()
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

    b2b = {} if args.no_back_to_back else per_shape_graph_us(qg, torch, work)
    for key, us in b2b.items():
        rec = per_shape[key]
        rec["us_per_call_back_to_back"] = round(us, 3)
        rec["GBps_back_to_back"] = round(rec["algorithmic_bytes"] / (us * 1e-6) / 1e9, 1)

    probe = None if args.no_probe else round(hbm_probe(qg, torch), 1)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "launch": "hip graph of the K steps" if graph_used else "eager",
        "eager_ms_per_step": round(eager_wall / args.steps * 1e3, 4),
        "eager_value": round(step_bytes * args.steps / eager_wall / 1e9, 1),
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
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": measured_traffic(),
                     "algorithmic_bytes": step_bytes,
                     "kernel": "qg::gemv_kernel (Q4_0, M=1)",
                     "note": "per step of six launches: achieved = algorithmic bytes / sum of their kernel "
                             "times (HIP events recorded by each launch); traffic = HBM bytes of the six launches "
                             "from rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated on copies of known size"},
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
