"""Turn rocprofv3 CSV output of bench.py runs into the short summaries kept
under profiles/.

    python rocprof_summary.py stats <kernel_stats.csv> <kernel_trace.csv> <out.md> <command>
    python rocprof_summary.py traffic <fetch_counter_collection.csv>
           <write_counter_collection.csv> <out.json> <command-fetch> <command-write>
    python rocprof_summary.py suite <kernel_stats.csv> <suite.jsonl> <out.md> <command>

Traffic calibration: the bench's own weight-copy kernels (__amd_rocclr_copyBuffer
of known sizes, dispatched while it builds its workload) give the factor each
counter reads per real byte; kernel counters are divided by it.
"""
from __future__ import annotations

import csv
import hashlib
import json
import os
import statistics
import sys

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quantized_weight_gemv_amd")
# the files that determine the GEMV kernel and its launch shapes
GEMV_SOURCES = ["csrc/qgemv_gemv_impl.h", "csrc/qgemv_gemv_q4_0.hip", "csrc/qgemv_gemv.hip", "csrc/qgemv_capi.hip",
                "csrc/qgemv_internal.h"]

LLAMA_SHAPES = [(4096, 4096), (6144, 4096), (14336, 4096), (4096, 14336), (28672, 4096), (128256, 4096)]


def gemv_source_hash() -> str:
    h = hashlib.sha256()
    for rel in GEMV_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def algorithmic_bytes(N, K, M=1):
    return N * K // 32 * 18 + 2 * M * K + 4 * M * N


def packed_bytes(N, K):
    nb = N * K // 32
    s0 = (nb * 16 + 255) // 256 * 256
    return (s0 + 2 * nb + 255) // 256 * 256


def _rows(path, counter):
    rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _copy_sizes():
    out = []
    for N, K in LLAMA_SHAPES:
        nb = packed_bytes(N, K)
        out += [nb] * max(2, -(-(1 << 30) // nb))
    return out


def traffic(fetch_csv, write_csv, out_json, cmd_f, cmd_w):
    F = _rows(fetch_csv, "FETCH_SIZE")
    W = _rows(write_csv, "WRITE_SIZE")
    sizes = _copy_sizes()
    cf = [r for r in F if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 65536]
    cw = [r for r in W if "copyBuffer" in r["Kernel_Name"] and int(r["Grid_Size"]) >= 65536]
    assert len(cf) == len(sizes) == len(cw), (len(cf), len(cw), len(sizes))
    ff = statistics.median(float(r["Counter_Value"]) * 1024 / nb for r, nb in zip(cf, sizes))
    fw = statistics.median(float(r["Counter_Value"]) * 1024 / nb for r, nb in zip(cw, sizes))
    gf = [r for r in F if "gemv_kernel" in r["Kernel_Name"]]
    gw = [r for r in W if "gemv_kernel" in r["Kernel_Name"]]
    # bench.py --no-back-to-back: every GEMV dispatch belongs to an interleaved
    # step of the six shapes
    assert len(gf) == len(gw) and len(gf) % len(LLAMA_SHAPES) == 0
    per = {}
    for i, (N, K) in enumerate(LLAMA_SHAPES):
        fv = [float(r["Counter_Value"]) * 1024 / ff for r in gf[i::len(LLAMA_SHAPES)]]
        wv = [float(r["Counter_Value"]) * 1024 / fw for r in gw[i::len(LLAMA_SHAPES)]]
        t = statistics.median(fv) + statistics.median(wv)
        per[f"{N}x{K}"] = {"fetch_bytes": round(statistics.median(fv)), "write_bytes": round(statistics.median(wv)),
                           "traffic_bytes": round(t), "algorithmic_bytes": algorithmic_bytes(N, K),
                           "traffic_over_algorithmic": round(t / algorithmic_bytes(N, K), 4),
                           "kernel": gf[i]["Kernel_Name"]}
    total = sum(v["traffic_bytes"] for v in per.values())
    out = {"what": "HBM traffic of qgemv_q4_0 (M=1) per launch on the Llama-3-8B shapes, from rocprofv3 "
                   "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) divided by the factor each counter reads for a "
                   "plain copy of known size",
           "gemv_source_sha256": gemv_source_hash(),
           "fetch_factor": round(ff, 5), "write_factor": round(fw, 5),
           "traffic_bytes_per_step": total,
           "algorithmic_bytes_per_step": sum(algorithmic_bytes(N, K) for N, K in LLAMA_SHAPES),
           "per_shape": per, "commands": [cmd_f, cmd_w]}
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def stats(stats_csv, trace_csv, out_md, cmd):
    rows = list(csv.DictReader(open(stats_csv)))
    trace = list(csv.DictReader(open(trace_csv)))
    g = sorted([r for r in trace if "gemv_kernel" in r["Kernel_Name"]], key=lambda r: int(r["Start_Timestamp"]))
    lines = [f"# rocprofv3 kernel statistics: {os.path.basename(out_md)[:-3]}", "", "Command:", "", "```", cmd, "```",
             "", "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} |")
    # bench.py --no-back-to-back launches the six shapes in step order
    assert len(g) % len(LLAMA_SHAPES) == 0, len(g)
    lines += ["", "GEMV dispatches per shape (every step launches the six shapes in this order): average / median "
                  "duration", "", "| shape N x K | kernel | grid threads | calls | average us | median us |",
              "|---|---|---|---|---|---|"]
    for i, (N, K) in enumerate(LLAMA_SHAPES):
        rs = g[i::len(LLAMA_SHAPES)]
        v = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs]
        lines.append(f"| {N}x{K} | `{rs[0]['Kernel_Name'][:60]}` | {rs[0]['Grid_Size_X']} | {len(v)} | "
                     f"{statistics.mean(v) / 1e3:.3f} | {statistics.median(v) / 1e3:.3f} |")
    gaps = [int(b["Start_Timestamp"]) - int(a["End_Timestamp"]) for a, b in zip(g, g[1:])]
    if gaps:
        lines += ["", f"Gap between consecutive GEMV dispatches: median {statistics.median(gaps) / 1e3:.2f} us "
                      f"(host launch path included)."]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def suite(stats_csv, suite_jsonl, out_md, cmd, plain_cmd=""):
    """Kernel statistics of a rocprofv3 run of `bench.py --suite` plus the
    per-workload medians of a plain (unprofiled) suite run."""
    rows = list(csv.DictReader(open(stats_csv)))
    recs = [json.loads(l) for l in open(suite_jsonl) if l.strip()]
    lines = ["# rocprofv3 kernel statistics: every workload of bench.py --suite", "",
             "GEMV Q4_0 2048x2048; small-batch GEMV Q4_0/Q8_0 at 1, 2, 4, 8 tokens on 6144x2048, 2048x6144, "
             "8192x2048;", "one-launch MoE (10 of 128 experts 640x2560, 8 of 256 experts 512x2048); Q4_0 prefill "
             "at 64 and 512 tokens", "on 12288x2560, 2560x6144, 6144x2048 with the dense fp16 GEMM on "
             "pre-dequantized weights beside it (the faster of the weight layouts [N][K] and [K][N]); "
             "fp32-activation GEMV and stacked gate+up+SwiGLU with",
             "their unfused steps beside them; the GEMV on 8-bit activations beside the fp16-activation one;",
             "plain 2-bit weights (q2w) beside Q4_0, with 8-bit activations and through lookup tables.", "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{r['Name'][:80]}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | "
                     f"{r['MaxNs']} |")
    lines += ["", "Per-workload medians of a separate, unprofiled `bench.py --suite` run (median us: HIP events "
                  "of each launch; graph: per call in a captured graph of 20 calls; prefill: graph, whole call "
                  "incl. the zero fill of split-K launches):", ""] + (["```", plain_cmd, "```", ""] if plain_cmd else []) + [
              "| workload | median us | GB/s or TFLOP/s |", "|---|---|---|"]
    for r in recs:
        if r["kind"] == "gemv":
            lines.append(f"| GEMV {r['fmt']} {r['N']}x{r['K']} M={r['M']} | {r['us_median']} | {r['GBps']} GB/s |")
        elif r["kind"] == "q2w":
            i8 = r.get("int8_activations_us_median")
            i8s = f"; 8-bit activations {i8}" if i8 is not None else ""
            lt = r.get("lookup_table_us_median")
            lts = f"; lookup tables {lt}" if lt is not None else ""
            lines.append(f"| GEMV q2w (2-bit) {r['N']}x{r['K']} M={r['M']} | {r['us_median']} "
                         f"(Q4_0 {r['q4_0_us_median']}{i8s}{lts}) | {r['GBps']} GB/s |")
        elif r["kind"] == "q8act":
            lines.append(f"| GEMV {r['fmt']} 8-bit activations {r['N']}x{r['K']} M={r['M']} | {r['us_median']} "
                         f"(fp16 activations {r['fp16_activations_us_median']}) | {r['GBps']} GB/s |")
        elif r["kind"] == "f32in":
            lines.append(f"| GEMV {r['fmt']} fp32 activations in {r['N']}x{r['K']} M={r['M']} | {r['us_median']} "
                         f"(graph per call {r['graph_us_median']}; with a separate conversion "
                         f"{r['separate_conversion_graph_us_median']}; fp16 activations "
                         f"{r.get('fp16_input_graph_us_median')}) | {r['GBps']} GB/s |")
        elif r["kind"] == "swiglu":
            lines.append(f"| gate+up+SwiGLU {r['fmt']} fp32 in, 2x{r['N']}x{r['K']} M={r['M']} | {r['us_median']} "
                         f"(graph per call {r['graph_us_median']}; unfused {r['unfused_graph_us_median']}; "
                         f"plain GEMV of the 2N-row table: fp16 in {r.get('stacked_fp16_gemv_graph_us_median')}, "
                         f"fp32 in {r.get('stacked_f32in_gemv_graph_us_median')}) | {r['GBps']} GB/s |")
        elif r["kind"] == "moe":
            lines.append(f"| MoE {r['fmt']} {r['E']} of {r['P']} x {r['N']}x{r['K']} | {r['us_median']} | "
                         f"{r['GBps']} GB/s |")
        else:
            lay = (f": [N][K] {r['dense_nk_us_median']}, [K][N] {r['dense_kn_us_median']}"
                   if "dense_nk_us_median" in r else "")
            lines.append(f"| prefill {r['fmt']} {r['N']}x{r['K']} M={r['M']} | {r['us_median']} (dense fp16 "
                         f"{r['dense_fp16_us_median']}{lay}) | {r['TFLOPs']} TFLOP/s |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def counters(title, out_md, stats_csv, stats_cmd, *pairs):
    """Median of each rocprofv3 --pmc counter per kernel (per dispatch), next
    to the kernel-trace statistics of the same program.  `pairs`: counter
    CSV, command, counter CSV, command, ..."""
    per = {}
    cmds = [stats_cmd]
    for csv_path, cmd in zip(pairs[0::2], pairs[1::2]):
        cmds.append(cmd)
        for r in csv.DictReader(open(csv_path)):
            if "copyBuffer" in r["Kernel_Name"] or "fillBuffer" in r["Kernel_Name"]:
                continue
            per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = [f"# rocprofv3 counters: {title}", "", "Commands (counter passes each in a run of their own):", "", "```"]
    lines += cmds + ["```", "", "| kernel | calls | average ns |", "|---|---|---|"]
    for r in csv.DictReader(open(stats_csv)):
        if "copyBuffer" not in r["Name"]:
            lines.append(f"| `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']):.0f} |")
    per = {k: d for k, d in per.items() if max(len(v) for v in d.values()) >= 5}   # the timed kernels only
    names = sorted({c for d in per.values() for c in d})
    lines += ["", "Median per dispatch:", "", "| counter | " + " | ".join(f"`{k[:60]}`" for k in per) + " |",
              "|---|" + "---|" * len(per)]
    for c in names:
        vals = []
        for d in per.values():
            v = sorted(d.get(c, []))
            vals.append(f"{v[len(v) // 2]:.4g}" if v else "")
        lines.append(f"| {c} | " + " | ".join(vals) + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def probe(bench_json, out_md, cmd):
    """The read probe's per-size floors beside the GEMV on the same byte
    counts, from one bench.py JSON line."""
    d = json.loads([l for l in open(bench_json) if l.strip().startswith("{")][-1])
    p = d["hbm_probe"]
    b = p["best"]
    lines = ["# HBM read probe: per-size floors beside the Q4_0 GEMV (M=1, Llama-3-8B shapes)", "",
             "The probe reads a buffer with the GEMV's load path (non-temporal 16-byte buffer loads, several in "
             "flight per lane, whole 4 KiB tiles per workgroup round robin) and computes nothing; per size the "
             "fastest of the swept launch shapes (loads in flight x workgroups) is the floor a one-launch read of "
             "that many bytes reaches on this chip. Both sides cycle copies of >= 1 GiB so every launch reads HBM.",
             "", "Command:", "", "```", cmd, "```", "",
             f"Best streaming read: {b['GBps']} GB/s ({b['bytes']} bytes, {b['loads_in_flight']} loads in flight, "
             f"{b['workgroups']} workgroups, {b['us']} us).", "",
             "| shape N x K | bytes | probe us (events) | probe us (back to back) | probe launch | GEMV us (events) "
             "| GEMV us (back to back) | GEMV / probe (back to back) |", "|---|---|---|---|---|---|---|---|"]
    for shape, f in p["per_shape_floor"].items():
        g = d["per_shape"][shape]
        lines.append(f"| {shape} | {f['bytes']} | {f['us_median']} | {f['us_back_to_back']} | "
                     f"{f['loads_in_flight']} loads x {f['workgroups']} WGs | {g['us_median']} | "
                     f"{g['us_per_call_back_to_back']} | {g['us_per_call_back_to_back'] / f['us_back_to_back']:.3f} |")
    env = d.get("env", {})
    if env:
        lines += ["", "Environment: " + json.dumps({k: env[k] for k in env if k != "inputs_sha256"})[:1500]]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(*sys.argv[2:6])
    elif sys.argv[1] == "traffic":
        traffic(*sys.argv[2:7])
    elif sys.argv[1] == "suite":
        suite(*sys.argv[2:7])
    elif sys.argv[1] == "probe":
        probe(*sys.argv[2:5])
    elif sys.argv[1] == "counters":
        counters(*sys.argv[2:])
    else:
        raise SystemExit(__doc__)
