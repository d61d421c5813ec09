#!/usr/bin/env python3
"""Throughput of the affine group-quantized matvec on one MI355X.

Workload: the Llama-3-8B-shaped batch-1 decode GEMV set at 4 bits, group size
64: qkv 6144x4096, o 4096x4096, gate_up 28672x4096, down 4096x14336 and
lm_head 128256x4096. Inputs are seeded synthetic data (x ~ N(0,1) in bf16;
W ~ N(0, 0.02) quantized per 64-column group). One step is one batch-1
product through each of the five matrices, five kernel launches.

Every step reads its weights from one of ROT distinct copies, at least
512 MiB in total, so the 256 MB Infinity Cache cannot serve repeated reads.
Inputs are resident in HBM before timing starts.

value: algorithmic bytes per step / step time, in GB/s. Algorithmic bytes are
N*K*bits/8 (codes) + 4*N*K/64 (bf16 scale and bias) + 2*K (x) + 2*N (y) per
product. The timed steps are eager: one C call per product, queued from the
host ahead of the GPU. The same steps replayed from captured HIP graphs (one
graph per weight copy, checked bit for bit against the eager outputs) are
reported beside it; on this stack graph nodes add gaps, so eager is faster.

roofline: the kernel with the most time per step. With the launch planner's
choices that is the instantiation that runs lm_head and nothing else. HIP
events around each of its launches over a second timed pass of the same
steps, run eagerly on the same stream, give its average duration. Achieved
GB/s is its algorithmic bytes per launch over that duration, against the
8 TB/s HBM3E peak.

cpu_baseline: the CPU oracle (single thread, float64) on a row sample of the
same five matrices, sized to about --cpu-seconds of work.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
ROTATION_BYTES = 512 * 1024 * 1024
SHAPES = ["qkv", "o", "gate_up", "down", "lm_head"]


def algo_bytes(N, K, bits, M=1):
    return N * K * bits // 8 + 4 * N * K // 64 + 2 * M * K + 2 * M * N


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-shape", action="store_true", help="also time each matrix alone (to stderr)")
    ap.add_argument("--write-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="summarize rocprofv3 CSV output of this benchmark into profiles/ and exit")
    ap.add_argument("--workload", choices=["llama", "wide", "gather"], default="llama",
                    help="llama: the batch-1 decode set (the JSON line); wide: 14336x4096 and 4096x14336 at "
                         "M = 2..8; gather: the Mixtral-shaped expert gather (per-shape lines on stdout)")
    ap.add_argument("--calls", type=int, default=200, help="timed calls per shape (--workload wide/gather)")
    return ap.parse_args()


def cpu_baseline(data, target_s):
    """The oracle on the same five products, ~target_s seconds of single-threaded work.

    It takes an evenly spaced row sample of each matrix when one full pass would
    take longer than target_s, and repeats full passes when a pass is shorter.
    """
    import numpy as np

    import oracle
    x = {"x4096": data["x4096"], "x14336": data["x14336"]}

    def run(frac):
        total_b, t0 = 0, time.perf_counter()
        for name in SHAPES:
            m = data[name]
            n = max(1, int(m["N"] * frac))
            rows = np.linspace(0, m["N"] - 1, n).astype(np.int64)
            oracle.qmv(x[m["x"]], m["w"], m["scales"], m["biases"], m["K"], 4, rows=rows)
            total_b += algo_bytes(n, m["K"], 4)
        return total_b, time.perf_counter() - t0

    _, t0 = run(1 / 512)                      # calibration pass
    frac = min(1.0, (1 / 512) * target_s / max(t0, 1e-3))
    b = t = 0.0
    passes = 0
    while passes == 0 or t < 0.8 * target_s:
        bb, tt = run(frac)
        b, t, passes = b + bb, t + tt, passes + 1
    rows = sum(max(1, int(data[n]["N"] * frac)) for n in SHAPES)
    return {
        "value": round(b / t / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"{passes} pass(es) over {rows} evenly spaced weight rows ({frac:.4f} of each of the 5 "
                  f"matrices), batch 1, {b / 1e6:.1f} MB algorithmic in total, {t:.1f} s single-threaded float64",
        "host_cpus": len(os.sched_getaffinity(0)),
    }


KERNEL_SOURCES = ["affine_group_quantized_amd/csrc/qmv_kernels.hip", "affine_group_quantized_amd/csrc/qmv_device.hpp",
                  "affine_group_quantized_amd/csrc/qmv_kernels.hpp", "affine_group_quantized_amd/csrc/plan.hpp"]
TRAFFIC_MD = os.path.join(ROOT, "profiles", "qmv_lm_head_128256x4096_hbm_traffic.md")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_name):
    """HBM bytes per launch of the dominant kernel from the committed counter summary,
    or None when the summary is missing or the kernel sources changed since."""
    try:
        with open(TRAFFIC_MD) as f:
            for line in f:
                if line.startswith("traffic_json:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("source_hash") == kernel_source_hash() and rec.get("kernel") == kernel_name:
                        return rec["bytes_per_launch"]
    except OSError:
        pass
    return None


def _read_csv(d, suffix):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def write_profiles(trace_dir, fetch_dir, write_dir):
    """Summaries of rocprofv3 runs of this benchmark, as short markdown under profiles/.

    trace_dir: --kernel-trace --stats --output-format csv; fetch_dir / write_dir:
    --pmc FETCH_SIZE / --pmc WRITE_SIZE. The benchmark's weight clones run
    __amd_rocclr_copyBuffer on buffers of known size, which calibrates the counters.
    """
    import statistics
    lm_n, lm_k = 128256, 4096
    lm_w = lm_n * lm_k // 2                      # bytes of lm_head codes, copied by one clone
    stats = _read_csv(trace_dir, "kernel_stats.csv")
    trace = _read_csv(trace_dir, "kernel_trace.csv")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    lines = ["# rocprofv3 kernel statistics: Llama-3-8B-shaped decode GEMV set, batch 1, 4-bit gs64", "",
             "Command (from the repository root):", "",
             "    rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- "
             "python3 bench.py --steps 50 --warmup 5 --no-cpu-baseline", "",
             "| kernel | calls | average us | min us | max us | share of time |", "|---|---|---|---|---|---|"]
    for r in stats:
        name = r["Name"]
        if "agq::" not in name:
            continue
        lines.append(f"| `{name.split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    by_grid = {}
    for r in trace:
        if "agq::qmv_kernel" in r["Kernel_Name"]:
            by_grid.setdefault((r["Kernel_Name"].split("(")[0], r["Grid_Size_X"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "Per launch shape (grid size in threads):", "", "| kernel | grid | launches | median us |",
              "|---|---|---|---|"]
    for (k, g), d in sorted(by_grid.items(), key=lambda kv: -statistics.median(kv[1])):
        lines.append(f"| `{k}` | {g} | {len(d)} | {statistics.median(d):.2f} |")
    with open(os.path.join(ROOT, "profiles", "qmv_llama_decode_set_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines) + "\n")

    def counter(rows, cname):
        out = {}
        for r in rows:
            if r["Counter_Name"] != cname:
                continue
            out.setdefault((r["Kernel_Name"].split("(")[0], int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return out

    fetch = counter(_read_csv(fetch_dir, "counter_collection.csv"), "FETCH_SIZE")
    write = counter(_read_csv(write_dir, "counter_collection.csv"), "WRITE_SIZE")
    # The lm_head codes clone: the copyBuffer dispatch whose WRITE_SIZE is largest.
    cf = max((v for k, v in fetch.items() if "copyBuffer" in k[0]), key=lambda v: max(v))
    cw = max((v for k, v in write.items() if "copyBuffer" in k[0]), key=lambda v: max(v))
    fetch_scale = lm_w / (max(cf) * 1024.0)
    write_scale = lm_w / (max(cw) * 1024.0)
    lm_key = max((k for k in fetch if "qmv_kernel" in k[0]), key=lambda k: statistics.median(fetch[k]))
    f_kib = statistics.median(fetch[lm_key])
    w_kib = statistics.median(write.get(lm_key, [0.0]))
    traffic = f_kib * 1024 * fetch_scale + w_kib * 1024 * write_scale
    algo = lm_n * lm_k // 2 + 4 * lm_n * lm_k // 64 + 2 * lm_k + 2 * lm_n
    kname = lm_key[0].replace("void agq::", "")
    rec = {"kernel": kname, "bytes_per_launch": round(traffic), "fetch_kib": f_kib, "write_kib": w_kib,
           "fetch_scale": round(fetch_scale, 4), "write_scale": round(write_scale, 4),
           "algorithmic_bytes": algo, "source_hash": kernel_source_hash()}
    md = ["# HBM traffic of the lm_head launch (128256x4096, 4-bit gs64, batch 1)", "",
          "Commands (from the repository root), one counter per run:", "",
          "    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o bench -- "
          "python3 bench.py --steps 10 --warmup 2 --no-cpu-baseline",
          "    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o bench -- "
          "python3 bench.py --steps 10 --warmup 2 --no-cpu-baseline", "",
          "Calibration: the benchmark clones the lm_head codes (%d bytes) with `__amd_rocclr_copyBuffer`; "
          "that dispatch reads %.1f KiB FETCH_SIZE and %.1f KiB WRITE_SIZE, so the counters are scaled by "
          "%.4f (fetch) and %.4f (write)." % (lm_w, max(cf), max(cw), fetch_scale, write_scale), "",
          "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | algorithmic bytes | ratio |",
          "|---|---|---|---|---|---|",
          f"| `{kname}` | {f_kib:.1f} | {w_kib:.1f} | {traffic:.0f} | {algo} | {traffic / algo:.4f} |", "",
          "traffic_json: " + json.dumps(rec)]
    with open(TRAFFIC_MD, "w") as f:
        f.write("\n".join(md) + "\n")
    print(json.dumps(rec))


def time_calls(torch, fn, calls, repeats=5, warm_s=0.3):
    """Median over `repeats` of the mean event-timed duration of `calls` back-to-back calls.

    Untimed warm-up: at least 20 calls and `warm_s` seconds of them. The first product
    timed in a process otherwise reads 3-8 us slow, as if the clocks were still ramping."""
    t0 = time.perf_counter()
    i = 0
    while i < 20 or time.perf_counter() - t0 < warm_s:
        fn(i)
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(calls):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / calls)
    return sorted(per)[len(per) // 2]


def other_workload(args):
    """Per-shape timing of the small-batch (workload 2) or gather (workload 4) products.

    Weights rotate over at least 512 MiB of distinct copies, so reads come from HBM.
    One line per shape: us/call, GB/s of algorithmic bytes, % of the HBM peak, and the
    launch plan's engine (0: VALU dot products, 1: matrix cores).
    """
    import numpy as np
    import torch

    import seeded_inputs as si
    import affine_group_quantized_amd as agq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)

    def u32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(dev)

    def report(label, us, nbytes, plan):
        gb = nbytes / (us * 1e-6) / 1e9
        print(json.dumps({"shape": label, "us_per_call": round(us, 3), "GB/s": round(gb, 1),
                          "pct_of_hbm_peak": round(100 * gb / HBM_PEAK_GBPS, 2), "bytes": nbytes,
                          "engine": plan["engine"], "waves_per_group": plan["waves_per_group"],
                          "rows_per_iter": plan["rows_per_iter"], "blocks": plan["blocks"]}), flush=True)

    if args.workload == "wide":
        wl = si.workload(2)
        for name in ("w_a", "w_b"):
            m = wl[name]
            N, K = m["N"], m["K"]
            wbytes = N * K // 2 + 4 * N * K // 64
            rot = max(2, math.ceil(ROTATION_BYTES / wbytes))
            cp = [(u32(m["w"]), bf16(m["scales"]), bf16(m["biases"])) for _ in range(rot)]
            xall = bf16(wl["x4096"] if K == 4096 else wl["x14336"])
            for M in (2, 4, 6, 8):
                x = xall[:M].contiguous()
                y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
                agq.qmv_wide(x, *cp[0], bits=4, out=y)  # validates the operands once
                st = torch.cuda.current_stream().cuda_stream
                ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
                # Raw C calls (pointers prepared above) keep the host ahead of the GPU.
                us = time_calls(torch, lambda i: agq.lib.agq_qmv_wide(x.data_ptr(), *ptrs[i % rot], y.data_ptr(),
                                                                      M, N, K, 4, 64, st), args.calls)
                report(f"{N}x{K} M={M}", us, algo_bytes(N, K, 4, M), agq.launch_plan(M, N, K, 4))
            del cp
            torch.cuda.empty_cache()
    else:
        moe = si.workload(4)
        rhs = moe["rhs"]
        P = len(rhs)
        used = len(set(rhs.tolist()))
        for which in ("w1", "w2"):
            m = moe[which]
            K, N, E = m["K"], m["N"], m["E"]
            x = bf16(moe["x"] if which == "w1" else moe["h"])
            lhs = u32(moe["lhs1"]) if which == "w1" else None
            R = x.shape[0]
            rot = max(2, math.ceil(ROTATION_BYTES / (E * (N * K // 2 + 4 * N * K // 64))))
            cp = [(u32(m["w"]), bf16(m["scales"]), bf16(m["biases"])) for _ in range(rot)]
            ri = u32(rhs)
            y = torch.empty(P, N, dtype=torch.bfloat16, device=dev)
            agq.gather_qmv(x, *cp[0], rhs_indices=ri, lhs_indices=lhs, bits=4, out=y)  # validates once
            st = torch.cuda.current_stream().cuda_stream
            ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
            lp = None if lhs is None else lhs.data_ptr()
            us = time_calls(torch, lambda i: agq.lib.agq_gather_qmv(x.data_ptr(), *ptrs[i % rot], lp, ri.data_ptr(),
                                                                    y.data_ptr(), P, R, E, N, K, 4, 64, st),
                            max(1, args.calls // 4))
            nbytes = used * (N * K // 2 + 4 * N * K // 64) + 2 * R * K + 2 * P * N + 8 * P
            report(f"gather {which} {E}x{N}x{K} P={P} ({used} planes used)", us, nbytes,
                   agq.launch_plan(8, N, K, 4, experts=E))
            del cp
            torch.cuda.empty_cache()


def write_workload_profile(workload, trace_dir, fetch_dir, write_dir):
    """Summary of rocprofv3 runs of `bench.py --workload wide|gather` under profiles/.

    Kernel statistics per instantiation, and the HBM bytes per launch from FETCH_SIZE and
    WRITE_SIZE, scaled by the calibration recorded with the lm_head counters (the same
    counters on the same device; these runs clone no buffers to calibrate with).
    """
    import statistics
    with open(TRAFFIC_MD) as f:
        cal = next(json.loads(line.split(":", 1)[1]) for line in f if line.startswith("traffic_json:"))
    stats = _read_csv(trace_dir, "kernel_stats.csv")
    flags = {"wide": "--workload wide --calls 40", "gather": "--workload gather --calls 40"}[workload]
    pflags = {"wide": "--workload wide --calls 8", "gather": "--workload gather --calls 8"}[workload]
    title = {"wide": "small-batch products 14336x4096 and 4096x14336 at M = 2, 4, 6, 8 (4-bit gs64)",
             "gather": "Mixtral-shaped expert gather, 8 planes of 14336x4096 (W1) and 4096x14336 (W2), "
                       "32 pairs (4-bit gs64)"}[workload]
    lines = [f"# rocprofv3 kernel statistics: {title}", "", "Commands (from the repository root):", "",
             f"    rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- python3 bench.py {flags}",
             f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o bench -- python3 bench.py {pflags}",
             f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o bench -- python3 bench.py {pflags}", "",
             "Kernels `qmv_mfma_kernel` and `gather_mfma_kernel` run on the matrix cores (template arguments: "
             "16-row tiles per band, LDS copy of x, and for `qmv_mfma_kernel` the activation load form: 4 = one "
             "rotated load for M <= 4, 2 = staged through LDS for M = 5-8); `qmv_kernel` is the VALU form.", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        if "agq::" in r["Name"]:
            lines.append(f"| `{r['Name'].split('(')[0]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")

    def counter(d, cname):
        out = {}
        for r in _read_csv(d, "counter_collection.csv"):
            if r["Counter_Name"] == cname and "agq::" in r["Kernel_Name"]:
                out.setdefault((r["Kernel_Name"].split("(")[0], int(r["Grid_Size"])), []).append(
                    float(r["Counter_Value"]))
        return out

    fetch, write = counter(fetch_dir, "FETCH_SIZE"), counter(write_dir, "WRITE_SIZE")
    lines += ["", "HBM bytes per launch (FETCH_SIZE x %.4f + WRITE_SIZE x %.4f, KiB scaled to bytes; the "
              "factors come from the lm_head counter calibration):" % (cal["fetch_scale"], cal["write_scale"]), "",
              "| kernel | grid (threads) | launches | HBM MB per launch |", "|---|---|---|---|"]
    for k in sorted(fetch, key=lambda k: (k[0], k[1])):
        f_kib = statistics.median(fetch[k])
        w_kib = statistics.median(write.get(k, [0.0]))
        mb = (f_kib * cal["fetch_scale"] + w_kib * cal["write_scale"]) * 1024 / 1e6
        lines.append(f"| `{k[0].replace('void agq::', '')}` | {k[1]} | {len(fetch[k])} | {mb:.2f} |")
    out = os.path.join(ROOT, "profiles", f"qmv_{workload}_kernel_stats_and_traffic.md")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def main():
    args = parse()
    if args.write_profiles and args.workload != "llama":
        write_workload_profile(args.workload, *args.write_profiles)
        return
    if args.workload != "llama":
        other_workload(args)
        return
    if args.write_profiles:
        write_profiles(*args.write_profiles)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import seeded_inputs as si
    import affine_group_quantized_amd as agq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    data = si.workload(1)
    print(f"[bench] generated workload in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)

    def u32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(dev)

    step_bytes = sum(algo_bytes(data[n]["N"], data[n]["K"], 4) for n in SHAPES)
    rot = max(2, math.ceil(ROTATION_BYTES / step_bytes))
    xs = {"x4096": bf16(data["x4096"])[0], "x14336": bf16(data["x14336"])[0]}
    mats = {}
    for name in SHAPES:
        m = data[name]
        w0, s0, b0 = u32(m["w"]), bf16(m["scales"]), bf16(m["biases"])
        copies = [(w0, s0, b0)] + [(w0.clone(), s0.clone(), b0.clone()) for _ in range(rot - 1)]
        mats[name] = {"copies": copies, "x": xs[m["x"]], "N": m["N"], "K": m["K"],
                      "y": torch.empty(m["N"], dtype=torch.bfloat16, device=dev)}
    torch.cuda.synchronize()

    # Kernel instantiation of each product, as the launch planner picks it on this device.
    plans = {n: agq.launch_plan(1, mats[n]["N"], mats[n]["K"], 4) for n in SHAPES}
    kern = lambda p: (p["cpt"], p["mw"], p["rows_per_iter"], p["stages"],  # noqa: E731
                      p["waves_per_group"] if p["x_lds_bytes"] else 0)
    by_kernel = {}
    for n in SHAPES:
        by_kernel.setdefault(kern(plans[n]), []).append(n)
    dom_key = max(by_kernel, key=lambda k: sum(algo_bytes(mats[n]["N"], mats[n]["K"], 4) for n in by_kernel[k]))
    dom = set(by_kernel[dom_key])
    # Template arguments: bits, chunks per lane, activation rows, rows per iteration, ring
    # stages, K segments of the block's LDS copy of x (0: none).
    dom_name = "qmv_kernel<4, %d, %d, %d, %d, %d>" % dom_key

    stream = torch.cuda.Stream(dev)
    calls = [{name: agq.prepare_qmv(mats[name]["x"], *mats[name]["copies"][r], mats[name]["y"], bits=4,
                                    stream=stream) for name in SHAPES} for r in range(rot)]

    def step(i, events=None):
        c = calls[i % rot]
        for name in SHAPES:
            if events is not None and name in dom:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                c[name]()
                e1.record(stream)
                events.append((name, e0, e1))
            else:
                c[name]()

    def outputs():
        return {n: mats[n]["y"].view(torch.int16).cpu().numpy().copy() for n in SHAPES}

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    torch.cuda.synchronize()
    eager_out = outputs()

    # One graph per weight copy; each replay is one step.
    graphs = []
    for r in range(rot):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step(r)
        graphs.append(g)
    torch.cuda.synchronize()
    for r in range(rot):  # every replay must equal the eager result, bit for bit
        for n in SHAPES:
            mats[n]["y"].zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graphs[r].replay()
        torch.cuda.synchronize()
        got = outputs()
        for n in SHAPES:
            if not np.array_equal(got[n], eager_out[n]):
                raise SystemExit(f"graph replay {r} differs from the eager result on {n}")
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            graphs[i % rot].replay()

    def timed(fn):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            start.record(stream)
            for i in range(args.steps):
                fn(i)
            end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end)

    total_ms = timed(step)
    ms_per_step = total_ms / args.steps
    value_gbps = step_bytes * args.steps / (total_ms * 1e-3) / 1e9
    graph_ms = timed(lambda i: graphs[i % rot].replay())
    graph_gbps = step_bytes * args.steps / (graph_ms * 1e-3) / 1e9

    # Dominant kernel: HIP events around each of its launches over a timed pass of the same steps.
    events = []
    timed(lambda i: step(i, events))
    dom_ms = [e0.elapsed_time(e1) for _, e0, e1 in events]
    dom_bytes = sum(algo_bytes(mats[n]["N"], mats[n]["K"], 4) for n in dom)
    launches_per_step = len(dom)
    avg_launch_s = (sum(dom_ms) / len(dom_ms)) * 1e-3
    achieved = (dom_bytes / launches_per_step) / avg_launch_s / 1e9

    result = {
        "metric": "qmv achieved HBM GB/s (% of MI355X peak) + us/call, 4-bit gs64 decode shapes",
        "value": round(value_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u4 codes, bf16 in/out, fp32 accumulate",
        "data": "synthetic (seeded; x ~ N(0,1) bf16, W ~ N(0,0.02) quantized 4-bit gs64)",
        "config": {"workload": "Llama-3-8B-shaped decode GEMV set, batch 1, 4-bit gs64",
                   "shapes": {n: [mats[n]["N"], mats[n]["K"]] for n in SHAPES},
                   "bytes_per_step": step_bytes, "rotation_copies": rot, "timing": "eager, one C call per product",
                   "pct_of_hbm_peak": round(100 * value_gbps / HBM_PEAK_GBPS, 2),
                   "us_per_call_avg": round(ms_per_step * 1e3 / len(SHAPES), 3),
                   "graph_replay_value": round(graph_gbps, 2),
                   "graph_replay_ms_per_step": round(graph_ms / args.steps, 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(dom_name),
                     "kernel": dom_name, "shapes": sorted(dom), "launches_per_step": launches_per_step,
                     "avg_launch_us": round(avg_launch_s * 1e6, 3)},
    }

    if args.per_shape:
        for name in SHAPES:
            m = mats[name]
            ts = []
            for i in range(max(40, 2 * rot)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                calls[i % rot][name]()
                e1.record(stream)
                ts.append((e0, e1))
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) for a, b in ts])) * 1e3
            gb = algo_bytes(m["N"], m["K"], 4) / (us * 1e-6) / 1e9
            p = plans[name]
            print(f"[bench] {name:8s} {m['N']}x{m['K']}: {us:8.2f} us/call  {gb:8.1f} GB/s  "
                  f"{100 * gb / HBM_PEAK_GBPS:5.1f}% of peak  (cpt={p['cpt']} R={p['rows_per_iter']} "
                  f"groups={p['row_groups']} lds={p['x_lds_bytes']})", file=sys.stderr, flush=True)

    result["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(data, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
