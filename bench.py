#!/usr/bin/env python3
"""Throughput of the affine group-quantized matvec on one MI355X.

Default workload: the Llama-3-8B-shaped batch-1 decode GEMV set at 4 bits, group
size 64: qkv 6144x4096, o 4096x4096, gate_up 28672x4096, down 4096x14336 and
lm_head 128256x4096. Inputs are seeded synthetic data (x ~ N(0,1) in bf16;
W ~ N(0, 0.02) quantized per 64-column group). One step is one batch-1 product
through each of the five matrices: five kernel launches, queued eagerly, one C
call each.

Timing. Inputs are resident in HBM before timing starts. Every step reads its
weights from one of ROT distinct copies, at least 512 MiB in all, so the 256 MB
Infinity Cache cannot serve repeated reads. After the --warmup steps an untimed
warm-up runs for at least --warm-seconds (clocks ramp up over the first
milliseconds of work). Then --repeats windows of --steps steps are timed, each
between two HIP events on the stream the products run on; value is the median
window, and the JSON line also gives the fastest and slowest.

value: algorithmic bytes per step / step time, in GB/s. Algorithmic bytes are
N*K*bits/8 (codes) + 4*N*K/64 (bf16 scale and bias) + 2*M*K (x) + 2*M*N (y) per
product.

Per shape (config.per_shape): each product alone, back to back, rotating over
its own >= 512 MiB of copies, median of --repeats event-timed loops. Beside it,
the read ceiling: the fastest plain streaming read of the same byte count
(libagq_calib.so: non-temporal 16-byte loads, several wave counts, loads in
flight and piece layouts), timed the same way.

roofline: the kernel launch with the most time per step (with the launch
planner's choices, the bit-stream kernel on lm_head's grid: its instantiation
also runs gate_up, on a grid of its own); achieved GB/s is its algorithmic
bytes per launch over its average duration in its back-to-back loop, against
the 8 TB/s HBM3E peak. traffic is the HBM bytes per
launch from the committed rocprofv3 counter summary, or null when the kernel
sources changed since it was taken.

cpu_baseline: the CPU oracle (single thread, float64) on every row of each of
the five matrices, median of 3 calls per shape.

Other workloads (--workload): c0 (4096x4096), wide (14336x4096 and 4096x14336 at
M = 2..8), c3 (0.5B-class 8-bit shapes), gather (Mixtral-shaped expert gather),
qmm (quantized GEMM at M = 16..2048 and the Mixtral-shaped prefill gather, against the
2.5 PFLOP/s bf16 matrix-core peak and HBM), moe (the fused Mixtral-shaped decode MoE
layer against its unfused products), layer (the Llama-shaped decode layer's
projections through agq_qmv_fused: norm + qkv, o + residual, norm + gate/up + SwiGLU,
down + residual, final norm + lm_head, each against the bare product on the same
weights and against the unfused sequence of torch norm / add / SwiGLU around the bare
product), calib (the read ceiling and the empty-kernel launch floor); one JSON line per
shape.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak of MI355X
ROTATION_BYTES = 512 * 1024 * 1024
SHAPES = ["qkv", "o", "gate_up", "down", "lm_head"]
METRIC = "qmv achieved HBM GB/s (% of MI355X peak) + us/call, 4-bit gs64 decode shapes"
CALIB_LIB = os.path.join(ROOT, "affine_group_quantized_amd", "libagq_calib.so")


def algo_bytes(N, K, bits, M=1):
    return N * K * bits // 8 + 4 * N * K // 64 + 2 * M * K + 2 * M * N


def weight_bytes(N, K, bits):
    return N * K * bits // 8 + 4 * N * K // 64


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="steps per timed window")
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before the time-based warm-up")
    ap.add_argument("--warm-seconds", type=float, default=0.3, help="least untimed warm-up after --warmup")
    ap.add_argument("--repeats", type=int, default=7, help="timed windows (value is their median)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calib", action="store_true", help="skip the streaming-read ceiling")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP graph replay figure")
    ap.add_argument("--write-profiles", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 CSV output of this benchmark into profiles/ and exit: "
                         "TRACE_DIR [FETCH_DIR WRITE_DIR]")
    ap.add_argument("--workload", choices=["llama", "c0", "wide", "c3", "gather", "qmm", "moe", "layer", "nvfp4",
                                                  "bits", "calib"],
                    default="llama")
    ap.add_argument("--calls", type=int, default=200, help="calls per timed loop of one shape")
    return ap.parse_args()


# ----------------------------------------------------------------------------- timing


def warm(torch, fn, seconds, least=20):
    """Untimed calls of fn(i): at least `least` and `seconds` of them."""
    t0 = time.perf_counter()
    i = 0
    while i < least or time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def timed_loops(torch, fn, calls, repeats, stream):
    """`repeats` loops of `calls` calls of fn(i), each between two events on `stream`:
    microseconds per call of each loop."""
    per = []
    i0 = 0
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(calls):
            fn(i0 + i)
        e1.record(stream)
        torch.cuda.synchronize()
        i0 += calls
        per.append(e0.elapsed_time(e1) * 1e3 / calls)
    return per


def time_shape(torch, fn, calls, repeats, stream, warm_s=0.1):
    warm(torch, fn, warm_s)
    per = timed_loops(torch, fn, calls, repeats, stream)
    return statistics.median(per), min(per)


# ----------------------------------------------------------------------------- read ceiling


class ReadCeiling:
    """Fastest plain streaming read of a byte count (libagq_calib.so), and the
    empty-kernel launch floor. Each call reads a different region of one large
    buffer, rotating over at least 512 MiB."""

    WAVES = (2048, 4096, 8192, 16384, 32768)
    LOADS = (1, 2, 4)

    def __init__(self, torch, stream, max_bytes):
        import ctypes
        if not os.path.exists(CALIB_LIB):
            raise FileNotFoundError(f"{CALIB_LIB} is not built; run __graft_entry__.build()")
        self.torch, self.stream = torch, stream
        self.lib = ctypes.CDLL(CALIB_LIB)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        self.lib.agqc_read.argtypes = [P, I64, P, I, I, I, P]
        self.lib.agqc_read.restype = I
        self.lib.agqc_empty.argtypes = [I, P]
        self.lib.agqc_empty.restype = I
        region = (max_bytes + 4095) // 4096 * 4096
        self.total = max(ROTATION_BYTES + region, 2 * region)
        self.buf = torch.empty(self.total, dtype=torch.uint8, device="cuda")
        self.buf.random_(0, 256)
        self.sink = torch.zeros(max(self.WAVES) * 64, dtype=torch.int32, device="cuda")
        self.st = ctypes.c_void_p(stream.cuda_stream)
        self.cache = {}

    @staticmethod
    def regions(total, nbytes):
        """(bytes read per call, region stride, regions rotated over) for reads of `nbytes` from a
        buffer of `total` bytes: every region lies inside the buffer (two or more where they fit,
        for rotation); a read larger than the buffer is refused."""
        nbytes = (nbytes + 1023) // 1024 * 1024
        region = (nbytes + 4095) // 4096 * 4096
        fit = total // region
        if fit < 1:
            raise ValueError(f"a read of {nbytes} bytes does not fit the {total}-byte ceiling buffer")
        return nbytes, region, min(fit, max(2, math.ceil(ROTATION_BYTES / region) + 1))

    def _reader(self, nbytes, waves, u, contig):
        nbytes, region, regions = self.regions(self.total, nbytes)
        base = self.buf.data_ptr()
        sink = self.sink.data_ptr()
        read = self.lib.agqc_read

        def fn(i):
            rc = read(base + (i % regions) * region, nbytes, sink, waves, u, contig, self.st)
            if rc:
                raise RuntimeError(f"agqc_read failed ({rc})")
        return fn

    def ceiling(self, nbytes, calls=60, repeats=3):
        """-> (us, config) of the fastest configuration for `nbytes`."""
        if nbytes in self.cache:
            return self.cache[nbytes]
        best = None
        for contig in (0, 1):
            for waves in self.WAVES:
                for u in self.LOADS:
                    if waves * u * 1024 > 4 * nbytes and waves > self.WAVES[0]:
                        continue  # more pieces in flight than the read has
                    fn = self._reader(nbytes, waves, u, contig)
                    warm(self.torch, fn, 0.0, least=8)
                    us = min(timed_loops(self.torch, fn, calls, repeats, self.stream))
                    if best is None or us < best[0]:
                        best = (us, {"waves": waves, "loads_per_stage": u, "layout": "contiguous" if contig else
                                     "interleaved"})
        self.cache[nbytes] = best
        return best

    def empty_us(self, blocks=1024, calls=400, repeats=5):
        st = self.st
        fn = lambda i: self.lib.agqc_empty(blocks, st)  # noqa: E731
        warm(self.torch, fn, 0.05)
        return statistics.median(timed_loops(self.torch, fn, calls, repeats, self.stream))


# ----------------------------------------------------------------------------- CPU baseline


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shapes, xs, bits=4, calls=3):
    """The oracle on every row of each matrix: median of `calls` calls per shape.

    shapes: {name: dict(w, scales, biases, N, K, x)}; xs: {x name: bf16 rows}."""
    import oracle
    oracle.load()
    per, total_b, total_s = {}, 0, 0.0
    for name, m in shapes.items():
        ts = []
        for _ in range(calls):
            t0 = time.perf_counter()
            oracle.qmv(xs[m["x"]], m["w"], m["scales"], m["biases"], m["K"], bits)
            ts.append(time.perf_counter() - t0)
        t = statistics.median(ts)
        b = algo_bytes(m["N"], m["K"], bits)
        per[name] = {"us_per_call": round(t * 1e6, 1), "GB/s": round(b / t / 1e9, 4)}
        total_b += b
        total_s += t
    return {
        "value": round(total_b / total_s / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": f"every row of each of the {len(shapes)} matrices, batch 1, median of {calls} calls per "
                  f"matrix, single-threaded float64; value = total algorithmic bytes / total median time",
        "per_shape": per, "cpu_model": cpu_model(), "host_cpus": len(os.sched_getaffinity(0)),
    }


# ----------------------------------------------------------------------------- profiles


def kernel_label(name):
    """A kernel's demangled name without its argument list, "void " and anonymous-namespace
    qualifiers (template arguments can hold parentheses of their own)."""
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    return name.rsplit("(", 1)[0] if name.endswith(")") else name


KERNEL_SOURCES = ["affine_group_quantized_amd/csrc/qmv_kernels.hip", "affine_group_quantized_amd/csrc/qmv_core.hpp",
                  "affine_group_quantized_amd/csrc/qmv_device.hpp", "affine_group_quantized_amd/csrc/qmv_kernels.hpp",
                  "affine_group_quantized_amd/csrc/plan.hpp", "affine_group_quantized_amd/csrc/agq_api.cpp",
                  "affine_group_quantized_amd/csrc/qmv_stream.hip"]
TRAFFIC_MD = os.path.join(ROOT, "profiles", "qmv_llama_decode_set_hbm_traffic.md")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel_name):
    """HBM bytes per launch of `kernel_name` from the committed counter summary, or None
    when the summary is missing or the kernel sources changed since it was taken."""
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


def _counter(d, cname, pred):
    out = {}
    for r in _read_csv(d, "counter_collection.csv"):
        if r["Counter_Name"] == cname and pred(r["Kernel_Name"]):
            out.setdefault((kernel_label(r["Kernel_Name"]), int(r["Grid_Size"])), []).append(
                float(r["Counter_Value"]))
    return out


WORKLOAD_FLAGS = {"llama": "--steps 20 --repeats 3 --no-cpu-baseline --no-calib --no-graph",
                  "c0": "--workload c0 --calls 100", "wide": "--workload wide --calls 40",
                  "c3": "--workload c3 --calls 100", "gather": "--workload gather --calls 40",
                  "qmm": "--workload qmm --calls 20", "moe": "--workload moe",
                  "layer": "--workload layer --calls 40 --no-calib", "nvfp4": "--workload nvfp4 --calls 40",
                  "bits": "--workload bits --calls 40"}
PMC_FLAGS = {"llama": "--steps 5 --repeats 1 --warmup 2 --warm-seconds 0 --no-cpu-baseline --no-calib --no-graph",
             "c0": "--workload c0 --calls 8", "wide": "--workload wide --calls 8", "c3": "--workload c3 --calls 8",
             "gather": "--workload gather --calls 8", "qmm": "--workload qmm --calls 4", "moe": "--workload moe",
             "layer": "--workload layer --calls 8 --no-calib", "nvfp4": "--workload nvfp4 --calls 8 --no-calib",
             "bits": "--workload bits --calls 8 --no-calib"}
TITLES = {"llama": "Llama-3-8B-shaped decode GEMV set, batch 1, 4-bit gs64",
          "c0": "single product 4096x4096, batch 1, 4-bit gs64",
          "wide": "small-batch products 14336x4096 and 4096x14336 at M = 2, 4, 6, 8 (4-bit gs64)",
          "c3": "0.5B-class decode GEMVs, batch 1, 8-bit gs64 (4864x896, 896x4864, 1152x896, 151936x896)",
          "gather": "Mixtral-shaped expert gather, 8 planes of 14336x4096 (W1) and 4096x14336 (W2), 32 pairs "
                    "(4-bit gs64)",
          "qmm": "quantized GEMM 14336x4096 / 4096x14336 at M = 16..2048 and the Mixtral-shaped prefill gather "
                 "(512 tokens, top-2), 4-bit gs64",
          "moe": "Mixtral-shaped decode MoE layer, 16 tokens top-2 of 8 experts, H 4096, F 14336, fused against "
                 "unfused (4-bit gs64)",
          "layer": "Llama-shaped decode layer projections through the fused batch-1 kernel (norm + qkv, "
                   "o + residual, norm + gate/up + SwiGLU, down + residual, final norm + lm_head), against the "
                   "bare products and the unfused sequence (4-bit gs64)",
          "nvfp4": "Llama-3-8B-shaped decode GEMV set, batch 1 and 4, and GEMMs at M = 16, 256, 2048, NVFP4 weights "
                   "(E2M1 codes, E4M3 scale per 16 columns), against the affine 4-bit gs64 products on the same shapes",
          "bits": "Llama-3-8B-shaped decode GEMV set, batch 1 and 4, the Mixtral-shaped decode gather W1 and qmm "
                  "(prefill) on 4096x4096, at 2, 3, 5 and 6 bits (the bit-stream widths, gs64) and 4 bits for "
                  "reference"}


def write_profiles(workload, dirs):
    """Summaries of rocprofv3 runs of this benchmark, as short markdown under profiles/.

    dirs[0]: --kernel-trace --stats --output-format csv; dirs[1] / dirs[2] (optional):
    --pmc FETCH_SIZE / --pmc WRITE_SIZE. The llama run clones its weights with
    __amd_rocclr_copyBuffer, dispatches of known size that calibrate the counters; the
    other workloads reuse the factors recorded with the llama counters."""
    name = {"llama": "qmv_llama_decode_set", "c0": "qmv_c0_4096x4096", "wide": "qmv_wide", "c3": "qmv_c3_8bit",
            "gather": "qmv_gather", "qmm": "qmm_prefill", "moe": "moe_decode_layer",
            "layer": "qmv_fused_decode_layer", "nvfp4": "qmv_nvfp4_llama_decode_set",
            "bits": "qmv_bitstream_widths_llama_decode_set"}[workload]
    stats = _read_csv(dirs[0], "kernel_stats.csv")
    trace = _read_csv(dirs[0], "kernel_trace.csv")
    cmd = f"rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o bench -- python3 bench.py " \
          f"{WORKLOAD_FLAGS[workload]}"
    lines = [f"# rocprofv3 kernel statistics: {TITLES[workload]}", "", "Command (from the repository root):", "",
             f"    {cmd}", "",
             "Template arguments: `qmv_kernel<bits, chunks per lane, activation rows, rows per iteration, ring "
             "stages, LDS-copy segments>` and `gather_qmv_kernel<bits, chunks per lane, rows per iteration, ring "
             "stages, LDS-copy segments>` (VALU); `qmv_fused_kernel<bits, chunks per lane, rows per iteration, "
             "ring stages, LDS-copy segments, epilogue (0 residual, 1 SwiGLU, 2 GeGLU, 3 none), norm>` (VALU); "
             "`qmv_mfma_kernel<tiles per band, activation load form (4: compact, 2: staged, 1: four loads)>` and "
             "`gather_mfma_kernel<tiles>` (matrix cores); `qmm_kernel` / `gather_qmm_kernel<bits, tile rows / 32, "
             "tile columns / 32, ...>` and the MoE kernels (matrix cores); and `qmv_stream_kernel<bits, activation rows, expert gather>` (the bit-stream kernel: 2-6 bits, and large batch-1 4-bit products).", "",
             "| kernel | calls | average us | min us | max us | share of time |", "|---|---|---|---|---|---|"]
    for r in stats:
        if "agq::" in r["Name"]:
            lines.append(f"| `{kernel_label(r['Name'])}` | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    by_grid = {}
    for r in trace:
        if "agq::" in r["Kernel_Name"]:
            by_grid.setdefault((kernel_label(r["Kernel_Name"]), int(r["Grid_Size_X"])),
                               []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "Per launch shape (grid size in threads; grids are sized by occupancy, not by N, so one kernel "
              "and grid can serve several shapes of a workload, and then its row pools their launches):", "",
              "| kernel | grid | launches | median us | mean us |", "|---|---|---|---|---|"]
    for (k, g), d in sorted(by_grid.items(), key=lambda kv: -statistics.median(kv[1])):
        lines.append(f"| `{k}` | {g} | {len(d)} | {statistics.median(d):.2f} | {statistics.mean(d):.2f} |")
    if len(dirs) >= 3:
        pred = lambda k: "agq::" in k or "copyBuffer" in k  # noqa: E731
        fetch, write = _counter(dirs[1], "FETCH_SIZE", pred), _counter(dirs[2], "WRITE_SIZE", pred)
        if workload == "llama":
            lm_w = 128256 * 4096 // 2  # the lm_head codes clone, the largest copyBuffer dispatch
            cf = max((v for k, v in fetch.items() if "copyBuffer" in k[0]), key=max)
            cw = max((v for k, v in write.items() if "copyBuffer" in k[0]), key=max)
            fs, ws = lm_w / (max(cf) * 1024.0), lm_w / (max(cw) * 1024.0)
            cal = (f"Calibration: the benchmark clones the lm_head codes ({lm_w} bytes) with "
                   f"`__amd_rocclr_copyBuffer`; that dispatch reads {max(cf):.1f} KiB FETCH_SIZE and "
                   f"{max(cw):.1f} KiB WRITE_SIZE, so the counters are scaled by {fs:.4f} (fetch) and "
                   f"{ws:.4f} (write).")
        else:
            with open(TRAFFIC_MD) as f:
                rec0 = next(json.loads(line.split(":", 1)[1]) for line in f if line.startswith("traffic_json:"))
            fs, ws = rec0["fetch_scale"], rec0["write_scale"]
            cal = (f"Counters scaled by {fs:.4f} (fetch) and {ws:.4f} (write), the factors recorded with the "
                   f"Llama-set counters (same counters, same device; these runs clone no buffer of known size).")
        pflags = PMC_FLAGS[workload]
        lines += ["", "HBM traffic per launch. Commands, one counter per run:", "",
                  f"    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <dir> -o bench -- python3 bench.py {pflags}",
                  f"    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <dir> -o bench -- python3 bench.py {pflags}",
                  "", cal, "",
                  "| kernel | grid (threads) | launches | FETCH KiB | WRITE KiB | HBM MB per launch |",
                  "|---|---|---|---|---|---|"]
        recs = []
        for k in sorted(fetch, key=lambda k: (k[0], k[1])):
            if "copyBuffer" in k[0]:
                continue
            f_kib = statistics.median(fetch[k])
            w_kib = statistics.median(write.get(k, [0.0]))
            traffic = (f_kib * fs + w_kib * ws) * 1024
            lines.append(f"| `{k[0]}` | {k[1]} | {len(fetch[k])} | {f_kib:.1f} | {w_kib:.1f} | {traffic / 1e6:.3f} |")
            recs.append((k, traffic, f_kib, w_kib))
        if workload == "llama":
            # The dominant kernel: the lm_head launch (the largest traffic per launch).
            k, traffic, f_kib, w_kib = max(recs, key=lambda r: r[1])
            algo = algo_bytes(128256, 4096, 4)
            rec = {"kernel": k[0].replace("agq::", ""), "grid": k[1], "bytes_per_launch": round(traffic),
                   "fetch_kib": f_kib, "write_kib": w_kib, "fetch_scale": round(fs, 4), "write_scale": round(ws, 4),
                   "algorithmic_bytes": algo, "ratio": round(traffic / algo, 4), "source_hash": kernel_source_hash()}
            lines += ["", f"lm_head launch: {traffic:.0f} HBM bytes against {algo} algorithmic (ratio "
                      f"{traffic / algo:.4f}).", "", "traffic_json: " + json.dumps(rec)]
    out = os.path.join(ROOT, "profiles", f"{name}_kernel_stats{'_and_traffic' if len(dirs) >= 3 else ''}.md")
    if workload == "llama" and len(dirs) >= 3:
        out = TRAFFIC_MD
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


# ----------------------------------------------------------------------------- device data


def device_helpers(torch, dev):
    import numpy as np

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(dev)

    def u32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(dev)
    return bf16, u32


def rotation(u32, bf16, m, nbytes, least=2):
    """Device copies of one weight (codes, scales, biases), at least ROTATION_BYTES in all."""
    rot = max(least, math.ceil(ROTATION_BYTES / nbytes))
    w0, s0, b0 = u32(m["w"]), bf16(m["scales"]), bf16(m["biases"])
    return [(w0, s0, b0)] + [(w0.clone(), s0.clone(), b0.clone()) for _ in range(rot - 1)]


def shape_line(label, us, us_min, nbytes, plan, ceil=None):
    gb = nbytes / (us * 1e-6) / 1e9
    rec = {"shape": label, "us_per_call": round(us, 3), "us_min": round(us_min, 3), "GB/s": round(gb, 1),
           "pct_of_hbm_peak": round(100 * gb / HBM_PEAK_GBPS, 2), "bytes": nbytes}
    if ceil is not None:
        rec["read_ceiling_us"] = round(ceil[0], 3)
        rec["pct_of_read_ceiling"] = round(100 * ceil[0] / us, 1)
    if plan is not None:
        rec.update(engine=plan["engine"], waves_per_group=plan["waves_per_group"],
                   rows_per_iter=plan["rows_per_iter"], blocks=plan["blocks"])
    return rec


# ----------------------------------------------------------------------------- other workloads


def other_workload(args):
    """One JSON line per shape: us/call (median and min of event-timed back-to-back loops over
    >= 512 MiB of weight copies), GB/s of algorithmic bytes, % of HBM peak, % of the read
    ceiling for the same byte count, and the launch plan (engine 0: VALU, 1: matrix cores)."""
    import torch

    import seeded_inputs as si
    import affine_group_quantized_amd as agq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf16, u32 = device_helpers(torch, dev)
    stream = torch.cuda.current_stream(dev)
    st = stream.cuda_stream
    calib = None
    if not args.no_calib and args.workload not in ("calib", "qmm", "moe"):
        # the largest read each workload asks a ceiling for: 6-bit lm_head (427 MB), else 4-bit lm_head (297 MB)
        calib = ReadCeiling(torch, stream, (440 if args.workload == "bits" else 300) * 1024 * 1024)

    def emit(rec):
        print(json.dumps(rec), flush=True)

    if args.workload == "calib":
        calib = ReadCeiling(torch, stream, 300 * 1024 * 1024)
        emit({"empty_kernel_us": round(calib.empty_us(), 3), "blocks": 1024})
        sizes = sorted({algo_bytes(n, k, b) for cfg in (0, 1, 3) for _, _, n, k, b, _ in si.WORKLOADS[cfg]["w"]})
        sizes += [33_177_600, 265_289_856]
        for nb in sorted(set(sizes)):
            us, cfg = calib.ceiling(nb)
            emit({"read_bytes": nb, "us": round(us, 3), "GB/s": round(nb / us / 1e3, 1),
                  "pct_of_hbm_peak": round(100 * nb / us / 1e3 / HBM_PEAK_GBPS, 2), **cfg})
        return

    if args.workload == "qmm":
        qmm_workload(args, torch, si, agq, bf16, u32, stream, st, emit)
        return
    if args.workload == "moe":
        moe_workload(args, torch, si, agq, bf16, u32, stream, emit)
        return
    if args.workload == "layer":
        layer_workload(args, torch, si, agq, bf16, u32, stream, calib, emit)
        return
    if args.workload == "nvfp4":
        nvfp4_workload(args, torch, si, agq, bf16, u32, stream, calib, emit)
        return
    if args.workload == "bits":
        bits_workload(args, torch, si, agq, bf16, u32, stream, calib, emit)
        return

    if args.workload in ("c0", "c3"):
        cfg = 0 if args.workload == "c0" else 3
        wl = si.workload(cfg)
        bits = 4 if cfg == 0 else 8
        for t, name, N, K, _, xname in si.WORKLOADS[cfg]["w"]:
            m = wl[name]
            cp = rotation(u32, bf16, m, weight_bytes(N, K, bits))
            x = bf16(wl[xname])[0]
            y = torch.empty(N, dtype=torch.bfloat16, device=dev)
            agq.qmv(x, *cp[0], bits=bits, out=y)  # validates the operands once
            ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
            rot = len(cp)
            us, us_min = time_shape(torch, lambda i: agq.lib.agq_qmv(x.data_ptr(), *ptrs[i % rot], y.data_ptr(),
                                                                     N, K, bits, 64, st), args.calls, 5, stream)
            nb = algo_bytes(N, K, bits)
            emit(shape_line(f"{name} {N}x{K} {bits}-bit", us, us_min, nb, agq.launch_plan(1, N, K, bits),
                            calib.ceiling(nb) if calib else None))
            del cp
            torch.cuda.empty_cache()
    elif args.workload == "wide":
        wl = si.workload(2)
        for name in ("w_a", "w_b"):
            m = wl[name]
            N, K = m["N"], m["K"]
            cp = rotation(u32, bf16, m, weight_bytes(N, K, 4))
            rot = len(cp)
            xall = bf16(wl[m["x"]])
            for M in (2, 4, 6, 8):
                x = xall[:M].contiguous()
                y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
                agq.qmv_wide(x, *cp[0], bits=4, out=y)
                ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
                us, us_min = time_shape(torch, lambda i: agq.lib.agq_qmv_wide(x.data_ptr(), *ptrs[i % rot],
                                                                              y.data_ptr(), M, N, K, 4, 64, st),
                                        args.calls, 5, stream)
                nb = algo_bytes(N, K, 4, M)
                emit(shape_line(f"{N}x{K} M={M}", us, us_min, nb, agq.launch_plan(M, N, K, 4),
                                calib.ceiling(nb) if calib else None))
            del cp
            torch.cuda.empty_cache()
    else:  # gather
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
            cp = rotation(u32, bf16, m, E * weight_bytes(N, K, 4))
            rot = len(cp)
            ri = u32(rhs)
            y = torch.empty(P, N, dtype=torch.bfloat16, device=dev)
            agq.gather_qmv(x, *cp[0], rhs_indices=ri, lhs_indices=lhs, bits=4, out=y)
            ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
            lp = None if lhs is None else lhs.data_ptr()
            us, us_min = time_shape(torch, lambda i: agq.lib.agq_gather_qmv(x.data_ptr(), *ptrs[i % rot], lp,
                                                                            ri.data_ptr(), y.data_ptr(), P, R, E,
                                                                            N, K, 4, 64, st),
                                    max(1, args.calls // 4), 5, stream)
            nb = used * weight_bytes(N, K, 4) + 2 * R * K + 2 * P * N + 8 * P
            emit(shape_line(f"gather {which} {E}x{N}x{K} P={P} ({used} planes used)", us, us_min, nb,
                            agq.launch_plan(8, N, K, 4, experts=E), calib.ceiling(nb) if calib else None))
            del cp
            torch.cuda.empty_cache()


def qmm_line(label, us, us_min, flops, nbytes, plan=None):
    tf = flops / (us * 1e-6) / 1e12
    gb = nbytes / (us * 1e-6) / 1e9
    bound_us = max(flops / (MFMA_BF16_PEAK_TFLOPS * 1e12), nbytes / (HBM_PEAK_GBPS * 1e9)) * 1e6
    rec = {"shape": label, "us_per_call": round(us, 3), "us_min": round(us_min, 3), "TFLOP/s": round(tf, 1),
           "pct_of_mfma_bf16_peak": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 2), "GB/s": round(gb, 1),
           "pct_of_hbm_peak": round(100 * gb / HBM_PEAK_GBPS, 2), "flops": flops, "bytes": nbytes,
           "bound": "mfma" if flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBPS * 1e9) else "hbm",
           "pct_of_binding_roofline": round(100 * bound_us / us, 2)}
    return rec


def qmm_workload(args, torch, si, agq, bf16, u32, stream, st, emit):
    """Quantized GEMM (prefill): Llama-3-8B-shaped 4-bit matrices at M = 16 .. 2048 activation
    rows, and the Mixtral-shaped expert gather at 512 tokens, top-2 (1024 pairs over the 8 W1
    planes). Algorithmic flops are 2*M*N*K (2*P*N*K for the gather); bytes are the codes,
    scales and biases read once (used planes only), x and y."""
    import numpy as np
    dev = torch.device("cuda:0")
    wl = si.workload(1, only=("o", "gate_up", "down"))
    for name in ("o", "gate_up", "down"):
        m = wl[name]
        N, K = m["N"], m["K"]
        cp = rotation(u32, bf16, m, weight_bytes(N, K, 4))
        rot = len(cp)
        ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
        for M in (16, 64, 256, 512, 2048):
            x = bf16(si.draw_activations(6, M, M, K))
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            agq.qmm(x, *cp[0], bits=4, out=y)
            wsb = agq.lib.agq_qmm_workspace(M, N, K, 4, 64)
            ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
            wsp = ws.data_ptr() if wsb > 0 else None
            calls = max(4, min(args.calls, int(2e6 / (2 * M * N * K / 1e9 + 1))))
            us, us_min = time_shape(torch, lambda i: agq.lib.agq_qmm(x.data_ptr(), *ptrs[i % rot], y.data_ptr(), M,
                                                                     N, K, 4, 64, wsp, wsb, st), calls, 5, stream)
            emit(qmm_line(f"qmm {name} {N}x{K} M={M}", us, us_min, 2 * M * N * K,
                          weight_bytes(N, K, 4) + 2 * M * K + 2 * M * N))
            del x, y, ws
        del cp
        torch.cuda.empty_cache()
    moe = si.workload(4, only=("w1",))
    m = moe["w1"]
    pre = si.moe_prefill(512)
    E, N, K = m["E"], m["N"], m["K"]
    rhs, lhs = pre["rhs"], pre["lhs"]
    P, R = len(rhs), pre["x"].shape[0]
    used = len(set(rhs.tolist()))
    cp = rotation(u32, bf16, m, E * weight_bytes(N, K, 4))
    rot = len(cp)
    ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
    x, ri, li = bf16(pre["x"]), u32(rhs), u32(lhs)
    y = torch.empty(P, N, dtype=torch.bfloat16, device=dev)
    agq.gather_qmm(x, *cp[0], rhs_indices=ri, lhs_indices=li, out=y)
    us, us_min = time_shape(torch, lambda i: agq.lib.agq_gather_qmm(x.data_ptr(), *ptrs[i % rot], li.data_ptr(),
                                                                    ri.data_ptr(), y.data_ptr(), P, R, E, N, K, 4,
                                                                    64, st), 20, 5, stream)
    emit(qmm_line(f"gather_qmm w1 {E}x{N}x{K} P={P} (512 tokens top-2, {used} planes used)", us, us_min,
                  2 * P * N * K, used * weight_bytes(N, K, 4) + 2 * R * K + 2 * P * N + 8 * P))


def moe_workload(args, torch, si, agq, bf16, u32, stream, emit):
    """The Mixtral-shaped decode MoE layer (16 tokens, top-2 of 8 experts, H 4096, F 14336):
    agq_moe_decode (three launches) against the same layer from the unfused products (gate and
    up through agq_gather_qmv, SwiGLU and the weighted sum in torch, down through
    agq_gather_qmv). Weights rotate over >= 512 MiB of copies. Bytes: the used planes of
    the three matrices, x and y, the expert ids and router weights, and the two
    intermediates written and read once each (h: two bf16 rows of F per pair; the fp32
    down-projection row of H per pair)."""
    import numpy as np
    moe = si.workload(4)
    lay = si.moe_layer()
    T, k = moe["ids"].shape
    E, F, H = moe["w1"]["E"], moe["w1"]["N"], moe["w1"]["K"]
    used = len(set(moe["ids"].reshape(-1).tolist()))
    wb = weight_bytes(F, H, 4)
    cp = [[(u32(d["w"]), bf16(d["scales"]), bf16(d["biases"])) for d in (moe["w1"], lay["w3"], moe["w2"])]]
    rot = max(2, math.ceil(ROTATION_BYTES / (3 * E * wb)))
    for _ in range(rot - 1):
        cp.append([tuple(t.clone() for t in trio) for trio in cp[0]])
    x = bf16(moe["x"])
    ids = u32(moe["ids"])
    w = torch.as_tensor(lay["weights"], device="cuda")
    y = torch.empty(T, H, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(agq.moe_decode_workspace(T, k, H, F), dtype=torch.uint8, device="cuda")
    fused = lambda i: agq.moe_decode(x, *cp[i % rot], ids, w, out=y, workspace=ws)  # noqa: E731
    rhs = u32(moe["ids"].reshape(-1))
    lhs = u32(np.repeat(np.arange(T, dtype=np.uint32), k))

    def unfused(i):
        g_, u_, d_ = cp[i % rot]
        g = agq.gather_qmv(x, *g_, rhs_indices=rhs, lhs_indices=lhs).float()
        u = agq.gather_qmv(x, *u_, rhs_indices=rhs, lhs_indices=lhs).float()
        h = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
        o = agq.gather_qmv(h, *d_, rhs_indices=rhs).float()
        return (o.view(T, k, H) * w[:, :, None]).sum(1).to(torch.bfloat16)

    P = T * k
    nbytes = 3 * used * wb + 2 * T * H + 2 * T * H + 8 * P + 2 * (4 * P * F) + 2 * (4 * P * H)
    for label, fn in (("moe_decode fused (3 launches)", fused), ("unfused: 3 gathers + torch SwiGLU/sum", unfused)):
        us, us_min = time_shape(torch, fn, 20, 5, stream)
        gb = nbytes / (us * 1e-6) / 1e9
        emit({"shape": f"{label}: Mixtral-shaped layer, {T} tokens top-{k} of {E}, H {H}, F {F} ({used} experts used)",
              "us_per_call": round(us, 3), "us_min": round(us_min, 3), "us_per_token": round(us / T, 3),
              "GB/s": round(gb, 1), "pct_of_hbm_peak": round(100 * gb / HBM_PEAK_GBPS, 2), "bytes": nbytes})


def layer_workload(args, torch, si, agq, bf16, u32, stream, calib, emit):
    """The fused batch-1 projections of a Llama-shaped decode layer (workload 1's weights, the
    decode_layer norm weights and residual). Per projection: agq_qmv_fused; the bare agq_qmv
    on the same weights (what the fusion must not slow down); and the unfused sequence (torch
    RMS norm in fp32 rounded to bf16, agq_qmv, torch residual add or SwiGLU). Bytes of the
    fused call: weights + x + norm weight (when normed) + residual (when added) + y."""
    wl = si.workload(1)
    dl = si.decode_layer()
    eps = dl["eps"]
    st = stream.cuda_stream
    g_attn, g_mlp, g_final = bf16(dl["gamma_attn"]), bf16(dl["gamma_mlp"]), bf16(dl["gamma_final"])
    h = bf16(dl["h"])
    x14 = bf16(wl["x14336"])[0]
    x4 = bf16(wl["x4096"])[0]
    # (name, activation, norm weight, residual, act)
    steps = [("qkv", h, g_attn, None, 0), ("o", x4, None, h, 0), ("gate_up", h, g_mlp, None, 1),
             ("down", x14, None, h, 0), ("lm_head", h, g_final, None, 0)]
    silu = torch.nn.functional.silu

    def rms(x, g):
        xf = x.float()
        return (xf * torch.rsqrt(xf.pow(2).mean() + eps) * g.float()).to(torch.bfloat16)

    tot = {"fused": 0.0, "bare": 0.0, "unfused": 0.0}
    for name, x, g, r, act in steps:
        m = wl[name]
        N, K = m["N"], m["K"]
        cp = rotation(u32, bf16, m, weight_bytes(N, K, 4))
        rot = len(cp)
        ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
        n_out = N if act == 0 else N // 2
        y = torch.empty(n_out, dtype=torch.bfloat16, device=x.device)
        yb = torch.empty(N, dtype=torch.bfloat16, device=x.device)
        agq.qmv_fused(x, *cp[0], norm_weight=g, eps=eps, residual=r, act=act, out=y)  # validates once
        gp = None if g is None else g.data_ptr()
        rp = None if r is None else r.data_ptr()
        xp, yp, ybp = x.data_ptr(), y.data_ptr(), yb.data_ptr()
        fused = lambda i: agq.lib.agq_qmv_fused(xp, gp, eps, *ptrs[i % rot], rp, act, yp, N, K, 4, 64, st)  # noqa
        bare = lambda i: agq.lib.agq_qmv(xp, *ptrs[i % rot], ybp, N, K, 4, 64, st)  # noqa: E731

        def unfused(i):
            xin = x if g is None else rms(x, g)
            v = agq.qmv(xin, *cp[i % rot])
            if act:
                vv = v.float().view(-1, 2)
                return (silu(vv[:, 0]) * vv[:, 1]).to(torch.bfloat16)
            return v if r is None else (v.float() + r.float()).to(torch.bfloat16)
        nb = weight_bytes(N, K, 4) + 2 * K + (2 * K if g is not None else 0) + (2 * N if r is not None else 0) \
            + 2 * n_out
        ceil = calib.ceiling(nb) if calib else None
        label = f"{name} {N}x{K}" + (" norm" if g is not None else "") + (" +residual" if r is not None else "") \
            + (" SwiGLU" if act else "")
        for kind, fn, calls in (("fused", fused, args.calls), ("bare", bare, args.calls),
                                ("unfused", unfused, max(1, args.calls // 4))):
            us, us_min = time_shape(torch, fn, calls, 5, stream)
            tot[kind] += us
            rec = shape_line(f"{kind}: {label}", us, us_min, nb, agq.launch_plan(1, N, K, 4) if kind == "bare"
                             else None, ceil if kind == "fused" else None)
            emit(rec)
        del cp
        torch.cuda.empty_cache()
    emit({"layer": "Llama-shaped decode layer projections + lm_head, batch 1",
          **{f"{k}_us": round(v, 3) for k, v in tot.items()},
          "fused_over_bare": round(tot["fused"] / tot["bare"], 4),
          "unfused_over_fused": round(tot["unfused"] / tot["fused"], 3)})


def bits_workload(args, torch, si, agq, bf16, u32, stream, calib, emit):
    """Workload 1's five products with 2-, 3-, 5- and 6-bit codes (group size 64, the
    bit-stream widths) and, for reference, 4-bit codes, at M = 1 and 4 (agq_qmv_wide): us/call,
    GB/s of algorithmic bytes and % of the read ceiling per shape, and the set's sum per width.
    Then the Mixtral-shaped decode gather W1 and qmm on 4096x4096 at M = 64 .. 2048 per width.
    The weights are draw_quantized_weight rows (stream cfg 14) drawn for at most 4096 rows and
    repeated down to N: the kernels do the same work for every code value (nothing branches
    on a value), and drawing all 128256 lm_head rows per width would cost the host minutes."""
    import numpy as np
    st = stream.cuda_stream
    dev = stream.device
    tot = {}
    for t, name, N, K, _, xname in si.WORKLOADS[1]["w"]:
        xall = bf16(si.draw_activations(14, 100 + t, 4, K))
        for bits in (2, 3, 4, 5, 6):
            base = si.draw_quantized_weight(14, 10 * t + bits, min(N, 4096), K, bits)
            reps = -(-N // base["w"].shape[0])
            m = {k: np.tile(base[k], (reps, 1))[:N] for k in ("w", "scales", "biases")}
            cp = rotation(u32, bf16, m, weight_bytes(N, K, bits))
            ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
            rot = len(cp)
            for M in (1, 4):
                x = xall[:M].contiguous()
                y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
                agq.qmv_wide(x, *cp[0], bits=bits, out=y)  # validates the operands once
                xp, yp = x.data_ptr(), y.data_ptr()
                us, us_min = time_shape(torch, lambda i: agq.lib.agq_qmv_wide(xp, *ptrs[i % rot], yp, M, N, K, bits,
                                                                              64, st), args.calls, 5, stream)
                nb = algo_bytes(N, K, bits, M)
                emit(shape_line(f"{bits}-bit: {name} {N}x{K} M={M}", us, us_min, nb, None,
                                calib.ceiling(nb) if calib else None))
                tot[(bits, M)] = tot.get((bits, M), 0.0) + us
            del cp, m, base
            torch.cuda.empty_cache()
    emit({"set": "Llama-shaped decode products at each width (group size 64), us per set",
          **{f"bits{b}_m{M}_us": round(v, 3) for (b, M), v in sorted(tot.items())}})
    # The Mixtral-shaped decode gather W1 (8 planes of 14336x4096, 16 tokens top-2: the
    # routing of the gather workload) at each width; planes tiled from 4096 drawn rows.
    m = si.MOE
    E, N, K, T = m["experts"], m["ffn"], m["hidden"], m["tokens"]
    rhs = si.moe_expert_ids(4, 1, T, E, m["top_k"]).reshape(-1).astype(np.uint32)
    lhs = np.repeat(np.arange(T, dtype=np.uint32), m["top_k"])
    P, used = len(rhs), len(set(rhs.tolist()))
    x = bf16(si.draw_activations(4, 0, T, K))
    ri, li = u32(rhs), u32(lhs)
    for bits in (2, 3, 4, 5, 6):
        base = si.draw_quantized_weight(14, 90 + bits, 4096, K, bits)
        reps = -(-E * N // 4096)
        planes = {k: np.tile(base[k], (reps, 1))[:E * N].reshape(E, N, -1) for k in ("w", "scales", "biases")}
        cp = rotation(u32, bf16, planes, E * weight_bytes(N, K, bits))
        ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
        rot = len(cp)
        y = torch.empty(P, N, dtype=torch.bfloat16, device=dev)
        agq.gather_qmv(x, *cp[0], rhs_indices=ri, lhs_indices=li, bits=bits, out=y)
        us, us_min = time_shape(torch, lambda i: agq.lib.agq_gather_qmv(x.data_ptr(), *ptrs[i % rot], li.data_ptr(),
                                                                        ri.data_ptr(), y.data_ptr(), P, T, E, N, K,
                                                                        bits, 64, st),
                                max(1, args.calls // 4), 5, stream)
        nb = used * weight_bytes(N, K, bits) + 2 * T * K + 2 * P * N + 8 * P
        emit(shape_line(f"{bits}-bit: gather w1 {E}x{N}x{K} P={P} ({used} planes used)", us, us_min, nb, None,
                        calib.ceiling(nb) if calib else None))
        del cp, planes, base
        torch.cuda.empty_cache()
    # qmm (prefill) on o 4096x4096 at each width: from 64 rows the stream widths widen their
    # codes to 8 bits in the workspace and run the 8-bit GEMM; at 64 rows also the passes of
    # 8 rows without a workspace. Bytes as the qmm workload (codes, scales, biases, x, y).
    N, K = 4096, 4096
    for bits in (2, 3, 4, 5, 6):
        m = si.draw_quantized_weight(14, 80 + bits, N, K, bits)
        cp = rotation(u32, bf16, m, weight_bytes(N, K, bits))
        rot = len(cp)
        ptrs = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in cp]
        for M, use_ws in ((64, False), (64, True), (256, True), (2048, True)):
            x = bf16(si.draw_activations(6, M, M, K))
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            wsb = agq.lib.agq_qmm_workspace(M, N, K, bits, 64) if use_ws else 0
            ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
            wsp = ws.data_ptr() if wsb > 0 else None
            agq.qmm(x, *cp[0], bits=bits, out=y, workspace=ws if wsb > 0 else False)
            calls = max(4, min(args.calls, int(2e6 / (2 * M * N * K / 1e9 + 1))))
            us, us_min = time_shape(torch, lambda i: agq.lib.agq_qmm(x.data_ptr(), *ptrs[i % rot], y.data_ptr(), M,
                                                                     N, K, bits, 64, wsp, wsb, st), calls, 5, stream)
            route = "" if bits == 4 else (" (widened to 8 bits)" if wsb > 0 else " (passes of 8 rows)")
            emit(qmm_line(f"{bits}-bit: qmm o {N}x{K} M={M}{route}", us, us_min, 2 * M * N * K,
                          weight_bytes(N, K, bits) + 2 * M * K + 2 * M * N))
            del x, y, ws
        del cp, m
        torch.cuda.empty_cache()


def nvfp4_workload(args, torch, si, agq, bf16, u32, stream, calib, emit):
    """Workload 1's five products with NVFP4 weights at M = 1 and 4, each against the affine
    4-bit gs64 product (agq_qmv / agq_qmv_wide) on the same shape and activations, and the
    matrix-core GEMMs (agq_qmm_nvfp4, agq_qmm) at M = 16, 256 and 2048 on all but lm_head. Both
    formats carry N*K/2 code bytes and N*K/16 scale bytes, so the algorithmic bytes match.
    The NVFP4 weights are nvfp4_weight rows (stream cfg 12) drawn for at most 4096 rows and
    repeated down to N: every code word costs the kernel the same fixed-latency converts and
    nothing branches on a value, so the timing does not depend on the values, and drawing
    all 128256 lm_head rows would cost the host about 40 s."""
    import numpy as np
    wl = si.workload(1)
    st = stream.cuda_stream
    dev = stream.device
    tot = {}
    for t, name, N, K, _, xname in si.WORKLOADS[1]["w"]:
        base = si.nvfp4_weight(12, t, min(N, 4096), K)
        reps = -(-N // base["w"].shape[0])
        w_h = np.tile(base["w"], (reps, 1))[:N]
        s_h = np.tile(base["scales"], (reps, 1))[:N]
        ts = base["tensor_scale"]
        nb_w = N * K // 2 + N * K // 16
        rot = max(2, math.ceil(ROTATION_BYTES / nb_w))
        w0 = u32(w_h)
        s0 = torch.from_numpy(np.ascontiguousarray(s_h)).to(dev)
        fp4 = [(w0, s0)] + [(w0.clone(), s0.clone()) for _ in range(rot - 1)]
        fptr = [(a.data_ptr(), b.data_ptr()) for a, b in fp4]
        del w_h, s_h
        m = wl[name]
        aff = rotation(u32, bf16, m, weight_bytes(N, K, 4))
        aptr = [(c[0].data_ptr(), c[1].data_ptr(), c[2].data_ptr()) for c in aff]
        arot = len(aff)
        gemm_ms = (16, 256, 2048) if name != "lm_head" else ()
        xall = bf16(si.draw_activations(12, 100 + t, max(gemm_ms + (4,)), K))
        for M in (1, 4) + gemm_ms:
            x = xall[:M].contiguous()
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            agq.qmm_nvfp4(x, *fp4[0], ts, out=y)  # validates the operands once
            xp, yp = x.data_ptr(), y.data_ptr()
            nb = algo_bytes(N, K, 4, M)
            if M > 4:
                # the GEMM lines: both formats, against the bf16 matrix-core peak
                flops = 2 * M * N * K
                calls = max(2, args.calls // (4 if M >= 2048 else 1))
                wsn = agq.lib.agq_qmm_nvfp4_workspace(M, N, K)
                wsa = agq.lib.agq_qmm_workspace(M, N, K, 4, 64)
                ws = torch.empty(max(wsn, wsa, 16), dtype=torch.uint8, device=dev)
                wsp_n = ws.data_ptr() if wsn > 0 else None
                wsp_a = ws.data_ptr() if wsa > 0 else None
                us, us_min = time_shape(torch, lambda i: agq.lib.agq_qmm_nvfp4(xp, *fptr[i % rot], ts, yp, M, N, K,
                                                                                 wsp_n, wsn, st), calls, 5, stream)
                emit(qmm_line(f"nvfp4 qmm: {name} {N}x{K} M={M}", us, us_min, flops, nb))
                ua, ua_min = time_shape(torch, lambda i: agq.lib.agq_qmm(xp, *aptr[i % arot], yp, M, N, K, 4, 64, wsp_a,
                                                                         wsa, st), calls, 5, stream)
                emit(qmm_line(f"affine qmm: {name} {N}x{K} M={M}", ua, ua_min, flops, nb))
                continue
            ceil = calib.ceiling(nb) if calib else None
            us, us_min = time_shape(torch, lambda i: agq.lib.agq_qmv_nvfp4(xp, *fptr[i % rot], ts, yp, M, N, K, st),
                                    args.calls, 5, stream)
            emit(shape_line(f"nvfp4: {name} {N}x{K} M={M}", us, us_min, nb, None, ceil))
            if M == 1:
                aff_fn = lambda i: agq.lib.agq_qmv(xp, *aptr[i % arot], yp, N, K, 4, 64, st)  # noqa: E731
            else:
                aff_fn = lambda i: agq.lib.agq_qmv_wide(xp, *aptr[i % arot], yp, M, N, K, 4, 64, st)  # noqa
            ua, ua_min = time_shape(torch, aff_fn, args.calls, 5, stream)
            emit(shape_line(f"affine: {name} {N}x{K} M={M}", ua, ua_min, nb, agq.launch_plan(M, N, K, 4), ceil))
            for kind, v in (("nvfp4", us), ("affine", ua)):
                tot[f"{kind}_m{M}_us"] = tot.get(f"{kind}_m{M}_us", 0.0) + v
        del fp4, aff
        torch.cuda.empty_cache()
    emit({"set": "Llama-shaped decode products, NVFP4 against affine 4-bit gs64",
          **{k: round(v, 3) for k, v in tot.items()},
          "nvfp4_over_affine_m1": round(tot["nvfp4_m1_us"] / tot["affine_m1_us"], 4),
          "nvfp4_over_affine_m4": round(tot["nvfp4_m4_us"] / tot["affine_m4_us"], 4)})


# ----------------------------------------------------------------------------- main workload


def main():
    args = parse()
    if args.write_profiles:
        write_profiles(args.workload, args.write_profiles)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    if args.workload != "llama":
        other_workload(args)
        return

    import numpy as np
    import torch

    import seeded_inputs as si
    import affine_group_quantized_amd as agq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    data = si.workload(1)
    print(f"[bench] generated workload in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    bf16, u32 = device_helpers(torch, dev)

    step_bytes = sum(algo_bytes(data[n]["N"], data[n]["K"], 4) for n in SHAPES)
    rot = max(2, math.ceil(ROTATION_BYTES / step_bytes))
    xs = {"x4096": bf16(data["x4096"])[0], "x14336": bf16(data["x14336"])[0]}
    mats = {}
    for name in SHAPES:
        m = data[name]
        mats[name] = {"copies": rotation(u32, bf16, m, weight_bytes(m["N"], m["K"], 4), least=rot), "x": xs[m["x"]],
                      "N": m["N"], "K": m["K"], "y": torch.empty(m["N"], dtype=torch.bfloat16, device=dev)}
    torch.cuda.synchronize()

    # Kernel instantiation of each product, as the launch planner picks it on this device.
    plans = {n: agq.launch_plan(1, mats[n]["N"], mats[n]["K"], 4) for n in SHAPES}
    # (The bit-stream kernel, engine 2, is one instantiation for every shape it runs; its
    # grid tells the shapes apart, as the counter summary's per-launch rows do.)
    kern = lambda p: (("stream", p["blocks"]) if p["engine"] == 2 else  # noqa: E731
                      (p["cpt"], p["mw"], p["rows_per_iter"], p["stages"], p["waves_per_group"] if p["x_lds_bytes"] else 0))
    by_kernel = {}
    for n in SHAPES:
        by_kernel.setdefault(kern(plans[n]), []).append(n)
    dom_key = max(by_kernel, key=lambda k: sum(algo_bytes(mats[n]["N"], mats[n]["K"], 4) for n in by_kernel[k]))
    dom = by_kernel[dom_key]
    # Template arguments: bits, chunks per lane, activation rows, rows per iteration, ring
    # stages, K segments of the block's LDS copy of x (0: none).
    dom_name = ("qmv_stream_kernel<4, 1, false>" if dom_key[0] == "stream" else
                "qmv_kernel<4, %d, %d, %d, %d, %d>" % dom_key)

    stream = torch.cuda.Stream(dev)
    calls = {name: [agq.prepare_qmv(mats[name]["x"], *c, mats[name]["y"], bits=4, stream=stream)
                    for c in mats[name]["copies"]] for name in SHAPES}

    def step(i):
        for name in SHAPES:
            calls[name][i % rot]()

    def outputs():
        return {n: mats[n]["y"].view(torch.int16).cpu().numpy().copy() for n in SHAPES}

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        eager_out = outputs()
        warm_s = warm(torch, step, args.warm_seconds)
        windows = [w * 1e-3 for w in timed_loops(torch, step, args.steps, args.repeats, stream)]  # ms per step
    ms_per_step = statistics.median(windows)
    value_gbps = step_bytes / (ms_per_step * 1e-3) / 1e9

    graph = None
    if not args.no_graph:
        # One graph per weight copy; each replay is one step, checked bit for bit against eager.
        graphs = []
        for r in range(rot):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(r)
            graphs.append(g)
        torch.cuda.synchronize()
        for r in range(rot):
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
            replay = lambda i: graphs[i % rot].replay()  # noqa: E731
            warm(torch, replay, 0.1)
            gwin = [w * 1e-3 for w in timed_loops(torch, replay, args.steps, args.repeats, stream)]
        graph = statistics.median(gwin)

    # Each product alone, back to back over its own rotation set.
    calib = None
    if not args.no_calib:
        try:
            calib = ReadCeiling(torch, stream, max(algo_bytes(m["N"], m["K"], 4) for m in mats.values()))
        except FileNotFoundError as e:
            print(f"[bench] {e}", file=sys.stderr)
    per_shape = {}
    with torch.cuda.stream(stream):
        for name in SHAPES:
            cs = calls[name]
            n = len(cs)
            us, us_min = time_shape(torch, lambda i: cs[i % n](), max(args.calls, 2 * n), args.repeats, stream)
            nb = algo_bytes(mats[name]["N"], mats[name]["K"], 4)
            rec = shape_line(f"{mats[name]['N']}x{mats[name]['K']}", us, us_min, nb, plans[name],
                             calib.ceiling(nb) if calib else None)
            rec["rotation_copies"] = n
            per_shape[name] = rec
            print(f"[bench] {name:8s} {json.dumps(rec)}", file=sys.stderr, flush=True)

    # Host cost of one call (checks, plan, launch; the prepared one-C-call closure from Python),
    # timed on the host over back-to-back steps while the GPU drains the queue behind it.
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        n_host = 100
        t0 = time.perf_counter()
        for i in range(n_host):
            step(i)
        host_s = time.perf_counter() - t0
        torch.cuda.synchronize()

    dom_us = sum(per_shape[n]["us_per_call"] for n in dom) / len(dom)
    dom_bytes = sum(algo_bytes(mats[n]["N"], mats[n]["K"], 4) for n in dom) / len(dom)
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9

    config = {"workload": "Llama-3-8B-shaped decode GEMV set, batch 1, 4-bit gs64",
              "shapes": {n: [mats[n]["N"], mats[n]["K"]] for n in SHAPES},
              "bytes_per_step": step_bytes, "rotation_copies": rot,
              "timing": f"eager, one C call per product; median of {args.repeats} event-timed windows of "
                        f"{args.steps} steps",
              "warmup_steps": args.warmup, "warmup_s": round(warm_s, 3),
              "ms_per_step_min": round(min(windows), 5), "ms_per_step_max": round(max(windows), 5),
              "pct_of_hbm_peak": round(100 * value_gbps / HBM_PEAK_GBPS, 2),
              "value_best_window": round(step_bytes / (min(windows) * 1e-3) / 1e9, 2),
              "per_shape": per_shape,
              "host_us_per_call": round(host_s / (n_host * len(SHAPES)) * 1e6, 3)}
    if graph is not None:
        config["graph_replay_value"] = round(step_bytes / (graph * 1e-3) / 1e9, 2)
        config["graph_replay_ms_per_step"] = round(graph, 5)
    if calib is not None:
        ceil_us = sum(per_shape[n]["read_ceiling_us"] for n in SHAPES)
        config["read_ceiling_us_per_step"] = round(ceil_us, 3)
        config["pct_of_read_ceiling"] = round(100 * ceil_us / (ms_per_step * 1e3), 1)
        config["empty_kernel_us"] = round(calib.empty_us(), 3)

    result = {
        "metric": METRIC, "value": round(value_gbps, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "u4 codes, bf16 in/out, fp32 accumulate",
        "data": "synthetic (seeded; x ~ N(0,1) bf16, W ~ N(0,0.02) quantized 4-bit gs64)",
        "config": config,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": stored_traffic(dom_name),
                     "kernel": dom_name, "shapes": sorted(dom), "avg_launch_us": round(dom_us, 3),
                     "timing": "median of event-timed back-to-back loops of the kernel's products"},
    }
    result["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(
        {n: data[n] for n in SHAPES}, {"x4096": data["x4096"], "x14336": data["x14336"]})
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
