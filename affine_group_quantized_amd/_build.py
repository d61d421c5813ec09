"""Builds ``libagq.so`` (HIP kernels + C ABI) and ``libagq_calib.so`` (the benchmark's
streaming-read calibration kernel) in-tree for gfx950 with hipcc.

Each source compiles to its own object in parallel; the objects are then linked.
"""
from __future__ import annotations

import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libagq.so")
CALIB_LIB = os.path.join(PKG, "libagq_calib.so")

SOURCES = ["qmv_kernels.hip", "qmv_fused.hip", "qmv_nvfp4.hip", "qmv_stream.hip", "qmv_mfma.hip", "qmm_mfma.hip", "moe_mfma.hip",
           "quant.hip", "agq_api.cpp"]
CALIB_SOURCES = ["calib_read.hip"]

# Packed-FP32 instructions are disabled for all device code.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _link(sources, out, verbose, tmpdir):
    hipcc = _hipcc()
    objs = [os.path.join(tmpdir, os.path.basename(s) + ".o") for s in sources]

    def compile_one(i):
        cmd = [hipcc, *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", os.path.join(CSRC, sources[i]),
               "-o", objs[i]]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)

    with ThreadPoolExecutor(max_workers=min(len(sources), os.cpu_count() or 1)) as ex:
        list(ex.map(compile_one, range(len(sources))))
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="agq_build_") as tmpdir:
        with ThreadPoolExecutor(max_workers=2) as ex:
            main = ex.submit(_link, SOURCES, LIB, verbose, tmpdir)
            calib = ex.submit(_link, CALIB_SOURCES, CALIB_LIB, verbose, tmpdir)
            main.result()
            calib.result()
    return LIB


if __name__ == "__main__":
    build(verbose=True)
