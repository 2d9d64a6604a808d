"""Builds libmxfp8.so (the HIP kernels + C ABI) for gfx950 with hipcc.

    python -m quantize_grouped_gemm_amd.build [--resource-usage]

Objects go to _build/ at the repository root; the library is written next to
this file so it is found in-tree.
"""

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfp8.so")
SOURCES = ["mx_quant.hip", "mx_gemm.hip", "mx_pad_hp.hip", "mx_fp8.hip", "mx_abi.cpp"]
ARCH = "gfx950"

# -packed-fp32-ops keeps the compiler from emitting packed float32 VALU ops.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Wno-unused-function", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmxfp8.so")
    return exe


def _compile(src, resource_usage=False):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage and src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False, resource_usage=False):
    """Compile every source and link libmxfp8.so. Always recompiles."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_usage), SOURCES))
    objs = [o for o, _ in results]
    if verbose or resource_usage:
        for src, (_, err) in zip(SOURCES, results):
            if err.strip():
                print(f"--- {src}\n{err}", file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(args.verbose, args.resource_usage))
