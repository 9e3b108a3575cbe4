"""Build liboscar.so in-tree for gfx950: hipcc for the HIP sources, g++ for the
host-only calibration code, then one shared library next to this file."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liboscar.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")

HIP_SOURCES = ["abi.hip", "quantize_append.hip", "decode.hip", "calib.hip", "probe.hip", "noalloc.hip", "attend.hip"]
CXX_SOURCES = ["rotation_host.cpp"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
             # hipcc -O3 forms packed fp32 arithmetic by itself; keep it off
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
CXX_FLAGS = ["-O3", "-march=x86-64-v3", "-std=c++17", "-fPIC", "-pthread", "-Wall"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link liboscar.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I" + os.path.join(HERE, "..", "include")]
    jobs = []
    for s in HIP_SOURCES:
        jobs.append([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", os.path.join(BUILD, s + ".o")])
    for s in CXX_SOURCES:
        jobs.append(["g++", *CXX_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", os.path.join(BUILD, s + ".o")])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SOURCES + CXX_SOURCES]
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-pthread", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
