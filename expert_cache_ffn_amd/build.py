"""Build libecf.so in-tree for gfx950 with hipcc (no GPU needed to compile)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libecf.so")
BUILD = os.path.join(os.path.dirname(HERE), "_build")

HIP_SRCS = ["k_route.hip", "k_decode.hip", "k_prefill.hip", "k_util.hip", "noalloc.hip"]
CPP_SRCS = ["api.cpp", "cache.cpp", "qstar.cpp", "host_ffn.cpp", "bwprof.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", "-I", os.path.join(os.path.dirname(HERE), "include")]
# Packed fp32 ops off in device code (they are generated from plain float code otherwise).
HIP_FLAGS = COMMON + [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                      "-munsafe-fp-atomics"]
CPP_FLAGS = COMMON + ["-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for s in HIP_SRCS:
        jobs.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", os.path.join(BUILD, s + ".o")])
    for s in CPP_SRCS:
        jobs.append([HIPCC, *CPP_FLAGS, "-c", os.path.join(CSRC, s), "-o", os.path.join(BUILD, s + ".o")])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    objs = [os.path.join(BUILD, s + ".o") for s in HIP_SRCS + CPP_SRCS]
    tmp = OUT + ".tmp"
    _run([HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs, "-lpthread"])
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
