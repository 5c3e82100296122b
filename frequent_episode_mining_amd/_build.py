"""Builds libepcount.so (HIP, gfx950) in-tree with hipcc.

The per-N kernel unit (csrc/ep_inst.hip) is compiled once per episode size N
in 1..16 with -DEP_N=<N>, in parallel, and linked with the host unit
(csrc/ep_api.hip) into frequent_episode_mining_amd/libepcount.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libepcount.so")
MAX_NODES = 16
ARCH = "gfx950"

# Packed-FP32 instructions are kept out of every kernel.
HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library can not be built")
    return path


def _compile(args):
    src, obj, defines = args
    cmd = [hipcc()] + HIPCC_FLAGS + defines + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every HIP unit for gfx950 and link libepcount.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(16, os.cpu_count() or 4)
    units = [(os.path.join(CSRC, "ep_api.hip"), os.path.join(BUILD, "ep_api.o"), []),
             (os.path.join(CSRC, "ep_mine.hip"), os.path.join(BUILD, "ep_mine.o"), [])]
    for n in range(1, MAX_NODES + 1):
        units.append((os.path.join(CSRC, "ep_inst.hip"), os.path.join(BUILD, "ep_inst_n%d.o" % n),
                      ["-DEP_N=%d" % n]))
    # largest episode sizes first: they take longest
    units = units[:2] + units[2:][::-1]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, units))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC"] + sorted(objs) + ["-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), res.stdout, res.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
