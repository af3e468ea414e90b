"""Build libkda.so (all HIP sources under csrc/) for gfx950 with hipcc, in-tree.

Every translation unit is compiled to _build/<name>.o in parallel, then linked
into gated_delta_rule_47_amd/libkda.so.  Packed-fp32 instructions are disabled
on purpose (-packed-fp32-ops): plain fp32 VALU code only.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkda.so")
ARCH = "gfx950"
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    p = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx950-only feature flag; that note is harmless.
    err = "\n".join(l for l in p.stderr.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), err))
    return err


def build(jobs: int | None = None, verbose: bool = False) -> str:
    """Compile every source and link libkda.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources under " + CSRC)
    jobs = jobs or min(8, len(os.sched_getaffinity(0)))

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        warn = _run([HIPCC] + FLAGS + ["-c", src, "-o", obj])
        if verbose and warn.strip():
            print(warn, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(compile_one, sources))
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
