"""Build libexseq.so in-tree with hipcc for gfx950.

    python -m bit_exact_sequential_amd.build              # the library
    python -m bit_exact_sequential_amd.build --timeline   # its diagnostic twin

The diagnostic twin, libexseq_timeline.so, is the same sources with
EXSEQ_TIMELINE defined: the exact chain's tiles record the GPU's real-time
counter at their steps (read by ``python -m bit_exact_sequential_amd.timeline``).

Every HIP translation unit is compiled with -ffp-contract=off (no multiply
is ever fused into an add: the SSIM term is defined with one rounding per
operation), without fast-math, with fp64 denormals kept, and without packed
fp32 instructions.  Objects go to ``_build/``; the library next to this file.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libexseq.so")
SOURCES = ("exseq_api.cpp", "exseq_model.cpp", "exseq_twin.cpp", "exseq_sum.hip", "exseq_pass.hip",
           "exseq_ssim.hip")
ARCH = "gfx950"

COMMON = [
    "-O3", "-fPIC", "-std=c++17",
    "--offload-arch=" + ARCH,
    "-ffp-contract=off", "-fno-fast-math",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


TIMELINE_BUILD = os.path.join(HERE, "_build_timeline")
TIMELINE_LIB = os.path.join(HERE, "libexseq_timeline.so")


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(verbose: bool = False, timeline: bool = False) -> str:
    build_dir, lib, extra = BUILD, LIB, ()
    if timeline:
        build_dir, lib, extra = TIMELINE_BUILD, TIMELINE_LIB, ("-DEXSEQ_TIMELINE",)
    os.makedirs(build_dir, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, extra), SOURCES))
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, lib)
    if verbose:
        print("built", lib)
    return lib


if __name__ == "__main__":
    build(verbose=True, timeline="--timeline" in sys.argv[1:])
    sys.exit(0)
