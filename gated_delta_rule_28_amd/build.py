"""Build libkda.so (gfx950) in-tree with hipcc.

Usage: python -m gated_delta_rule_28_amd.build   (or build() from Python)
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libkda.so")
PEAKS_OUT = os.path.join(HERE, "libkda_peaks.so")  # measured-peak microbenchmarks (bench only)
BUILD_DIR = os.path.join(HERE, "_build")
ARCH = "gfx950"

SOURCES = ["kda_api.cpp", "kda_backward.hip", "kda_cp.hip", "kda_decode.hip", "kda_prefill.hip",
           "kda_prefill_split.hip"]
PEAKS_SOURCES = ["kda_peaks.hip"]

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 VALU forms stay off (see the ISA notes in kda_device.h)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-8000:]}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libkda.so (and the
    measured-peak library libkda_peaks.so) next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], OUT)
    _link([objs[s] for s in PEAKS_SOURCES], PEAKS_OUT)
    if verbose:
        print(f"built {OUT} and {PEAKS_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
