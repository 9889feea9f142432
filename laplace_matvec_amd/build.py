"""Build the LAPLEX HIP libraries for gfx950 with hipcc.

Outputs, next to this file:
  liblaplex.so         the operator library (C ABI of include/laplex.h)
  liblaplex_inputs.so  the device input generator (Philox4x32-10) and a
                       plain copy kernel for counter calibration, kept
                       separate because they are not part of the operator
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("LAPLEX_ARCH", "gfx950")

LIB_SOURCES = ["api.hip", "sort.hip", "small.hip", "scan.hip", "general.hip", "gram.hip", "grad.hip", "merge.hip"]
INPUT_SOURCES = ["inputs_philox.hip", "calib_copy.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-munsafe-fp-atomics",
    # keep the compiler from emitting packed fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if r.stderr.strip():
        warn = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
        if warn:
            sys.stderr.write(r.stderr)
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {out}:\n{r.stderr}")
    os.replace(tmp, out)


def build(jobs: int = 8) -> list[str]:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        lib_objs = list(ex.map(_compile, LIB_SOURCES))
        in_objs = list(ex.map(_compile, INPUT_SOURCES))
    outs = [os.path.join(PKG, "liblaplex.so"), os.path.join(PKG, "liblaplex_inputs.so")]
    _link(lib_objs, outs[0])
    _link(in_objs, outs[1])
    return outs


if __name__ == "__main__":
    for p in build():
        print(p)
