"""Build the LAPLEX HIP libraries for gfx950 with hipcc.

Outputs, next to this file:
  liblaplex.so         the operator library (C ABI of include/laplex.h)
  liblaplex_stress.so  the same library with 4096-key sort tiles and a
                       look-back that reads one predecessor per round: twice
                       the tiles and the longest look-back walks, for the
                       sort stress test only
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


STRESS_DEFINES = ["-DLX_SORT_THREADS=256", "-DLX_SORT_ITEMS=16", "-DLX_LOOKBACK=1"]


def _compile(src: str, variant: str = "", defines: tuple = ()) -> str:
    out_dir = os.path.join(BUILD, variant) if variant else BUILD
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC, *FLAGS, *defines, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
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
        stress_objs = list(ex.map(lambda f: _compile(f, "stress", tuple(STRESS_DEFINES)), LIB_SOURCES))
    outs = [os.path.join(PKG, "liblaplex.so"), os.path.join(PKG, "liblaplex_inputs.so"),
            os.path.join(PKG, "liblaplex_stress.so")]
    _link(lib_objs, outs[0])
    _link(in_objs, outs[1])
    _link(stress_objs, outs[2])
    return outs


if __name__ == "__main__":
    for p in build():
        print(p)
