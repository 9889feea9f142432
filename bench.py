#!/usr/bin/env python3
"""Benchmark of the LAPLEX operator apply on one MI355X.

Default workload (the headline measurement): symmetric apply y = K(a, a) x
at n = 2^30, float32, one vector, a ~ 1e4 N(0,1) and x ~ N(0,1) drawn on the
device (Philox4x32-10), timed END TO END with laplex_plan_create_apply: the
radix argsort of the anchors (x travelling through its passes), the prefix
and suffix scans, the replay of y back to original order, plan release.

One step = one pass of the whole path over the resident inputs.  W untimed
warm-up steps, then K timed steps between device synchronizations; kernel
durations come from HIP events recorded by the library around each launch
in the same timed region.  Rank 0 prints one JSON line.

Other workloads (for the record, not the headline line): --workload
c1 | c2 | c3 | c4 (see laplace_matvec_amd/workloads.py); --backward times a
training step (forward product plus its backward pass) instead.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD published
METRIC = "LAPLEX apply elements/s + achieved HBM GB/s (% peak), symmetric n=2^30, 1 GPU"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="c5", choices=["c1", "c2", "c3", "c4", "c5"])
    p.add_argument("--n", type=int, default=None, help="override n (testing only)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=1 << 26)
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run a plain 1 GiB device copy (counter calibration)")
    p.add_argument("--backward", action="store_true",
                   help="time a training step instead: forward product plus its backward pass "
                        "(input and anchor gradients, and phase gradients for a phased operator)")
    return p.parse_args()


# --------------------------------------------------------------- byte model
# Algorithmic bytes per launch of each kernel (what the algorithm must move,
# not what the counters see), for a sorted side of n anchors, B vectors and
# C phase channels.  Radix passes: 4 B key in, 4 B key out, 2 B replay record
# per key, plus a 6 B x 256 table per 8192-key tile.

TILE_TABLE = 6.0 * 256 / 8192


def model_bytes(kernel: str, n: int, batch: int = 1, channels: int = 1, vals: int = 0) -> float | None:
    """vals: value rows carried by each radix pass (read and written)."""
    factors = 8.0 if channels == 2 else 0.0
    per = {
        "sort_hist": 4.0,
        "sort_pass": 10.0 + TILE_TABLE + 8.0 * vals,
        "replay_forward": 2.0 + TILE_TABLE + 8.0 * batch,
        "replay_backward": 2.0 + TILE_TABLE + 8.0 * batch,
        "scan_reduce": 4.0 + factors + 4.0 * batch,
        "scan_apply": 4.0 + 2 * factors + 8.0 * batch,
        "scan_reduce_gather": 8.0 + factors + 8.0 * batch,
        "scan_apply_scatter": 8.0 + 2 * factors + 8.0 * batch,
        # gradient by rank: s, u and w read; the apply also writes the anchor
        # row, dx and (phased) the two phase rows
        "grad_reduce": 4.0 + 2 * factors + 8.0 * batch,
        "grad_apply": 4.0 + 2 * factors + 8.0 * batch + 4.0 + 4.0 * batch + factors,
    }.get(kernel)
    return None if per is None else per * n


def model_step_bytes(n: int, batch: int) -> float:
    """Whole symmetric step (plan_create_apply on the replay path: the rows
    of x travel with the keys through the four radix passes)."""
    launches = {"sort_hist": 1, "sort_pass": 4, "scan_reduce": 1, "scan_apply": 1, "replay_backward": 4}
    return sum(c * model_bytes(k, n, batch, vals=batch) for k, c in launches.items())


def counter_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if
    their recorded source hash still matches the kernel source."""
    for path in glob.glob(os.path.join(ROOT, "profiles", "*counters*.txt")):
        kv = {}
        for line in open(path):
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel") != kernel or kv.get("workload") != workload:
            continue
        src = os.path.join(ROOT, "laplace_matvec_amd", "csrc", kv.get("source", ""))
        if not os.path.exists(src):
            continue
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
        if sha != kv.get("source_sha"):
            return None
        try:
            return float(kv["hbm_bytes_per_launch"])
        except (KeyError, ValueError):
            return None
    return None


def counter_step_bytes(workload: str):
    """HBM bytes of one whole step from the committed rocprofv3 counter
    record (every kernel of the step, calibrated FETCH_SIZE + WRITE_SIZE),
    if the hashes of all the kernel sources it names still match."""
    for path in glob.glob(os.path.join(ROOT, "profiles", "*counters*.txt")):
        kv = {}
        for line in open(path):
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
        if kv.get("kernel") != "step" or kv.get("workload") != workload:
            continue
        srcs = kv.get("source", "").split(",")
        shas = kv.get("source_sha", "").split(",")
        if len(srcs) != len(shas):
            return None
        for src, want in zip(srcs, shas):
            path_src = os.path.join(ROOT, "laplace_matvec_amd", "csrc", src)
            if not os.path.exists(path_src):
                return None
            if hashlib.sha256(open(path_src, "rb").read()).hexdigest()[:16] != want:
                return None
        try:
            return float(kv["hbm_bytes_per_step"])
        except (KeyError, ValueError):
            return None
    return None


def cpu_baseline(sample: int):
    """The fp64 oracle (sort + two sweeps, single thread) on a bounded sample
    of the same workload; elements/s."""
    import numpy as np

    import oracle
    from laplace_matvec_amd import workloads as wl
    a = wl.normal(sample, 5, wl.S_A, 0.0, 1.0e4)
    x = wl.normal(sample, 5, wl.S_X)
    oracle.apply_sweep(a[:4096], x[:4096])  # load/build outside the timing
    t0 = time.perf_counter()
    y = oracle.apply_sweep(a, x)
    dt = time.perf_counter() - t0
    assert np.isfinite(y).all()
    return {"value": sample / dt, "unit": "elements/s", "cores": 1, "kind": "oracle",
            "sample": f"symmetric n={sample} (a ~ 1e4 N(0,1), x ~ N(0,1), same streams), "
                      f"fp64 qsort argsort + two sweeps, {dt:.1f} s on 1 host thread "
                      f"(host has {os.cpu_count()} logical CPUs)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from laplace_matvec_amd import laplex as lx
    from laplace_matvec_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        # a plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch
        # give the factor between those counters and bytes moved
        src = torch.ones(1 << 28, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cfg = int(args.workload[1])
    W = wl.WORKLOADS[cfg]
    n = args.n or W.n
    inp = wl.device_config_inputs(cfg, n=n, device=dev, with_w=True)
    torch.cuda.synchronize()
    batch = W.batch

    if W.kind == "sym" and args.backward:
        a, x = inp["a"], inp["x"]
        g = wl.device_normal(tuple(x.shape), cfg, wl.S_W, device=dev)
        y = torch.empty_like(x)
        dx = torch.empty_like(x)
        da = torch.empty(n, device=dev)
        lib = lx.load()
        import ctypes

        def step():
            plan, _ = lx.laplex_plan_create_apply(a, x, y)
            # x = NULL: the plan kept the rows of x it sorted
            st = lib.laplex_backward(plan.handle, None, ctypes.c_void_p(g.data_ptr()),
                                     batch, 0, ctypes.c_void_p(dx.data_ptr()), ctypes.c_void_p(da.data_ptr()),
                                     None, None, None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != lx.OK:
                raise lx.LaplexError(st, "laplex_backward")
            plan.destroy()
        elements = n * batch
        desc = {"workload": W.name, "n": n, "batch": batch,
                "path": "training step: plan_create_apply + backward (dx, da) (end to end)",
                "anchors": "a ~ 1e4 N(0,1)" if cfg == 5 else W.note}
    elif W.kind == "sym":
        a, x = inp["a"], inp["x"]
        y = torch.empty_like(x)

        def step():
            plan, _ = lx.laplex_plan_create_apply(a, x, y)
            plan.destroy()
        elements = n * batch
        desc = {"workload": W.name, "n": n, "batch": batch,
                "path": "plan_create_apply: sort + apply (end to end)",
                "anchors": "a ~ 1e4 N(0,1)" if cfg == 5 else W.note}
    elif W.kind == "general" and args.backward:
        plan = lx.laplex_plan_create(inp["a"], b=inp["b"], phi=inp["phi"], psi=inp["psi"])
        y = torch.empty((batch, n), device=dev)

        def step():
            lx.laplex_apply(plan, inp["x"], y)
            lx.laplex_backward(plan, inp["x"], inp["w"])
        elements = n * batch
        desc = {"workload": W.name, "n": n, "k": W.k, "batch": batch,
                "path": "training step through y=Kx: apply + backward (dx, da, db, dphi, dpsi), plan excluded"}
    elif W.kind == "general":
        plan = lx.laplex_plan_create(inp["a"], b=inp["b"], phi=inp["phi"], psi=inp["psi"])
        y = torch.empty((batch, n), device=dev)
        z = torch.empty((batch, W.k), device=dev)

        def step():
            lx.laplex_apply(plan, inp["x"], y)
            lx.laplex_apply(plan, inp["w"], z, transpose=True)
        elements = 2 * n * batch
        desc = {"workload": W.name, "n": n, "k": W.k, "batch": batch, "path": "apply y=Kx and z=K^T w (plan excluded)"}
    else:
        plan = lx.laplex_plan_create(inp["a"], b=inp["b"])
        M = torch.empty((n, n), device=dev)

        def step():
            lx.laplex_gram(plan, inp["D"], M)
        elements = n * n
        desc = {"workload": W.name, "n": n, "k": W.k, "path": "gram (plan excluded)"}

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    lx.profile_reset()
    lx.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = lx.profile_read()
    lx.profile_enable(False)
    ms = (t1 - t0) * 1e3 / args.steps

    kernels = {}
    for name, (cnt, tot) in prof.items():
        per = cnt / args.steps
        kernels[name] = {"launches_per_step": per, "avg_ms": tot / cnt, "ms_per_step": tot / args.steps}
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"]) if kernels else None
    roof = None
    if dominant:
        ab = model_bytes(dominant, n, batch, vals=batch if W.kind == "sym" else 0)
        avg_s = kernels[dominant]["avg_ms"] / 1e3
        if ab is not None:
            ach = ab / avg_s / 1e9
            roof = {"bound": "hbm", "kernel": dominant, "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4),
                    "traffic": counter_traffic(dominant, W.name),
                    "algorithmic_bytes_per_launch": ab, "avg_launch_ms": kernels[dominant]["avg_ms"]}
    # whole-step model bandwidth (symmetric end to end: 4 + 60 sort + 32 apply bytes/elem at B=1)
    extra = {}
    if W.kind == "sym" and not args.backward:
        model = model_step_bytes(n, batch)
        extra["model_bytes_per_step"] = model
        extra["model_gbps_end_to_end"] = round(model / (ms / 1e3) / 1e9, 1)
        extra["model_frac_end_to_end"] = round(model / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)
        # bytes any implementation must move: read a and x, write y
        comp = (4.0 + 8.0 * batch) * n
        extra["compulsory_bytes_per_step"] = comp
        extra["compulsory_gbps_end_to_end"] = round(comp / (ms / 1e3) / 1e9, 1)
        # what the HBM counters saw for a whole step (committed record), over this run's step time
        cb = counter_step_bytes(W.name)
        extra["counter_bytes_per_step"] = cb
        extra["counter_gbps_end_to_end"] = None if cb is None else round(cb / (ms / 1e3) / 1e9, 1)
        extra["counter_frac_end_to_end"] = None if cb is None else round(cb / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)
    out = {
        "metric": (METRIC if cfg == 5 else f"LAPLEX {W.kind} elements/s ({W.name})") if not args.backward
        else f"LAPLEX training step (forward + backward) elements/s ({W.name})",
        "value": elements / (ms / 1e3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (fp64 scan arithmetic, u32 sort keys)",
        "data": "synthetic (Philox4x32-10 on device)",
        "config": desc,
        "roofline": roof,
        "kernels": {k: {kk: round(vv, 5) for kk, vv in v.items()} for k, v in kernels.items()},
        **extra,
    }
    if cfg == 5 and not args.no_cpu_baseline and not args.backward:
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
