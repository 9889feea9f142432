#!/usr/bin/env python3
"""Benchmark of the LAPLEX operator apply on one MI355X.

Default workload (the headline measurement): symmetric apply y = K(a, a) x
at n = 2^30, float32, one vector, a ~ 1e4 N(0,1) and x ~ N(0,1) drawn on the
device (Philox4x32-10), timed END TO END with laplex_plan_create_apply: the
radix argsort of the anchors (x travelling through its passes), the prefix
and suffix scans, the replay of y back to original order, plan release.

One step = one pass of the whole path over the resident inputs.  W untimed
warm-up steps; then K untimed steps with HIP events recorded by the library
around every launch, for the per-kernel breakdown and to find the dominant
kernel; then K timed steps between device synchronizations, with events
around the dominant kernel's launches only (its roofline time is measured
there, live; an event record between every pair of launches would add
several microseconds to short steps).  Rank 0 prints one JSON line.

Other workloads (for the record, not the headline line): --workload
c1 | c2 | c3 | c4 (see laplace_matvec_amd/workloads.py); --backward times a
training step (forward product plus its backward pass) instead.
"""
from __future__ import annotations

import argparse
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


# --------------------------------------------------------------- byte models
# Two byte counts per launch of each kernel, for a sorted side of n anchors,
# B vectors and C phase channels:
#
#  * survey bytes: the hot-path scope table's per-element figures (the bytes
#    the method's steps move in a plain design: a radix pass reads and
#    writes key + index, 12 B for the first pass and 16 B for each later
#    one; the scan reads s and x twice and writes y once; the gather and the
#    scatter each move an index, the value in and the value out).  The
#    roofline fraction is quoted on these.  When x travels through the
#    radix passes as value rows (plan_create_apply), those passes carry out
#    the gather, so each of the four launches is credited with a quarter of
#    the gather's bytes (4 + 8B per element); the sort's own share is given
#    beside it.  General case: the evaluation reads the output anchors and
#    phase factors and writes y (4 + 8 + 4B), the bucketing reads w (4B) and
#    its layout pass the input anchors and phase factors (4 + 8).
#  * design bytes: what this design's kernels must move: radix passes carry
#    x as a value row and write replay records (2 B per key plus a 6 B x 256
#    table per 8192-key tile) instead of an index; the four backward replays
#    read the records again.

TILE_TABLE = 6.0 * 256 / 8192
SURVEY_SORT_PASS = (12.0 + 16.0 + 16.0 + 16.0) / 4  # average over the four launches of one sort


def survey_bytes(kernel: str, n: int, batch: int = 1, channels: int = 1, carried_rows: int = 0) -> float | None:
    factors = 8.0 if channels == 2 else 0.0
    per = {
        "sort_hist": 4.0,
        "sort_pass": SURVEY_SORT_PASS + ((4.0 + 8.0 * carried_rows) / 4 if carried_rows else 0.0),
        "eval": 4.0 + factors + 4.0 * batch,
        "bucket_layout": 4.0 + factors,
        "bucket_sorted": 4.0 * batch,
        "small_sym": 4.0 + factors + 8.0 * batch,
        # one gather (index, value in, value out) and one scatter, each
        # spread over the four replays that carry it out
        "replay_forward": (4.0 + 8.0 * batch) / 4,
        "replay_backward": (4.0 + 8.0 * batch) / 4,
        "scan_reduce": 4.0 + factors + 4.0 * batch,
        "scan_apply": 4.0 + 2 * factors + 8.0 * batch,
        "scan_reduce_gather": 8.0 + factors + 8.0 * batch,
        "scan_apply_scatter": 8.0 + 2 * factors + 8.0 * batch,
    }.get(kernel)
    return None if per is None else per * n


def model_bytes(kernel: str, n: int, batch: int = 1, channels: int = 1, vals: int = 0) -> float | None:
    """Design bytes; vals: value rows carried by each radix pass (read and written)."""
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


SYM_STEP = {"sort_hist": 1, "sort_pass": 4, "scan_reduce": 1, "scan_apply": 1, "replay_backward": 4}


def survey_step_bytes(n: int, batch: int) -> float:
    """Whole symmetric step by the scope table: sort 68, gather 4 + 8B,
    scan 8 + 12B, scatter 4 + 8B bytes per element (112 at B = 1)."""
    return (68.0 + (4.0 + 8.0 * batch) + (8.0 + 12.0 * batch) + (4.0 + 8.0 * batch)) * n


def model_step_bytes(n: int, batch: int) -> float:
    """Whole symmetric step by design bytes (plan_create_apply on the replay
    path: the rows of x travel with the keys through the four radix passes)."""
    return sum(c * model_bytes(k, n, batch, vals=batch) for k, c in SYM_STEP.items())


# Kernel labels of each phase of the path.
PHASES = {
    "sort": ("util_fill", "sort_hist", "sort_scan_hist", "sort_pass", "perm_replay"),
    "scan": ("scan_reduce", "scan_carry", "scan_apply", "scan_reduce_gather", "scan_apply_scatter",
             "scan_reduce_uv", "scan_apply_tables"),
    "gather_scatter": ("replay_forward", "replay_backward"),
}


def gram_bytes(kernel: str, n: int, k: int, weight_sets: int = 1) -> float | None:
    """Gram: the M write (4 B per entry), b and D read once (8 B per column
    anchor), the sorted rows (4 B each)."""
    return {"gram_tile": 4.0 * n * n, "gram_bins": 8.0 * k + 4.0 * n,
            "gram_scan": (8.0 * 3 * weight_sets + 4.0) * n}.get(kernel)


def counter_record(workload: str):
    """The committed rocprofv3 counter record of a workload, if it was taken
    from the current library sources (else None)."""
    from laplace_matvec_amd import counters
    return counters.find_record(workload, ROOT)


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
        # a plain copy of known size (1 GiB read, 1 GiB written, one
        # dispatch): its FETCH_SIZE / WRITE_SIZE give the factor between
        # those counters and bytes moved
        src = torch.ones(1 << 28, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            wl.device_copy(src, dst)
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
    # Per-kernel breakdown: the same number of steps with every launch
    # bracketed by timing events, outside the timed region (each event
    # record adds a packet between launches, visible on short steps).
    lx.profile_only(None)
    lx.profile_reset()
    lx.profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof_all = lx.profile_read()
    lx.profile_enable(False)
    kernels = {}
    for name, (cnt, tot) in prof_all.items():
        kernels[name] = {"launches_per_step": cnt / args.steps, "avg_ms": tot / cnt, "ms_per_step": tot / args.steps}
    dominant = max(kernels, key=lambda k: kernels[k]["ms_per_step"]) if kernels else None

    # Timed region: K steps, with timing events around the launches of the
    # dominant kernel only; its average launch time below is from these.
    lx.profile_only(dominant)
    lx.profile_reset()
    lx.profile_enable(dominant is not None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    prof = lx.profile_read()
    lx.profile_enable(False)
    lx.profile_only(None)
    ms = (t1 - t0) * 1e3 / args.steps
    live = prof.get(dominant) if dominant else None
    dominant_avg_ms = live[1] / live[0] if live and live[0] else None

    rec = counter_record(W.name)
    rec_labels = rec["labels"] if rec else {}
    channels = 2 if W.phased else 1
    carried = batch if W.kind == "sym" else 0  # value rows through the radix passes
    roof = None
    if dominant and dominant_avg_ms:
        avg_s = dominant_avg_ms / 1e3
        if W.kind == "gram":
            ab = gram_bytes(dominant, n, W.k)
            design = ab
        else:
            ab = survey_bytes(dominant, n, batch, channels, carried)
            design = model_bytes(dominant, n, batch, vals=carried)
        if ab is not None:
            ach = ab / avg_s / 1e9
            traffic = rec_labels.get(dominant, (None, None))[1]
            roof = {"bound": "hbm", "kernel": dominant, "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4), "traffic": traffic,
                    "algorithmic_bytes_per_launch": ab, "avg_launch_ms": round(dominant_avg_ms, 6),
                    "design_bytes_per_launch": design,
                    "design_frac": None if design is None else round(design / avg_s / 1e9 / PEAK_HBM_GBPS, 4),
                    "counter_record": rec["path"] if rec else None}
            if dominant == "sort_pass" and carried:
                sort_only = survey_bytes("sort_pass", n, batch)
                roof["sort_only_bytes_per_launch"] = sort_only
                roof["sort_only_frac"] = round(sort_only / avg_s / 1e9 / PEAK_HBM_GBPS, 4)
                roof["bytes_note"] = ("scope-table bytes of one radix pass (12 B per element for the first, "
                                      "16 for the others) plus a quarter of the gather's (4 + 8B per element), "
                                      "which these passes carry out with x travelling as value rows")
    extra = {}
    # per phase: time in this run, survey / design bytes, and what the counters saw
    phases = {}
    for ph, labels in PHASES.items():
        ms_ph = sum(kernels[k]["ms_per_step"] for k in labels if k in kernels)
        if ms_ph == 0:
            continue
        d = {"ms_per_step": round(ms_ph, 4)}
        sb = [survey_bytes(k, n, batch, channels, carried) * kernels[k]["launches_per_step"] for k in labels
              if k in kernels and survey_bytes(k, n, batch, channels, carried) is not None]
        if W.kind == "sym" and sb:
            d["survey_gbps"] = round(sum(sb) / (ms_ph / 1e3) / 1e9, 1)
        cb = [rec_labels[k][0] * rec_labels[k][1] for k in labels if k in kernels and k in rec_labels]
        if rec and cb:
            d["counter_bytes_per_step"] = sum(cb)
            d["counter_gbps"] = round(sum(cb) / (ms_ph / 1e3) / 1e9, 1)
            d["counter_frac"] = round(sum(cb) / (ms_ph / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)
        phases[ph] = d
    if phases:
        extra["phases"] = phases
    if W.kind == "sym" and not args.backward:
        sv = survey_step_bytes(n, batch)
        extra["survey_bytes_per_step"] = sv
        extra["survey_frac_end_to_end"] = round(sv / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)
        model = model_step_bytes(n, batch)
        extra["design_bytes_per_step"] = model
        extra["design_frac_end_to_end"] = round(model / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)
        # bytes any implementation must move: read a and x, write y
        comp = (4.0 + 8.0 * batch) * n
        extra["compulsory_bytes_per_step"] = comp
        extra["compulsory_gbps_end_to_end"] = round(comp / (ms / 1e3) / 1e9, 1)
    if rec:
        # what the HBM counters saw for a whole step (committed record taken
        # from these sources), over this run's step time
        cbs = float(rec["step_bytes"])
        extra["counter_bytes_per_step"] = cbs
        extra["counter_gbps_end_to_end"] = round(cbs / (ms / 1e3) / 1e9, 1)
        extra["counter_frac_end_to_end"] = round(cbs / (ms / 1e3) / 1e9 / PEAK_HBM_GBPS, 4)
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
        "kernels_from": "an instrumented pass of K steps before the timed region (every launch bracketed)",
        **extra,
    }
    if cfg == 5 and not args.no_cpu_baseline and not args.backward:
        out["cpu_baseline"] = cpu_baseline(args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
