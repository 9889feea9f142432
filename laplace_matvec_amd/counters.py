"""HBM traffic and kernel-time records from rocprofv3 (measurement tooling).

Two rocprofv3 counter runs of the same benchmark command, one with
``--pmc FETCH_SIZE`` and one with ``--pmc WRITE_SIZE``, give per-dispatch
counter values in KiB.  The command also runs a plain device copy of a known
size (``bench.py --calibrate-copy``: 1 GiB read and written by one dispatch
of the input library's copy kernel, 4-byte accesses like the operator's
streaming kernels), so the factor between each counter and the bytes
actually moved is measured on the same box in the same process.  (The
runtime's own blit kernel is not used: its counters scale differently from
those of plain loads and stores.)  This module folds the
dispatches into HBM bytes per launch of each kernel label the library uses
for its own timing events, and writes a text record that ``bench.py`` reads:

    workload=<workload name>
    source_sha=<digest of every library source: csrc/*.hip, csrc/*.h, include/*.h>
    steps=<steps the profiled command ran (warm-up included)>
    fetch_factor=<bytes per FETCH_SIZE KiB / 1024>
    write_factor=<bytes per WRITE_SIZE KiB / 1024>
    label.<label>=<launches per step> <HBM bytes per launch>
    step_bytes=<HBM bytes of one step over every library kernel>

A record whose source digest differs from the current sources is stale and
``bench.py`` ignores it.  ``stats`` turns a ``--kernel-trace --stats``
kernel_stats CSV into a markdown table.

    python -m laplace_matvec_amd.counters record --fetch F.csv --write W.csv \
        --workload sym_n2^30 --steps 3 --command "..." --out profiles/X_counters.txt
    python -m laplace_matvec_amd.counters stats --csv S.csv --title "..." \
        --command "..." --out profiles/X_kernel_stats.md
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)

COPY_BYTES = 1 << 30  # bytes read (and written) by one calibration copy dispatch
COPY_KERNEL = "lx_calib_copy"  # the input library's plain copy kernel


def source_files(root: str = ROOT) -> list[str]:
    pats = [os.path.join(root, "laplace_matvec_amd", "csrc", "*.hip"),
            os.path.join(root, "laplace_matvec_amd", "csrc", "*.h"),
            os.path.join(root, "include", "*.h")]
    files = []
    for p in pats:
        files += glob.glob(p)
    return sorted(files, key=lambda f: os.path.relpath(f, root))


def source_digest(root: str = ROOT) -> str:
    """Digest over the names and contents of every library source file."""
    h = hashlib.sha256()
    for f in source_files(root):
        h.update(os.path.relpath(f, root).encode())
        h.update(b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
        h.update(b"\0")
    return h.hexdigest()[:16]


# rocprofv3 kernel name -> the label of the library's timing event for it
# (the names passed to LX_LAUNCH in csrc/).
def label_of(kernel: str) -> str | None:
    k = kernel.strip().replace("(anonymous namespace)::", "")
    base = re.split(r"[<(]", k, 1)[0].strip()
    base = base.split("::")[-1]
    args = k[len(k.split("<", 1)[0]):] if "<" in k else ""
    targs = [t.strip() for t in args.strip("<>").split(">")[0].split(",")] if args else []
    if base in ("lx_gen", "lx_calib_copy"):
        return None  # the input library (inputs and the calibration copy), not the operator
    if base in ("lx_fill_u32", "lx_sort_clear"):
        return "util_fill"
    if base in ("lx_sort_hist", "lx_sort_scan_hist", "lx_sort_pass"):
        return base[3:]
    if base == "lx_replay_fwd2":
        return "perm_replay" if "unsigned int" in args else "replay_forward"
    if base == "lx_replay_bwd2":
        return "replay_backward"
    if base == "lx_replay":
        if "unsigned int" in args:
            return "perm_replay"
        return "replay_forward" if len(targs) > 1 and targs[1] == "true" else "replay_backward"
    if base in ("lx_scan_reduce", "lx_scan_apply"):
        mode = int(targs[1]) if len(targs) > 1 and targs[1].isdigit() else 0
        rnd = len(targs) > 2 and targs[2] == "true"
        if base == "lx_scan_reduce":
            return "scan_reduce_uv" if mode in (1, 3) else ("scan_reduce_gather" if rnd else "scan_reduce")
        return "scan_apply_tables" if mode in (2, 3) else ("scan_apply_scatter" if rnd else "scan_apply")
    if base in ("lx_scan_carry_groups", "lx_scan_carry_tiles"):
        return "scan_carry"
    named = {"lx_eval_rows": "eval", "lx_eval_grad_rows": "eval_grad", "lx_grad_sym_apply": "grad_apply",
             "lx_grad_sym_reduce": "grad_reduce", "lx_phase_factors": "plan_phase",
             "lx_check_finite": "plan_check"}
    if base in named:
        return named[base]
    if base.startswith("lx_"):
        return base[3:]
    return None


def _rows(path: str):
    with open(path, newline="") as fh:
        yield from csv.DictReader(fh)


def _col(row: dict, *names):
    for n in names:
        for k in row:
            if k.strip().lower() == n.lower():
                return row[k]
    raise KeyError(f"none of {names} in {list(row)}")


def dispatch_counters(path: str, counter: str) -> list[tuple[str, float]]:
    """(kernel name, counter value) per dispatch, in dispatch order."""
    out = []
    for r in _rows(path):
        if _col(r, "Counter_Name").strip() != counter:
            continue
        out.append((_col(r, "Kernel_Name"), float(_col(r, "Counter_Value"))))
    return out


def calibration_factor(disp: list[tuple[str, float]], bytes_per_dispatch: int) -> float:
    """Bytes per counter KiB, from the dispatches of the calibration copy
    kernel (each moves `bytes_per_dispatch` one way)."""
    vals = [v for name, v in disp if COPY_KERNEL in name]
    if not vals:
        raise ValueError("no calibration copy dispatch found (run the command with --calibrate-copy)")
    mean = sum(vals) / len(vals)
    return bytes_per_dispatch / (mean * 1024.0)


def make_record(fetch_csv: str, write_csv: str, workload: str, steps: int, command: str) -> str:
    f = dispatch_counters(fetch_csv, "FETCH_SIZE")
    w = dispatch_counters(write_csv, "WRITE_SIZE")
    ff = calibration_factor(f, COPY_BYTES)
    wf = calibration_factor(w, COPY_BYTES)
    per = {}
    for disp, fac in ((f, ff), (w, wf)):
        for name, v in disp:
            lab = label_of(name)
            if lab is None:
                continue
            per.setdefault(lab, [0, 0.0, 0])
            per[lab][1] += v * 1024.0 * fac
    counts = {}
    for name, _ in f:
        lab = label_of(name)
        if lab is None:
            continue
        counts[lab] = counts.get(lab, 0) + 1
    lines = [f"# rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated against a plain 1 GiB device copy;",
             f"# every library kernel of the {workload} step (input generator and calibration copy excluded)"]
    for c in command.split(" ;; "):
        lines.append(f"# command: {c}")
    lines += [f"workload={workload}", f"source_sha={source_digest()}", f"steps={steps}",
              f"fetch_factor={ff:.4f}", f"write_factor={wf:.4f}"]
    total = 0.0
    for lab in sorted(per):
        launches = counts.get(lab, 0)
        if launches == 0:
            continue
        b = per[lab][1]
        total += b
        lines.append(f"label.{lab}={launches / steps:g} {b / launches:.0f}")
    lines.append(f"step_bytes={total / steps:.0f}")
    return "\n".join(lines) + "\n"


def read_record(path: str) -> dict:
    kv, labels = {}, {}
    with open(path) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=", 1)
            if k.startswith("label."):
                lp, bpl = v.split()
                labels[k[6:]] = (float(lp), float(bpl))
            else:
                kv[k] = v
    kv["labels"] = labels
    return kv


def find_record(workload: str, root: str = ROOT) -> dict | None:
    """The committed counter record of a workload, if it was taken from the
    current sources (else None)."""
    want = source_digest(root)
    for path in sorted(glob.glob(os.path.join(root, "profiles", "*_counters.txt"))):
        try:
            rec = read_record(path)
        except (OSError, ValueError):
            continue
        if rec.get("workload") == workload and rec.get("source_sha") == want:
            rec["path"] = os.path.relpath(path, root)
            return rec
    return None


def stats_markdown(stats_csv: str, title: str, command: str, note: str = "") -> str:
    rows = []
    for r in _rows(stats_csv):
        name = _col(r, "Name", "KERNEL_NAME", "Kernel_Name")
        calls = int(float(_col(r, "Calls")))
        avg = float(_col(r, "AverageNs", "Average_Ns", "Average")) / 1e3
        pct = float(_col(r, "Percentage", "Percent"))
        rows.append((name, calls, avg, pct))
    rows.sort(key=lambda t: -t[3])
    out = [f"# rocprofv3 kernel statistics: {title}", "", "Command (run from the repository root; committed files only):",
           "", "```"] + command.split(" ;; ") + ["```", ""]
    if note:
        out += [note, ""]
    out += ["| kernel | calls | average (us) | share of GPU time |", "|---|---|---|---|"]
    for name, calls, avg, pct in rows:
        out.append(f"| `{name}` | {calls} | {avg:.1f} | {pct:.2f}% |")
    return "\n".join(out) + "\n"


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = p.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("record")
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--workload", required=True)
    r.add_argument("--steps", type=int, required=True)
    r.add_argument("--command", required=True)
    r.add_argument("--out", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--out", required=True)
    a = p.parse_args(argv)
    if a.cmd == "record":
        text = make_record(a.fetch, a.write, a.workload, a.steps, a.command)
    else:
        text = stats_markdown(a.csv, a.title, a.command, a.note)
    with open(a.out, "w") as fh:
        fh.write(text)
    print(text)


if __name__ == "__main__":
    main()
