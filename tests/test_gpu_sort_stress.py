"""Stress of the radix passes' decoupled look-back, on the GPU.

liblaplex_stress.so is the operator library built with 4096-key sort tiles
(256 threads) and a look-back that reads one predecessor per round, so a
side has twice the tiles of the default build and every tile walks its
predecessors one at a time: the longest chains of waits on unpublished
counts the design allows.  One child process loads that library (and not
the default one) and sorts and applies at several sizes on the replay path,
with x travelling through the key-value passes; this process checks against
the fp64 oracle ("LAPLEX: The FFT of Learnable Laplace Kernels", summary
§2.2): the permutation bit for bit against the oracle's stable argsort, y
within tolerance, and plan_create + apply bit-equal to plan_create_apply.
"""
import os
import subprocess
import sys
import tempfile

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu
TOL = 1e-5
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRESS_LIB = os.path.join(ROOT, "laplace_matvec_amd", "liblaplex_stress.so")

# (kind, n, batch, phased): n >= 2^20 takes the replay path
CASES = [("normal", (1 << 20) + 77, 1, False), ("ties", 3 * (1 << 20) + 12345, 2, True),
         ("few_values", (1 << 21) + 3, 1, False), ("normal", (1 << 22) + 5, 1, False)]


def inputs(kind, n, batch, phased):
    rng = np.random.default_rng(n + 11 * batch)
    if kind == "few_values":  # four distinct anchors: three digits of every key equal
        a = rng.choice(np.array([-3.5, 0.25, 0.25000003, 7.0], dtype=np.float32), n)
    else:
        a = (rng.standard_normal(n) * 50).astype(np.float32)
        if kind == "ties":
            a[rng.integers(0, n, n // 7)] = a[rng.integers(0, n, n // 7)]
    phi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    psi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    x = rng.standard_normal((batch, n)).astype(np.float32)
    return a.astype(np.float32), phi, psi, x


CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from laplace_matvec_amd import laplex as lx
from tests.test_gpu_sort_stress import CASES, STRESS_LIB, inputs
lx.LIB_PATH = STRESS_LIB
lx._lib = None
out = sys.argv[2]

def dev(v):
    return None if v is None else torch.as_tensor(np.ascontiguousarray(v, dtype=np.float32)).cuda()

def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()

for kind, n, batch, phased in CASES:
    print(f"[sort stress child] {kind} n={n} batch={batch} phased={phased}", flush=True)
    a, phi, psi, x = inputs(kind, n, batch, phased)
    plan, y = lx.laplex_plan_create_apply(dev(a), dev(x), phi=dev(phi), psi=dev(psi))
    with plan:
        perm_ca = host(lx.laplex_plan_perm(plan))
        y_ca = host(y)
    with lx.laplex_plan_create(dev(a), phi=dev(phi), psi=dev(psi)) as p2:
        perm = host(lx.laplex_plan_perm(p2))
        y_ap = host(lx.laplex_apply(p2, dev(x)))
    np.savez(f"{out}/case_{kind}_{n}.npz", y_ca=y_ca, y_ap=y_ap, perm=perm, perm_ca=perm_ca)
maps = open("/proc/self/maps").read()
print("[sort stress child] stress library mapped:", "liblaplex_stress.so" in maps,
      "default library mapped:", "/liblaplex.so" in maps, flush=True)
assert "liblaplex_stress.so" in maps and "/liblaplex.so" not in maps
print("[sort stress child] done", flush=True)
"""


def test_lookback_stress_small_tiles_one_predecessor_per_round(gpu):
    if not os.path.exists(STRESS_LIB):
        pytest.fail(f"{STRESS_LIB} is missing: build the package first")
    with tempfile.TemporaryDirectory() as out:
        print("[sort stress] child process on liblaplex_stress.so", flush=True)
        r = subprocess.run([sys.executable, "-u", "-c", CHILD, ROOT, out], cwd=ROOT, capture_output=True,
                           text=True, timeout=300)
        print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
        assert r.returncode == 0, r.stderr[-2000:]
        for kind, n, batch, phased in CASES:
            print(f"[sort stress] check {kind} n={n} batch={batch} phased={phased}", flush=True)
            a, phi, psi, x = inputs(kind, n, batch, phased)
            d = np.load(f"{out}/case_{kind}_{n}.npz")
            want = oracle.argsort(a).astype(d["perm"].dtype)
            assert np.array_equal(d["perm"], want)
            assert np.array_equal(d["perm_ca"], want)
            ref = oracle.apply_sweep(a, x, phi=phi, psi=psi)
            for v in range(batch):
                assert oracle.rel_l2(d["y_ca"][v], ref[v]) < TOL
            assert np.array_equal(d["y_ap"], d["y_ca"])
