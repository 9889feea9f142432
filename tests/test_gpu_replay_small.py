"""GPU parity of the replay path at tile-boundary sizes.

Sides of at least LAPLEX_REPLAY_MIN anchors (default 2^20) move x into
sorted order and y back by replaying the radix passes' records, two
neighbouring 8192-element tiles per workgroup; shorter sides gather and
scatter through the permutation.  The threshold is read once per process,
so a child process with LAPLEX_REPLAY_MIN=0 runs the replay path at sizes
around whole pairs of tiles (a single tile, one ragged pair, one full pair,
a pair and a lone tile, several pairs), and this process checks its results against the
fp64 oracle ("LAPLEX: The FFT of Learnable Laplace Kernels", summary §2.2):
the permutation bit for bit, y = K x within tolerance, plan_create + apply
equal to plan_create_apply bit for bit (same scans on the same sorted x),
and the backward's dx and da (replayed back as two rows at once).
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

# (n, batch, phased)
CASES = [(1, 1, False), (5000, 2, True), (8193, 1, False), (16384, 2, False), (16385, 1, True), (24577, 3, False),
         (40000, 2, True)]


def inputs(n, batch, phased):
    rng = np.random.default_rng(7 * n + batch + 3 * phased)
    a = (rng.standard_normal(n) * 40).astype(np.float32)
    a[rng.integers(0, n, n // 9)] = a[rng.integers(0, n, n // 9)]  # ties
    phi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    psi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    x = rng.standard_normal((batch, n)).astype(np.float32)
    g = rng.standard_normal((batch, n)).astype(np.float32)
    return a, phi, psi, x, g


CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from laplace_matvec_amd import laplex as lx
from tests.test_gpu_replay_small import CASES, inputs
out = sys.argv[2]

def dev(v):
    return None if v is None else torch.as_tensor(np.ascontiguousarray(v, dtype=np.float32)).cuda()

def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()

lx.profile_enable(True)
for n, batch, phased in CASES:
    print(f"[replay child] n={n} batch={batch} phased={phased}", flush=True)
    lx.profile_reset()
    a, phi, psi, x, g = inputs(n, batch, phased)
    plan, y = lx.laplex_plan_create_apply(dev(a), dev(x), phi=dev(phi), psi=dev(psi))
    with plan:
        y_ca = host(y)
        grads = {k: host(v) for k, v in lx.laplex_backward(plan, None, dev(g)).items()}
    with lx.laplex_plan_create(dev(a), phi=dev(phi), psi=dev(psi)) as p2:
        perm = host(lx.laplex_plan_perm(p2))
        y_ap = host(lx.laplex_apply(p2, dev(x)))
    prof = lx.profile_read()
    launches = np.array([prof.get("replay_forward", (0, 0.0))[0], prof.get("replay_backward", (0, 0.0))[0]])
    np.savez(f"{out}/case_{n}_{batch}_{int(phased)}.npz", y_ca=y_ca, y_ap=y_ap, perm=perm, launches=launches,
             **{"g_" + k: v for k, v in grads.items()})
print("[replay child] done", flush=True)
"""


def test_replay_path_at_tile_pair_boundaries(gpu):
    with tempfile.TemporaryDirectory() as out:
        env = dict(os.environ, LAPLEX_REPLAY_MIN="0")
        print("[replay small] child process with LAPLEX_REPLAY_MIN=0", flush=True)
        r = subprocess.run([sys.executable, "-u", "-c", CHILD, ROOT, out], env=env, cwd=ROOT,
                           capture_output=True, text=True, timeout=240)
        print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
        assert r.returncode == 0, r.stderr[-2000:]
        for n, batch, phased in CASES:
            print(f"[replay small] check n={n} batch={batch} phased={phased}", flush=True)
            a, phi, psi, x, g = inputs(n, batch, phased)
            d = np.load(f"{out}/case_{n}_{batch}_{int(phased)}.npz")
            # the replay kernels ran: x and g forward, y, dx and da back
            assert d["launches"][0] > 0 and d["launches"][1] > 0, d["launches"]
            assert np.array_equal(d["perm"], oracle.argsort(a).astype(d["perm"].dtype))
            ref = oracle.apply_sweep(a, x, phi=phi, psi=psi)
            for v in range(batch):
                assert oracle.rel_l2(d["y_ca"][v], ref[v]) < TOL
            assert np.array_equal(d["y_ap"], d["y_ca"])
            # through y = K x: dx = K^T g, and da from the entrywise derivatives
            dx_ref = oracle.apply_sweep(a, g, phi=phi, psi=psi, transpose=True)
            for v in range(batch):
                assert oracle.rel_l2(d["g_dx"][v], dx_ref[v]) < TOL
            rows = np.arange(0, n, max(1, n // 300))
            if n == 1:  # one anchor: no other anchor pulls on it
                assert np.all(d["g_da"] == 0)
                continue
            gref = oracle.grad_dense(a, g, x, phi=phi, psi=psi, rows=rows)
            assert oracle.rel_l2(d["g_da"][rows], gref["da"]) < TOL
