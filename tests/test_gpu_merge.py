"""GPU parity of the merge-path bucketing (both anchor sets long): a general
plan's u, v come from merging the sorted inputs into the intervals of the
sorted outputs ("LAPLEX: The FFT of Learnable Laplace Kernels", summary
§2.2, general case), in float64 and a fixed order.  Compared with the fp64
oracle's general sweep over whole vectors, and repeated bit for bit."""
import sys

import numpy as np
import pytest
import torch

import oracle
from laplace_matvec_amd import laplex as lx

pytestmark = pytest.mark.gpu
TOL = 1e-5
TILE = 2048  # merged items per workgroup


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def max_rel(y, ref):
    y, ref = np.atleast_2d(y), np.atleast_2d(ref)
    return max(oracle.rel_l2(y[i], ref[i]) for i in range(y.shape[0]))


def run_both(a, b, x, w, phi=None, psi=None, t=None, algo=lx.ALGO_BUCKET):
    kw = {} if phi is None else dict(phi=dev(phi), psi=dev(psi))
    with lx.laplex_plan_create(dev(a), b=dev(b), **kw) as plan:
        lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, algo)
        if t is not None:
            lx.laplex_plan_set_temperature(plan, t)
        y = host(lx.laplex_apply(plan, dev(x)))
        z = host(lx.laplex_apply(plan, dev(w), transpose=True))
    return y, z


def check(a, b, x, w, phi=None, psi=None, t=1.0):
    y, z = run_both(a, b, x, w, phi, psi, None if t == 1.0 else t)
    ry = oracle.apply_sweep(a, x, b=b, phi=phi, psi=psi, t=t)
    rz = oracle.apply_sweep(a, w, b=b, phi=phi, psi=psi, transpose=True, t=t)
    ey, ez = max_rel(y, ry), max_rel(z, rz)
    say(f"  rel L2 y {ey:.2e} z {ez:.2e}")
    assert ey < TOL and ez < TOL
    return y, z


@pytest.mark.timeout(600)
@pytest.mark.parametrize("phased", [False, True])
def test_merge_both_sides_long(gpu, phased):
    """Both sides past 2^20 (n = 2^21 + 5 outputs of y = K x, k = 3 * 2^20 + 7
    inputs), ties between the sides, both directions through the bucketing."""
    n, k = (1 << 21) + 5, (3 << 20) + 7
    say(f"[merge] n={n} k={k} phased={phased}")
    rng = np.random.default_rng(11 + phased)
    a = (rng.standard_normal(n) * 300).astype(np.float32)
    b = rng.uniform(-1200, 1200, k).astype(np.float32)
    b[rng.integers(0, k, k // 50)] = a[rng.integers(0, n, k // 50)]  # inputs on top of outputs
    phi = rng.uniform(0, 6.3, n).astype(np.float32) if phased else None
    psi = rng.uniform(0, 6.3, k).astype(np.float32) if phased else None
    x = rng.standard_normal((2, k)).astype(np.float32)
    w = rng.standard_normal((2, n)).astype(np.float32)
    check(a, b, x, w, phi, psi)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n_out,n_in", [(1 << 20, 1 << 22), (4096, 1 << 24)])
def test_merge_long_input_side(gpu, n_out, n_in):
    """The input side much longer than the output side (many inputs per
    interval, runs spanning several workgroups)."""
    say(f"[merge] n_out={n_out} n_in={n_in}")
    rng = np.random.default_rng(n_out + n_in)
    a = (rng.standard_normal(n_out) * 100).astype(np.float32)
    b = (rng.standard_normal(n_in) * 100).astype(np.float32)
    x = rng.standard_normal((1, n_in)).astype(np.float32)
    w = rng.standard_normal((1, n_out)).astype(np.float32)
    y, _ = run_both(a, b, x, w)
    ry = oracle.apply_sweep(a, x, b=b)
    e = max_rel(y, ry)
    say(f"  rel L2 y {e:.2e}")
    assert e < TOL


@pytest.mark.parametrize("case", ["clustered", "all_below", "all_above", "ties", "ragged_tile", "one_output_gap"])
def test_merge_layouts(gpu, case):
    """Layouts that stress the segments: whole tiles of inputs with no output
    (runs carried across many workgroups), every input below or above every
    output, inputs equal to outputs, a merged length one past a tile
    multiple, and all inputs inside one interval."""
    rng = np.random.default_rng(["clustered", "all_below", "all_above", "ties", "ragged_tile",
                                 "one_output_gap"].index(case))
    n, k = 3001, 40000
    if case == "ragged_tile":
        n, k = 3001, 5 * TILE - 3001 + 1
    a = np.sort(rng.uniform(-50, 50, n)).astype(np.float32)
    if case == "clustered":
        b = np.concatenate([rng.normal(-20, 0.01, k // 2), rng.normal(30, 0.01, k - k // 2)]).astype(np.float32)
    elif case == "all_below":
        b = rng.uniform(-90, -60, k).astype(np.float32)
    elif case == "all_above":
        b = rng.uniform(60, 90, k).astype(np.float32)
    elif case == "ties":
        b = a[rng.integers(0, n, k)]
    elif case == "one_output_gap":
        a = np.concatenate([rng.uniform(-50, -10, n // 2), rng.uniform(10, 50, n - n // 2)]).astype(np.float32)
        b = rng.uniform(-9, 9, k).astype(np.float32)
    else:
        b = rng.uniform(-55, 55, k).astype(np.float32)
    a = rng.permutation(a)
    x = rng.standard_normal((3, k)).astype(np.float32)
    w = rng.standard_normal((3, n)).astype(np.float32)
    say(f"[merge layout] {case} n={n} k={k}")
    check(a, b, x, w)


def test_merge_temperature_and_vector_groups(gpu):
    """Temperature 0.3, phases, 11 vectors (groups of 6 and 5)."""
    rng = np.random.default_rng(99)
    n, k = 5003, 60001
    a = (rng.standard_normal(n) * 10).astype(np.float32)
    b = (rng.standard_normal(k) * 12).astype(np.float32)
    phi = rng.uniform(0, 6.3, n).astype(np.float32)
    psi = rng.uniform(0, 6.3, k).astype(np.float32)
    x = rng.standard_normal((11, k)).astype(np.float32)
    w = rng.standard_normal((11, n)).astype(np.float32)
    check(a, b, x, w, phi, psi, t=0.3)


def test_merge_zero_temperature_countsketch_bitwise(gpu):
    """t = 0 routes by equality: several inputs equal to one output sum
    exactly (integer-valued, so any order gives the same float)."""
    rng = np.random.default_rng(5)
    n, k = 2000, 30000
    a = (4.0 * rng.permutation(n)).astype(np.float32)
    b = a[rng.integers(0, n, k)]
    b[:100] = 1e6  # above every output: routed nowhere
    x = rng.integers(-8, 9, (2, k)).astype(np.float32)
    w = rng.integers(-8, 9, (2, n)).astype(np.float32)
    y, z = run_both(a, b, x, w, t=0.0)
    ry = oracle.apply_sweep(a, x, b=b, t=0.0)
    rz = oracle.apply_sweep(a, w, b=b, transpose=True, t=0.0)
    assert np.array_equal(y, ry.astype(np.float32))
    assert np.array_equal(z, rz.astype(np.float32))


def test_merge_repeat_bitwise(gpu):
    """The same call three times gives the same bits (no atomics; the
    summation order follows the sizes alone)."""
    rng = np.random.default_rng(8)
    n, k = 50000, 400000
    a = (rng.standard_normal(n) * 30).astype(np.float32)
    b = (rng.standard_normal(k) * 30).astype(np.float32)
    x = dev(rng.standard_normal((4, k)))
    with lx.laplex_plan_create(dev(a), b=dev(b)) as plan:
        lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, lx.ALGO_BUCKET)
        outs = [host(lx.laplex_apply(plan, x)) for _ in range(3)]
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    ref = oracle.apply_sweep(a, host(x), b=b)
    assert max_rel(outs[0], ref) < TOL
