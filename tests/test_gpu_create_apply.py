"""GPU parity of laplex_plan_create_apply (a symmetric plan and y = K x at
once, the rows of x sorted along with the anchors): within tolerance of the
fp64 oracle ("LAPLEX: The FFT of Learnable Laplace Kernels", summary §2.2)
and equal to plan_create followed by apply -- bit for bit where both take
the same scans; to 1e-6 for plans of at most 8192 anchors, whose product is
computed inside the one-workgroup plan kernel (another summation order)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from laplace_matvec_amd import laplex as lx

pytestmark = pytest.mark.gpu
TOL = 1e-5


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


@pytest.mark.parametrize("n,batch,phased", [
    (5000, 2, False),              # short: plan_create + apply inside
    ((1 << 20) + 77, 1, False),    # rows travel with the sort
    ((1 << 20) + 77, 3, True),
    ((3 << 20) + 5, 18, True),     # 18 + 2 phase rows: the most that travel
    ((1 << 20) + 9, 19, True),     # one row too many: plan_create + apply inside
])
def test_create_apply_matches_create_then_apply(gpu, n, batch, phased):
    print(f"[create_apply] n={n} batch={batch} phased={phased}", flush=True)
    rng = np.random.default_rng(n + batch)
    a = (rng.standard_normal(n) * 50).astype(np.float32)
    a[rng.integers(0, n, n // 9)] = a[rng.integers(0, n, n // 9)]
    phi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    psi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    x = rng.standard_normal((batch, n)).astype(np.float32)
    A, X = dev(a), dev(x)
    P = None if phi is None else dev(phi)
    Q = None if psi is None else dev(psi)
    plan, y = lx.laplex_plan_create_apply(A, X, phi=P, psi=Q)
    with plan:
        y = host(y)
        y_again = host(lx.laplex_apply(plan, X))
        perm = host(lx.laplex_plan_perm(plan))
    with lx.laplex_plan_create(A, phi=P, psi=Q) as plan2:
        y_ref = host(lx.laplex_apply(plan2, X))
    if n <= 8192 and batch <= 8:
        for v in range(batch):
            assert oracle.rel_l2(y[v], y_ref[v].astype(np.float64)) < 1e-6
    else:
        assert np.array_equal(y, y_ref)
    assert np.array_equal(y_again, y_ref)
    assert np.array_equal(perm, oracle.argsort(a).astype(np.int64))
    ref = oracle.apply_sweep(a, x[:2], phi=phi, psi=psi)
    for v in range(min(batch, 2)):
        assert oracle.rel_l2(y[v], ref[v]) < TOL


def test_create_apply_rejects_nonfinite(gpu):
    n = (1 << 20) + 3
    a = np.zeros(n, np.float32)
    a[12345] = np.nan
    with pytest.raises(lx.LaplexError) as e:
        lx.laplex_plan_create_apply(dev(a), dev(np.ones(n)))
    assert e.value.status == lx.ERR_NONFINITE_ANCHOR
    phi = np.zeros(n, np.float32)
    phi[7] = np.inf
    with pytest.raises(lx.LaplexError) as e:
        lx.laplex_plan_create_apply(dev(np.arange(n)), dev(np.ones(n)), phi=dev(phi), psi=dev(np.zeros(n)))
    assert e.value.status == lx.ERR_NONFINITE_ANCHOR


@pytest.mark.parametrize("n,batch,phased", [(3000, 2, True), ((1 << 20) + 77, 2, False), ((1 << 20) + 77, 1, True)])
def test_backward_with_kept_input(gpu, n, batch, phased):
    # plan_create_apply keeps x: backward(x=None) equals backward(x) bit for bit
    print(f"[kept x backward] n={n} batch={batch} phased={phased}", flush=True)
    rng = np.random.default_rng(n + 3 * batch)
    a = (rng.standard_normal(n) * 30).astype(np.float32)
    a[rng.integers(0, n, n // 9)] = a[rng.integers(0, n, n // 9)]
    phi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    psi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    x = rng.standard_normal((batch, n)).astype(np.float32)
    g = rng.standard_normal((batch, n)).astype(np.float32)
    P = None if phi is None else dev(phi)
    Q = None if psi is None else dev(psi)
    plan, _ = lx.laplex_plan_create_apply(dev(a), dev(x), phi=P, psi=Q)
    with plan:
        kept = {k: host(v) for k, v in lx.laplex_backward(plan, None, dev(g)).items()}
        given = {k: host(v) for k, v in lx.laplex_backward(plan, dev(x), dev(g)).items()}
        with pytest.raises(lx.LaplexError) as e:
            lx.laplex_backward(plan, None, dev(g), transpose=True)
        assert e.value.status == lx.ERR_INVALID_ARGUMENT
    assert set(kept) == set(given)
    for k in kept:
        assert np.array_equal(kept[k], given[k]), k
    ref = oracle.grad_dense(a, g, x, phi=phi, psi=psi, rows=np.arange(0, n, max(1, n // 300)))
    assert oracle.rel_l2(kept["da"][::max(1, n // 300)], ref["da"]) < TOL
    with lx.laplex_plan_create(dev(a)) as p2:
        with pytest.raises(lx.LaplexError) as e:
            lx.laplex_backward(p2, None, dev(g))
        assert e.value.status == lx.ERR_INVALID_ARGUMENT


def _anchors(kind, n, rng):
    if kind == "one_bin":  # every key in one top-digit bin: the last radix pass keeps tiles whole
        return (1.0 + rng.random(n)).astype(np.float32)
    if kind == "wide":  # signs and exponents spread over many top-digit bins
        return (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 6, n)).astype(np.float32)
    if kind == "ties":  # few distinct values: long equal runs, decay 1
        a = rng.integers(-40, 40, n).astype(np.float32) * 0.25
        a[rng.integers(0, n, 64)] = -0.0
        return a
    if kind == "equal":
        return np.full(n, 3.5, np.float32)
    if kind == "gaps":  # far apart clusters: decays underflow between them
        return (rng.integers(0, 8, n) * 2000.0 + rng.random(n)).astype(np.float32)
    return (rng.standard_normal(n) * 1e4).astype(np.float32)


@pytest.mark.parametrize("kind,n", [
    ("normal", (1 << 20) + 1), ("normal", (3 << 20) + 12345), ("one_bin", (1 << 20) + 8191),
    ("wide", (2 << 20) + 4097), ("ties", (1 << 20) + 77), ("equal", 1 << 20), ("gaps", (1 << 21) + 3),
])
def test_create_apply_anchor_layouts(gpu, kind, n):
    # one row at n >= 2^20 (x travels through the radix passes) for anchor
    # layouts that stress the sort's bins and the scans' decays, against the
    # fp64 sweep of the oracle
    print(f"[create_apply layouts] kind={kind} n={n}", flush=True)
    rng = np.random.default_rng(n)
    a = _anchors(kind, n, rng)
    x = rng.standard_normal((1, n)).astype(np.float32)
    plan, y = lx.laplex_plan_create_apply(dev(a), dev(x))
    with plan:
        y = host(y)
        y_again = host(lx.laplex_apply(plan, dev(x)))
    ref = oracle.apply_sweep(a, x)
    assert oracle.rel_l2(y[0], ref[0]) < TOL
    assert oracle.rel_l2(y_again[0], ref[0]) < TOL
    # deterministic: a second plan gives the same bits
    plan2, y2 = lx.laplex_plan_create_apply(dev(a), dev(x))
    with plan2:
        assert np.array_equal(host(y2), y)


@pytest.mark.parametrize("n", [1, 2, 3, 63, 64, 65, 511, 512, 1000, 4096, 8191, 8192, 8193])
@pytest.mark.parametrize("phased", [False, True])
@pytest.mark.parametrize("batch", [1, 3, 9])
def test_create_apply_small_plans(gpu, n, phased, batch):
    # n <= 8192: sort, permutation, phase factors and y in one workgroup
    # (batch 9 and n = 8193 take the multi-launch path); ties and -0.0 included
    print(f"[create_apply small] n={n} phased={phased} batch={batch}", flush=True)
    rng = np.random.default_rng(3 * n + batch + 7 * phased)
    a = (rng.standard_normal(n) * 5).astype(np.float32)
    if n > 4:
        a[rng.integers(0, n, n // 4)] = a[rng.integers(0, n, n // 4)]
        a[rng.integers(0, n, 2)] = -0.0
        a[rng.integers(0, n, 2)] = 0.0
    phi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    psi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    x = rng.standard_normal((batch, n)).astype(np.float32)
    P = None if phi is None else dev(phi)
    Q = None if psi is None else dev(psi)
    plan, y = lx.laplex_plan_create_apply(dev(a), dev(x), phi=P, psi=Q)
    with plan:
        y = host(y)
        perm = host(lx.laplex_plan_perm(plan))
        srt = host(lx.laplex_plan_sorted(plan))
        kept = {k: host(v) for k, v in lx.laplex_backward(plan, None, dev(x)).items()}
        given = {k: host(v) for k, v in lx.laplex_backward(plan, dev(x), dev(x)).items()}
    order = oracle.argsort(a)
    assert np.array_equal(perm, order.astype(np.int64))
    assert np.array_equal(srt.view(np.uint32), a[order].view(np.uint32))
    ref = oracle.apply_sweep(a, x, phi=phi, psi=psi)
    for v in range(batch):
        assert oracle.rel_l2(y[v], ref[v]) < TOL
    for k in kept:
        assert np.array_equal(kept[k], given[k]), k


def test_create_apply_small_rejects_nonfinite(gpu):
    a = np.linspace(-1, 1, 3000).astype(np.float32)
    a[17] = np.inf
    with pytest.raises(lx.LaplexError) as e:
        lx.laplex_plan_create_apply(dev(a), dev(np.ones(3000)))
    assert e.value.status == lx.ERR_NONFINITE_ANCHOR
    with pytest.raises(lx.LaplexError) as e:
        lx.laplex_plan_create(dev(a))
    assert e.value.status == lx.ERR_NONFINITE_ANCHOR
    phi = np.zeros(3000, np.float32)
    phi[5] = np.nan
    with pytest.raises(lx.LaplexError) as e:
        lx.laplex_plan_create_apply(dev(np.arange(3000)), dev(np.ones(3000)), phi=dev(phi),
                                    psi=dev(np.zeros(3000)))
    assert e.value.status == lx.ERR_NONFINITE_ANCHOR
