"""GPU parity of laplex_plan_create_apply (a symmetric plan and y = K x at
once, the rows of x sorted along with the anchors): bit for bit equal to
plan_create followed by apply, and within tolerance of the fp64 oracle
("LAPLEX: The FFT of Learnable Laplace Kernels", summary §2.2)."""
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
    assert np.array_equal(y, y_ref)
    assert np.array_equal(y, y_again)
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
