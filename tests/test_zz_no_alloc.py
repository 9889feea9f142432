"""laplex_apply_noalloc through the C ABI: the same y as laplex_apply, bit for
bit, from the library's fixed per-GPU scratch array instead of any device
allocation; two calls in a row, the second with a smaller input (the array
keeps the first call's contents, which must not leak into the second);
requests beyond the array are refused."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from laplace_matvec_amd import laplex as lx

pytestmark = pytest.mark.gpu
TOL = 1e-5
SCRATCH = 64 << 20  # LAPLEX_NOALLOC_SCRATCH_BYTES


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def noalloc(plan, x, y, batch, transpose=0):
    torch.cuda.synchronize()
    st = lx.load().laplex_apply_noalloc(plan.handle, lx._ptr(x), lx._ptr(y), batch, transpose,
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return st


def both(plan, x, batch, n_out, transpose=0):
    y_ref = torch.empty((batch, n_out), device="cuda")
    assert lx.load().laplex_apply(plan.handle, lx._ptr(x), lx._ptr(y_ref), batch, transpose,
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) == lx.OK
    y = torch.full((batch, n_out), float("nan"), device="cuda")
    st = noalloc(plan, x, y, batch, transpose)
    assert st == lx.OK, lx.load().laplex_last_error()
    return y.cpu().numpy(), y_ref.cpu().numpy()


def check(y, y_ref, ref):
    assert np.array_equal(y, y_ref)
    for v in range(y.shape[0]):
        assert oracle.rel_l2(y[v], ref[v]) < TOL


def test_symmetric_long_then_short():
    rng = np.random.default_rng(1)
    n1, b1 = (1 << 20) + 77, 3  # replay path: sorted-order rows in the scratch
    a1 = (rng.standard_normal(n1) * 100).astype(np.float32)
    x1 = rng.standard_normal((b1, n1)).astype(np.float32)
    n2, b2 = 50001, 2           # gather path, a smaller input
    a2 = (rng.standard_normal(n2) * 10).astype(np.float32)
    x2 = rng.standard_normal((b2, n2)).astype(np.float32)
    with lx.laplex_plan_create(dev(a1)) as p1, lx.laplex_plan_create(dev(a2)) as p2:
        y, y_ref = both(p1, dev(x1), b1, n1)
        check(y, y_ref, oracle.apply_sweep(a1, x1))
        y, y_ref = both(p2, dev(x2), b2, n2)
        check(y, y_ref, oracle.apply_sweep(a2, x2))


def test_general_phased_long_then_short():
    rng = np.random.default_rng(2)
    n, k, B = 40000, 300000, 2  # y = K x merges; z = K^T w takes the evaluation path
    a = (rng.standard_normal(n) * 30).astype(np.float32)
    b = (rng.standard_normal(k) * 30).astype(np.float32)
    phi = rng.uniform(0, 6.3, n).astype(np.float32)
    psi = rng.uniform(0, 6.3, k).astype(np.float32)
    x = rng.standard_normal((B, k)).astype(np.float32)
    w = rng.standard_normal((1, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=dev(phi), psi=dev(psi)) as plan:
        y, y_ref = both(plan, dev(x), B, n, 0)
        check(y, y_ref, oracle.apply_sweep(a, x, b=b, phi=phi, psi=psi))
        z, z_ref = both(plan, dev(w), 1, k, 1)
        check(z, z_ref, oracle.apply_sweep(a, w, b=b, phi=phi, psi=psi, transpose=True))
    # a short output side: the LDS-binned bucketing, smaller again
    n2, k2 = 700, 9000
    a2 = (rng.standard_normal(n2) * 30).astype(np.float32)
    b2 = (rng.standard_normal(k2) * 30).astype(np.float32)
    x2 = rng.standard_normal((3, k2)).astype(np.float32)
    with lx.laplex_plan_create(dev(a2), b=dev(b2)) as plan:
        lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, lx.ALGO_BUCKET)
        y, y_ref = both(plan, dev(x2), 3, n2, 0)
        check(y, y_ref, oracle.apply_sweep(a2, x2, b=b2))


def test_request_beyond_scratch_is_refused():
    n, B = 1 << 22, 4  # two [4][2^22] float rows alone take 128 MiB
    a = dev(np.arange(n, dtype=np.float32))
    x = torch.zeros((B, n), device="cuda")
    y = torch.zeros((B, n), device="cuda")
    with lx.laplex_plan_create(a) as plan:
        st = noalloc(plan, x, y, B)
        assert st == lx.ERR_INVALID_ARGUMENT
        assert "scratch" in lx.load().laplex_last_error().decode()
        # one vector fits: it still works after the refusal
        xs = torch.from_numpy(np.random.default_rng(3).standard_normal(n).astype(np.float32)).cuda()
        y1 = torch.empty(n, device="cuda")
        assert noalloc(plan, xs, y1, 1) == lx.OK
        assert torch.equal(y1, lx.laplex_apply(plan, xs))


def test_invalid_arguments_checked_first():
    lib = lx.load()
    assert lib.laplex_apply_noalloc(None, None, None, 1, 0, None) == lx.ERR_INVALID_ARGUMENT
