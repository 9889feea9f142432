"""GPU parity of the temperature argument and of the backward pass, through
the C ABI, against the fp64 oracle on the same seeded inputs.

Temperature: entries exp(-|a - b| / t), t = 0 the equality-routing limit
("LAPLEX: The FFT of Learnable Laplace Kernels", summary §2.1 and §2.3).
Backward: gradients of a step through y = K x or y = K^T x with respect to
x, the anchors and the phases (summary §2.1: trainable anchors), from the
oracle's entrywise derivatives of the definition (sgn(0) = 0 at ties).

Tolerance: relative L2 1e-5 per output vector, as for the forward product;
the anchor and phase gradients are sums of the same float64-scanned products
rounded once to float32 and accumulated over the batch in float32.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

import oracle
from laplace_matvec_amd import laplex as lx

pytestmark = pytest.mark.gpu

TOL = 1e-5
RNG = np.random.default_rng(77001)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().astype(np.float64)


def tied(n, scale, rng):
    a = (rng.standard_normal(n) * scale).astype(np.float32)
    m = n // 7
    if m:
        a[rng.integers(0, n, m)] = a[rng.integers(0, n, m)]
    return a


def phases(m, rng):
    return rng.uniform(-np.pi, np.pi, m).astype(np.float32)


# ---------------------------------------------------------------- temperature

@pytest.mark.parametrize("n", [5000, (1 << 20) + 77])
@pytest.mark.parametrize("t", [0.25, 3.0])
@pytest.mark.parametrize("phased", [False, True])
def test_temperature_symmetric(gpu, n, t, phased):
    say(f"[temperature sym] n={n} t={t} phased={phased}")
    rng = np.random.default_rng(n + int(8 * t))
    a = tied(n, 10.0, rng)
    phi = phases(n, rng) if phased else None
    psi = phases(n, rng) if phased else None
    x = rng.standard_normal((2, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        lx.laplex_plan_set_temperature(plan, t)
        for tr in (False, True):
            y = host(lx.laplex_apply(plan, dev(x), transpose=tr))
            ref = oracle.apply_sweep(a, x, phi=phi, psi=psi, transpose=tr, t=t)
            for v in range(2):
                assert oracle.rel_l2(y[v], ref[v]) < TOL


@pytest.mark.parametrize("n,k", [(300, 5000), (5000, 300), (20000, 1024)])
@pytest.mark.parametrize("algo", [lx.ALGO_BUCKET, lx.ALGO_EVALUATE])
@pytest.mark.parametrize("phased", [False, True])
def test_temperature_general(gpu, n, k, algo, phased):
    say(f"[temperature general] n={n} k={k} algo={algo} phased={phased}")
    rng = np.random.default_rng(n * 3 + k + algo)
    a = tied(n, 20.0, rng)
    b = tied(k, 20.0, rng)
    b[: min(n, k) // 5] = a[: min(n, k) // 5]
    phi = phases(n, rng) if phased else None
    psi = phases(k, rng) if phased else None
    x = rng.standard_normal((3, k)).astype(np.float32)
    w = rng.standard_normal((3, n)).astype(np.float32)
    t = 0.5
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, algo)
        lx.laplex_plan_set_temperature(plan, t)
        y = host(lx.laplex_apply(plan, dev(x)))
        z = host(lx.laplex_apply(plan, dev(w), transpose=True))
    ry = oracle.apply_sweep(a, x, b=b, phi=phi, psi=psi, t=t)
    rz = oracle.apply_sweep(a, w, b=b, phi=phi, psi=psi, transpose=True, t=t)
    for v in range(3):
        assert oracle.rel_l2(y[v], ry[v]) < TOL
        assert oracle.rel_l2(z[v], rz[v]) < TOL


@pytest.mark.parametrize("algo", [lx.ALGO_AUTO, lx.ALGO_BUCKET, lx.ALGO_EVALUATE])
def test_zero_temperature_routing_close_anchors(gpu, algo):
    # distinct anchors 1e-4 apart: at t = 1 a dense matrix, at t = 0 a routing
    n = 4000
    a = np.unique((np.arange(n) * 1e-4).astype(np.float32))
    n = a.size
    sigma = RNG.permutation(n)
    b = a[sigma]                                    # permutation routing: exact
    x = RNG.standard_normal((2, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b)) as plan:
        lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, algo)
        lx.laplex_plan_set_temperature(plan, 0.0)
        y = host(lx.laplex_apply(plan, dev(x)))
        z = host(lx.laplex_apply(plan, dev(x), transpose=True))
    inv = np.argsort(sigma)
    assert np.array_equal(y, x[:, inv].astype(np.float64))
    assert np.array_equal(z, x[:, sigma].astype(np.float64))
    # symmetric at t = 0: the identity, bitwise (random and replay paths)
    for m in (n, (1 << 20) + 3):
        s = np.unique(RNG.uniform(0, 1, m).astype(np.float32))
        xs = RNG.standard_normal(s.size).astype(np.float32)
        with lx.laplex_plan_create(dev(RNG.permutation(s))) as plan:
            lx.laplex_plan_set_temperature(plan, 0.0)
            ys = host(lx.laplex_apply(plan, dev(xs)))
        assert np.array_equal(ys, xs.astype(np.float64))


def test_zero_temperature_countsketch_and_phases(gpu):
    n, k = 500, 6000
    a = np.unique(RNG.uniform(0, 0.5, n).astype(np.float32))
    n = a.size
    b = a[RNG.integers(0, n, k)]
    b[:300] = RNG.uniform(0.6, 0.7, 300).astype(np.float32)  # no partner
    phi, psi = phases(n, RNG), phases(k, RNG)
    x = RNG.standard_normal((2, k)).astype(np.float32)
    w = RNG.standard_normal((2, n)).astype(np.float32)
    for algo in (lx.ALGO_BUCKET, lx.ALGO_EVALUATE):
        with lx.laplex_plan_create(dev(a), b=dev(b), phi=dev(phi), psi=dev(psi)) as plan:
            lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, algo)
            lx.laplex_plan_set_temperature(plan, 0.0)
            y = host(lx.laplex_apply(plan, dev(x)))
            z = host(lx.laplex_apply(plan, dev(w), transpose=True))
        ry = oracle.apply_dense(a, x, b=b, phi=phi, psi=psi, t=0.0)
        rz = oracle.apply_dense(a, w, b=b, phi=phi, psi=psi, transpose=True, t=0.0)
        for v in range(2):
            assert oracle.rel_l2(y[v], ry[v]) < TOL
            assert oracle.rel_l2(z[v], rz[v]) < TOL


@pytest.mark.parametrize("t", [0.5, 0.0])
@pytest.mark.parametrize("phased", [False, True])
def test_temperature_gram(gpu, t, phased):
    n, k = 400, 30000
    rng = np.random.default_rng(31 + int(phased))
    a = (rng.standard_normal(n) * 20).astype(np.float32)
    b = (rng.standard_normal(k) * 20).astype(np.float32)
    b[:200] = a[rng.integers(0, n, 200)]
    phi = phases(n, rng) if phased else None
    psi = phases(k, rng) if phased else None
    D = rng.uniform(0, 1, k).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        lx.laplex_plan_set_temperature(plan, t)
        M = host(lx.laplex_gram(plan, dev(D)))
    ref = oracle.gram_direct(a, b, D, phi=phi, psi=psi, t=t)
    assert oracle.rel_l2(M, ref) < TOL


def test_temperature_rejects_invalid(gpu):
    with lx.laplex_plan_create(dev(np.arange(10))) as plan:
        for bad in (-1.0, float("nan"), float("inf"), 1e-40):
            with pytest.raises(lx.LaplexError) as e:
                lx.laplex_plan_set_temperature(plan, bad)
            assert e.value.status == lx.ERR_INVALID_ARGUMENT


# ------------------------------------------------------------------- backward

def check_grads(got, ref, keys, tol=TOL):
    for key in keys:
        err = oracle.rel_l2(got[key], ref[key])
        assert err < tol, f"{key}: rel L2 {err:.3e}"


@pytest.mark.parametrize("n", [1, 2, 3, 1000, 9001])
@pytest.mark.parametrize("phased", [False, True])
@pytest.mark.parametrize("transpose", [False, True])
def test_backward_symmetric(gpu, n, phased, transpose):
    say(f"[backward sym] n={n} phased={phased} transpose={transpose}")
    rng = np.random.default_rng(7 * n + 2 * phased + transpose)
    a = tied(n, 5.0, rng)
    phi = phases(n, rng) if phased else None
    psi = phases(n, rng) if phased else None
    B = 3
    x = rng.standard_normal((B, n)).astype(np.float32)
    g = rng.standard_normal((B, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        out = lx.laplex_backward(plan, dev(x), dev(g), transpose=transpose)
        got = {k: host(v) for k, v in out.items()}
    u, w = (x, g) if transpose else (g, x)
    ref = oracle.grad_dense(a, u, w, phi=phi, psi=psi)
    ref["dx"] = oracle.apply_sweep(a, g, phi=phi, psi=psi, transpose=not transpose)
    keys = ["dx", "da"] + (["dphi", "dpsi"] if phased else [])
    assert set(got) == set(keys)
    if n == 1:
        assert np.array_equal(got["da"], [0.0])  # no other anchor to pull on it
    for v in range(B):
        assert oracle.rel_l2(got["dx"][v], ref["dx"][v]) < TOL
    check_grads(got, ref, [k for k in keys if k != "dx"])


@pytest.mark.parametrize("phased", [False, True])
def test_backward_symmetric_replay_path(gpu, phased):
    # n above the replay threshold: gathers and scatters through the radix records
    n = (1 << 20) + 4099
    say(f"[backward sym replay] n={n} phased={phased}")
    rng = np.random.default_rng(4242 + phased)
    a = tied(n, 300.0, rng)
    phi = phases(n, rng) if phased else None
    psi = phases(n, rng) if phased else None
    x = rng.standard_normal((2, n)).astype(np.float32)
    g = rng.standard_normal((2, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        out = lx.laplex_backward(plan, dev(x), dev(g))
        got = {k: host(v) for k, v in out.items()}
    ref_dx = oracle.apply_sweep(a, g, phi=phi, psi=psi, transpose=True)
    for v in range(2):
        assert oracle.rel_l2(got["dx"][v], ref_dx[v]) < TOL
    rows = np.sort(rng.choice(n, 400, replace=False))
    ref = oracle.grad_dense(a, g, x, phi=phi, psi=psi, rows=rows)
    for key in ["da"] + (["dphi", "dpsi"] if phased else []):
        err = oracle.rel_l2(got[key][rows], ref[key])
        assert err < TOL, f"{key}: rel L2 {err:.3e}"


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (300, 5000), (5000, 300), (20000, 1024)])
@pytest.mark.parametrize("phased", [False, True])
@pytest.mark.parametrize("transpose", [False, True])
def test_backward_general(gpu, n, k, phased, transpose):
    say(f"[backward general] n={n} k={k} phased={phased} transpose={transpose}")
    rng = np.random.default_rng(n + 5 * k + 2 * phased + transpose)
    a = tied(n, 20.0, rng)
    b = tied(k, 20.0, rng)
    m = min(n, k) // 5
    b[:m] = a[rng.integers(0, n, m)]
    phi = phases(n, rng) if phased else None
    psi = phases(k, rng) if phased else None
    B = 4
    n_in, n_out = (n, k) if transpose else (k, n)
    x = rng.standard_normal((B, n_in)).astype(np.float32)
    g = rng.standard_normal((B, n_out)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        out = lx.laplex_backward(plan, dev(x), dev(g), transpose=transpose)
        got = {key: host(v) for key, v in out.items()}
    u, w = (x, g) if transpose else (g, x)
    ref = oracle.grad_dense(a, u, w, b=b, phi=phi, psi=psi)
    ref_dx = oracle.apply_sweep(a, g, b=b, phi=phi, psi=psi, transpose=not transpose)
    for v in range(B):
        assert oracle.rel_l2(got["dx"][v], ref_dx[v]) < TOL
    check_grads(got, ref, ["da", "db"] + (["dphi", "dpsi"] if phased else []))


@pytest.mark.parametrize("phased", [False, True])
def test_backward_general_vector_groups(gpu, phased):
    """19 vectors: the evaluation runs them in groups (7, 7, 5) and sums the
    anchor and phase gradients over the groups; ragged output count, ties
    within and between the sides."""
    n, k, B = 20011, 700, 19
    say(f"[backward general groups] n={n} k={k} B={B} phased={phased}")
    rng = np.random.default_rng(1919 + phased)
    a = tied(n, 20.0, rng)
    b = tied(k, 20.0, rng)
    b[:100] = a[rng.integers(0, n, 100)]
    phi = phases(n, rng) if phased else None
    psi = phases(k, rng) if phased else None
    x = rng.standard_normal((B, k)).astype(np.float32)
    g = rng.standard_normal((B, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        out = lx.laplex_backward(plan, dev(x), dev(g))
        got = {key: host(v) for key, v in out.items()}
    ref = oracle.grad_dense(a, g, x, b=b, phi=phi, psi=psi)
    ref_dx = oracle.apply_sweep(a, g, b=b, phi=phi, psi=psi, transpose=True)
    for v in range(B):
        assert oracle.rel_l2(got["dx"][v], ref_dx[v]) < TOL
    check_grads(got, ref, ["da", "db"] + (["dphi", "dpsi"] if phased else []))


@pytest.mark.parametrize("t", [0.5, 0.0])
def test_backward_temperature(gpu, t):
    n, k = 3000, 800
    rng = np.random.default_rng(99)
    a = np.unique(rng.uniform(0, 30, n).astype(np.float32))
    n = a.size
    b = a[rng.integers(0, n, k)]
    b[:100] = rng.uniform(0, 30, 100).astype(np.float32)
    phi, psi = phases(n, rng), phases(k, rng)
    x = rng.standard_normal((2, k)).astype(np.float32)
    g = rng.standard_normal((2, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=dev(phi), psi=dev(psi)) as plan:
        lx.laplex_plan_set_temperature(plan, t)
        got = {key: host(v) for key, v in lx.laplex_backward(plan, dev(x), dev(g)).items()}
    ref = oracle.grad_dense(a, g, x, b=b, phi=phi, psi=psi, t=t)
    if t == 0.0:
        assert not got["da"].any() and not got["db"].any()
        check_grads(got, ref, ["dphi", "dpsi"])
    else:
        check_grads(got, ref, ["da", "db", "dphi", "dpsi"])
    # symmetric plan at the same temperature
    xs = rng.standard_normal((2, n)).astype(np.float32)
    gs = rng.standard_normal((2, n)).astype(np.float32)
    psi_s = phases(n, rng)
    with lx.laplex_plan_create(dev(a), phi=dev(phi), psi=dev(psi_s)) as plan:
        lx.laplex_plan_set_temperature(plan, t)
        got = {key: host(v) for key, v in lx.laplex_backward(plan, dev(xs), dev(gs)).items()}
    ref = oracle.grad_dense(a, gs, xs, phi=phi, psi=psi_s, t=t)
    if t == 0.0:
        assert not got["da"].any()
        check_grads(got, ref, ["dphi", "dpsi"])
    else:
        check_grads(got, ref, ["da", "dphi", "dpsi"])


def test_backward_subset_of_outputs_and_errors(gpu):
    n = 2000
    rng = np.random.default_rng(5)
    a = tied(n, 4.0, rng)
    x = rng.standard_normal(n).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    with lx.laplex_plan_create(dev(a)) as plan:
        only_da = lx.laplex_backward(plan, dev(x), dev(g), want=("da",))
        assert set(only_da) == {"da"}
        ref = oracle.grad_dense(a, g, x)
        assert oracle.rel_l2(host(only_da["da"]), ref["da"]) < TOL
        lib = lx.load()
        X, G, D = dev(x), dev(g), torch.empty(n, device="cuda")
        vp = ctypes.c_void_p
        h = plan.handle
        # db on a symmetric plan, phase gradients of an unphased plan, overlaps
        assert lib.laplex_backward(h, vp(X.data_ptr()), vp(G.data_ptr()), 1, 0, None, None,
                                   vp(D.data_ptr()), None, None, None) == lx.ERR_INVALID_ARGUMENT
        assert lib.laplex_backward(h, vp(X.data_ptr()), vp(G.data_ptr()), 1, 0, None, None, None,
                                   vp(D.data_ptr()), None, None) == lx.ERR_INVALID_ARGUMENT
        assert lib.laplex_backward(h, vp(X.data_ptr()), vp(G.data_ptr()), 1, 0, vp(X.data_ptr()), None,
                                   None, None, None, None) == lx.ERR_INVALID_ARGUMENT
        assert lib.laplex_backward(h, vp(X.data_ptr()), vp(G.data_ptr()), 1, 0, vp(D.data_ptr()),
                                   vp(D.data_ptr()), None, None, None, None) == lx.ERR_INVALID_ARGUMENT
        assert lib.laplex_backward(h, vp(X.data_ptr()), vp(G.data_ptr()), 1, 2, vp(D.data_ptr()), None,
                                   None, None, None, None) == lx.ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("phased", [False, True])
def test_backward_general_small_output_side_large(gpu, phased):
    # y = K x with a small column side (k <= 1024) and a large row side: the
    # gradients on b come from the rows bucketed into b's intervals; checked
    # on sampled outputs against the dense definition
    n, k, B = (1 << 21) + 5, 1000, 2
    say(f"[backward general large] n={n} k={k} phased={phased}")
    rng = np.random.default_rng(77 + phased)
    a = (rng.standard_normal(n) * 30).astype(np.float32)
    b = rng.uniform(-60, 60, k).astype(np.float32)
    b[:50] = a[rng.integers(0, n, 50)]  # ties between the sides
    b[50:60] = b[60]                    # ties within b
    phi = phases(n, rng) if phased else None
    psi = phases(k, rng) if phased else None
    x = rng.standard_normal((B, k)).astype(np.float32)
    g = rng.standard_normal((B, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        got = {key: host(v) for key, v in lx.laplex_backward(plan, dev(x), dev(g)).items()}
    ref_dx = oracle.apply_sweep(a, g, b=b, phi=phi, psi=psi, transpose=True)
    for v in range(B):
        assert oracle.rel_l2(got["dx"][v], ref_dx[v]) < TOL
    cols = np.concatenate([np.arange(0, 70), rng.integers(0, k, 30)])
    rows = rng.integers(0, n, 200)
    ref = oracle.grad_dense(a, g, x, b=b, phi=phi, psi=psi, rows=rows, cols=cols)
    for key, idx in [("db", cols), ("da", rows)] + ([("dpsi", cols), ("dphi", rows)] if phased else []):
        err = oracle.rel_l2(got[key][idx], ref[key])
        assert err < TOL, f"{key}: rel L2 {err:.3e}"
