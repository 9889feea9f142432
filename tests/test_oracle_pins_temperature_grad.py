"""Pins of the oracle's temperature argument and of its gradients.

Sources: "LAPLEX: The FFT of Learnable Laplace Kernels", technical summary
§2.1 (the operator and its temperature t -> 0 regime, trainable anchors and
phases), §2.3 (zero-temperature limit: equality routing, permutations and
CountSketch; uniform grids give Toeplitz matrices).

Temperature reading: entries exp(-|a - b| / t); t = 0 is the limit, the
equality-routing matrix.  Gradient reading: derivatives of the definition
with the symmetric subgradient 0 for |a - b| at a == b.

What pins them from outside the oracle: the Kac-Murdock-Szego closed form at
rho = exp(-h / t); the exact scaling identity K_t(a, b) = K_1(a / t, b / t)
for dyadic t and anchors; routing sums computed by equality tests; central
finite differences of the pinned forward definition (Richardson-extrapolated,
also at ties, where the central difference is exactly the mean of the two
one-sided slopes); a hand-derived two-point case; translation invariance.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(424242)


def kms_rowsums(n, rho):
    i = np.arange(1, n + 1, dtype=np.float64)
    return (1 + rho - rho ** i - rho ** (n - i + 1)) / (1 - rho)


# ---------------------------------------------------------------- temperature

@pytest.mark.parametrize("t", [0.25, 3.0])
@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_temperature_kms_rowsums(t, fn):
    n, h = 600, 2.0 ** -4
    sigma = RNG.permutation(n)
    a = (h * sigma).astype(np.float32)
    f = oracle.apply_dense if fn == "dense" else oracle.apply_sweep
    y = f(a, np.ones(n, np.float32), t=t)
    ref = kms_rowsums(n, np.exp(-h / t))[sigma]
    assert np.allclose(y, ref, rtol=1e-12, atol=0)


@pytest.mark.parametrize("t", [2.0 ** -3, 4.0])
def test_temperature_scaling_identity(t):
    # dyadic anchors and t: a / t is exact in float32, so K_t(a, b) = K_1(a/t, b/t)
    n, k = 120, 90
    a = (RNG.integers(-400, 400, n) * 2.0 ** -5).astype(np.float32)
    b = (RNG.integers(-400, 400, k) * 2.0 ** -5).astype(np.float32)
    b[:10] = a[:10]
    phi = RNG.uniform(-3, 3, n).astype(np.float32)
    psi = RNG.uniform(-3, 3, k).astype(np.float32)
    x = RNG.standard_normal((2, k)).astype(np.float32)
    xs = RNG.standard_normal((2, n)).astype(np.float32)
    at, bt = (a / np.float32(t)), (b / np.float32(t))
    assert np.array_equal(at.astype(np.float64) * t, a.astype(np.float64))
    for ph in [(None, None), (phi, psi)]:
        y_t = oracle.apply_sweep(a, x, b=b, phi=ph[0], psi=ph[1], t=t)
        y_1 = oracle.apply_dense(at, x, b=bt, phi=ph[0], psi=ph[1])
        assert np.allclose(y_t, y_1, rtol=1e-12, atol=1e-13)
        z_t = oracle.apply_sweep(a, xs, phi=ph[0], psi=ph[0], t=t)
        z_1 = oracle.apply_dense(at, xs, phi=ph[0], psi=ph[0])
        assert np.allclose(z_t, z_1, rtol=1e-12, atol=1e-13)
    D = RNG.uniform(0, 1, k).astype(np.float32)
    M_t = oracle.gram_direct(a, b, D, t=t)
    M_1 = oracle.gram_direct(at, bt, D)
    assert np.allclose(M_t, M_1, rtol=1e-12, atol=1e-14)


def routing_apply(out_anchor, in_anchor, x, out_phase=None, in_phase=None):
    """Zero-temperature operator by equality tests: y_i = sum_{q_j == o_i} cos(.) x_j."""
    y = np.zeros((x.shape[0], out_anchor.size))
    for i, o in enumerate(out_anchor):
        js = np.nonzero(in_anchor == o)[0]
        f = np.ones(js.size)
        if out_phase is not None:
            f = np.cos(out_phase[i].astype(np.float64) - in_phase[js].astype(np.float64))
        y[:, i] = (x[:, js].astype(np.float64) * f).sum(axis=1)
    return y


@pytest.mark.parametrize("fn", ["dense", "sweep"])
@pytest.mark.parametrize("phased", [False, True])
def test_zero_temperature_routes_close_anchors(fn, phased):
    # anchors close together (spacing ~1e-3): only t = 0 makes this a routing
    n, k = 300, 500
    a = np.unique(RNG.uniform(0, 0.3, n).astype(np.float32))
    n = a.size
    b = a[RNG.integers(0, n, k)]                          # CountSketch: several b per a
    b[:50] = RNG.uniform(0.5, 0.6, 50).astype(np.float32)  # b with no partner
    phi = RNG.uniform(-3, 3, n).astype(np.float32) if phased else None
    psi = RNG.uniform(-3, 3, k).astype(np.float32) if phased else None
    x = RNG.standard_normal((2, k)).astype(np.float32)
    w = RNG.standard_normal((2, n)).astype(np.float32)
    f = oracle.apply_dense if fn == "dense" else oracle.apply_sweep
    y = f(a, x, b=b, phi=phi, psi=psi, t=0.0)
    z = f(a, w, b=b, phi=phi, psi=psi, transpose=True, t=0.0)
    assert np.allclose(y, routing_apply(a, b, x, phi, psi), rtol=1e-14, atol=1e-14)
    assert np.allclose(z, routing_apply(b, a, w, psi, phi), rtol=1e-14, atol=1e-14)
    # symmetric at t = 0: identity on distinct anchors
    ys = f(a, w, t=0.0)
    assert np.array_equal(ys, w.astype(np.float64))


def test_zero_temperature_gram_and_limit():
    n, k = 200, 400
    a = np.unique(RNG.uniform(0, 1, n).astype(np.float32))
    n = a.size
    b = a[RNG.integers(0, n, k)]
    D = RNG.uniform(0, 1, k).astype(np.float32)
    M = oracle.gram_direct(a, b, D, t=0.0)
    ref = np.zeros((n, n))
    for i in range(n):
        ref[i, i] = D[b == a[i]].astype(np.float64).sum()
    assert np.allclose(M, ref, rtol=1e-14, atol=0)
    # gaps >= 1 at t = 1e-3: every off-partner entry underflows, equal to t = 0
    g = (np.arange(n) * 1.0).astype(np.float32)
    gb = g[RNG.integers(0, n, k)]
    x = RNG.standard_normal(k).astype(np.float32)
    assert np.array_equal(oracle.apply_sweep(g, x, b=gb, t=1e-3), oracle.apply_sweep(g, x, b=gb, t=0.0))


@pytest.mark.parametrize("bad", [-1.0, np.nan, np.inf])
def test_temperature_rejects_invalid(bad):
    a = np.zeros(3, np.float32)
    with pytest.raises(ValueError):
        oracle.apply_sweep(a, a, t=bad)


# ------------------------------------------------------------------ gradients

def forward_F(a, b, phi, psi, u, w, t):
    """F = sum_v <u_v, K w_v> through the (pinned) dense definition."""
    return float((u.astype(np.float64) * oracle.apply_dense(a, w, b=b, phi=phi, psi=psi, t=t)).sum())


def fd(fun, x0, i, h):
    """Central difference of fun along coordinate i, Richardson-extrapolated."""
    def d(step):
        xp, xm = x0.copy(), x0.copy()
        xp[i] += np.float32(step)
        xm[i] -= np.float32(step)
        assert xp[i] - x0[i] == np.float32(step) and x0[i] - xm[i] == np.float32(step)
        return (fun(xp) - fun(xm)) / (2 * step)
    return (4 * d(h / 2) - d(h)) / 3


def grid_case(n, k, phased, seed):
    rng = np.random.default_rng(seed)
    a = (rng.integers(-40, 40, n) * 2.0 ** -5).astype(np.float32)
    b = (rng.integers(-40, 40, k) * 2.0 ** -5).astype(np.float32)
    b[:3] = a[:3]  # ties between the sides
    a[3] = a[4]    # ties within a side
    phi = (rng.integers(-300, 300, n) * 2.0 ** -8).astype(np.float32) if phased else None
    psi = (rng.integers(-300, 300, k) * 2.0 ** -8).astype(np.float32) if phased else None
    u = rng.standard_normal((2, n)).astype(np.float32)
    w = rng.standard_normal((2, k)).astype(np.float32)
    return a, b, phi, psi, u, w


@pytest.mark.parametrize("phased", [False, True])
@pytest.mark.parametrize("t", [1.0, 0.5])
def test_grad_finite_differences_general(phased, t):
    n, k = 14, 11
    a, b, phi, psi, u, w = grid_case(n, k, phased, 5)
    g = oracle.grad_dense(a, u, w, b=b, phi=phi, psi=psi, t=t)
    h = 2.0 ** -10
    fda = [fd(lambda v: forward_F(v, b, phi, psi, u, w, t), a, i, h) for i in range(n)]
    fdb = [fd(lambda v: forward_F(a, v, phi, psi, u, w, t), b, j, h) for j in range(k)]
    assert np.allclose(g["da"], fda, rtol=1e-7, atol=1e-8)
    assert np.allclose(g["db"], fdb, rtol=1e-7, atol=1e-8)
    if phased:
        hp = 2.0 ** -12
        fdp = [fd(lambda v: forward_F(a, b, v, psi, u, w, t), phi, i, hp) for i in range(n)]
        fdq = [fd(lambda v: forward_F(a, b, phi, v, u, w, t), psi, j, hp) for j in range(k)]
        assert np.allclose(g["dphi"], fdp, rtol=1e-7, atol=1e-8)
        assert np.allclose(g["dpsi"], fdq, rtol=1e-7, atol=1e-8)
    else:
        assert "dphi" not in g


@pytest.mark.parametrize("phased", [False, True])
def test_grad_finite_differences_symmetric(phased):
    # one anchor vector on both sides: moving a_i moves row i and column i
    n = 13
    a, _, phi, _, u, _ = grid_case(n, n, phased, 9)
    psi = (RNG.integers(-300, 300, n) * 2.0 ** -8).astype(np.float32) if phased else None
    w = RNG.standard_normal((2, n)).astype(np.float32)
    g = oracle.grad_dense(a, u, w, phi=phi, psi=psi)
    assert "db" not in g
    h = 2.0 ** -10
    fda = [fd(lambda v: forward_F(v, v, phi, psi, u, w, 1.0), a, i, h) for i in range(n)]
    assert np.allclose(g["da"], fda, rtol=1e-7, atol=1e-8)
    if phased:
        hp = 2.0 ** -12
        fdp = [fd(lambda v: forward_F(a, a, v, psi, u, w, 1.0), phi, i, hp) for i in range(n)]
        fdq = [fd(lambda v: forward_F(a, a, phi, v, u, w, 1.0), psi, i, hp) for i in range(n)]
        assert np.allclose(g["dphi"], fdp, rtol=1e-7, atol=1e-8)
        assert np.allclose(g["dpsi"], fdq, rtol=1e-7, atol=1e-8)


def test_grad_two_point_closed_form():
    # K = [[1, e^-d], [e^-d, 1]] with d = a2 - a1 > 0 (symmetric, unphased):
    # F = u1 w1 + u2 w2 + e^-d (u1 w2 + u2 w1), dF/da1 = e^-d (u1 w2 + u2 w1) = -dF/da2
    a = np.array([0.25, 1.5], np.float32)
    u = np.array([2.0, -3.0], np.float32)
    w = np.array([0.5, 4.0], np.float32)
    g = oracle.grad_dense(a, u, w)["da"]
    c = np.exp(-1.25) * (2.0 * 4.0 + (-3.0) * 0.5)
    assert np.allclose(g, [c, -c], rtol=1e-15, atol=0)
    # at a tie the symmetric subgradient is 0
    assert np.array_equal(oracle.grad_dense(np.array([1.0, 1.0], np.float32), u, w)["da"], [0.0, 0.0])


def test_grad_translation_and_phase_shift_invariance():
    # K depends on a - b and phi - psi only: shifting everything leaves F unchanged
    n, k = 300, 200
    a = (RNG.standard_normal(n) * 3).astype(np.float32)
    b = (RNG.standard_normal(k) * 3).astype(np.float32)
    b[:20] = a[:20]
    phi = RNG.uniform(-3, 3, n).astype(np.float32)
    psi = RNG.uniform(-3, 3, k).astype(np.float32)
    u = RNG.standard_normal((3, n)).astype(np.float32)
    w = RNG.standard_normal((3, k)).astype(np.float32)
    g = oracle.grad_dense(a, u, w, b=b, phi=phi, psi=psi, t=0.7)
    scale = np.abs(g["da"]).sum() + np.abs(g["db"]).sum()
    assert abs(g["da"].sum() + g["db"].sum()) < 1e-12 * scale
    scale = np.abs(g["dphi"]).sum() + np.abs(g["dpsi"]).sum()
    assert abs(g["dphi"].sum() + g["dpsi"].sum()) < 1e-12 * scale


def test_grad_temperature_scaling_and_subsets():
    t = 2.0 ** -2
    n, k = 40, 30
    a = (RNG.integers(-200, 200, n) * 2.0 ** -6).astype(np.float32)
    b = (RNG.integers(-200, 200, k) * 2.0 ** -6).astype(np.float32)
    u = RNG.standard_normal((2, n)).astype(np.float32)
    w = RNG.standard_normal((2, k)).astype(np.float32)
    g_t = oracle.grad_dense(a, u, w, b=b, t=t)
    g_1 = oracle.grad_dense(a / np.float32(t), u, w, b=b / np.float32(t))
    # d/da F(a / t) = (1/t) F'(a / t)
    assert np.allclose(g_t["da"], g_1["da"] / t, rtol=1e-13, atol=1e-14)
    assert np.allclose(g_t["db"], g_1["db"] / t, rtol=1e-13, atol=1e-14)
    rows, cols = [3, 0, 39], [29, 5]
    gs = oracle.grad_dense(a, u, w, b=b, t=t, rows=rows, cols=cols)
    assert np.array_equal(gs["da"], g_t["da"][rows]) and np.array_equal(gs["db"], g_t["db"][cols])


def test_grad_zero_temperature():
    n, k = 50, 80
    a = np.unique(RNG.uniform(0, 1, n).astype(np.float32))
    n = a.size
    b = a[RNG.integers(0, n, k)]
    phi = RNG.uniform(-3, 3, n).astype(np.float32)
    psi = RNG.uniform(-3, 3, k).astype(np.float32)
    u = RNG.standard_normal((2, n)).astype(np.float32)
    w = RNG.standard_normal((2, k)).astype(np.float32)
    g = oracle.grad_dense(a, u, w, b=b, phi=phi, psi=psi, t=0.0)
    assert np.array_equal(g["da"], np.zeros(n)) and np.array_equal(g["db"], np.zeros(k))
    # dF/dphi_i = -sum over partners j of u_i w_j sin(phi_i - psi_j)
    ref = np.zeros(n)
    for i in range(n):
        js = np.nonzero(b == a[i])[0]
        uw = (u[:, i:i + 1].astype(np.float64) * w[:, js]).sum(axis=0)
        ref[i] = -(uw * np.sin(phi[i].astype(np.float64) - psi[js])).sum()
    assert np.allclose(g["dphi"], ref, rtol=1e-13, atol=1e-14)
