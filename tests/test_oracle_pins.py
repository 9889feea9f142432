"""Pins of the fp64 CPU oracle against facts that do not come from the oracle
itself: closed forms, textbook routines, invariants, brute force and the
hand-derived zero-temperature fixture.

Sources: "LAPLEX: The FFT of Learnable Laplace Kernels", technical summary
§2.1 (operator), §2.2 (sort + prefix/suffix recurrences, u/v bucketing, Gram)
and §2.3 (uniform-grid anchors give a Toeplitz matrix; the zero-temperature
limit routes by equality: permutations and CountSketch).
"""
import os

import numpy as np
import pytest

import oracle
from laplace_matvec_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(20261203)


def flip_keys_numpy(a):
    u = np.asarray(a, dtype=np.float32).view(np.uint32)
    return np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)


# --------------------------------------------------------------- argsort pins

@pytest.mark.parametrize("n", [1, 2, 7, 1000, 65537])
def test_argsort_matches_numpy_stable(n):
    a = (RNG.standard_normal(n) * 3).astype(np.float32)
    a[RNG.integers(0, n, size=n // 3)] = a[RNG.integers(0, n, size=n // 3)]  # ties
    ref = np.argsort(flip_keys_numpy(a), kind="stable")
    assert np.array_equal(oracle.argsort(a), ref.astype(np.uint32))


def test_argsort_signed_zero_denormal_and_ties():
    a = np.array([0.0, -0.0, 1e-45, -1e-45, 5.0, -5.0, 0.0, -0.0, 5.0, 3.4e38, -3.4e38],
                 dtype=np.float32)
    p = oracle.argsort(a)
    # -3.4e38 < -5 < -1e-45 < -0.0 (idx 1, 7) < +0.0 (idx 0, 6) < 1e-45 < 5 (4, 8) < 3.4e38
    assert p.tolist() == [10, 5, 3, 1, 7, 0, 6, 2, 4, 8, 9]
    ref = np.argsort(flip_keys_numpy(a), kind="stable")
    assert np.array_equal(p, ref.astype(np.uint32))


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_argsort_rejects_nonfinite(bad):
    a = np.array([1.0, bad, 2.0], dtype=np.float32)
    with pytest.raises(oracle.OracleError, match="non-finite"):
        oracle.argsort(a)


# ------------------------------------------------------ KMS / Toeplitz pins

def kms_case(n, h=2.0 ** -4, seed=1):
    """Anchors on a uniform grid, handed over in shuffled order."""
    rng = np.random.default_rng(seed)
    sigma = rng.permutation(n)
    a = (h * sigma).astype(np.float32)
    assert np.array_equal(a.astype(np.float64), h * sigma)  # exact in float32
    return a, sigma, np.exp(-h)


def kms_rowsums(n, rho):
    i = np.arange(1, n + 1, dtype=np.float64)
    return (1 + rho - rho ** i - rho ** (n - i + 1)) / (1 - rho)


def kms_inverse_apply(y_sorted, rho):
    """K^{-1} y for K_ij = rho^|i-j|: tridiagonal (-rho, [1, 1+rho^2, ..., 1], -rho)/(1-rho^2)."""
    n = y_sorted.shape[-1]
    d = np.full(n, 1 + rho * rho)
    d[0] = d[-1] = 1.0
    out = d * y_sorted
    out[..., 1:] -= rho * y_sorted[..., :-1]
    out[..., :-1] -= rho * y_sorted[..., 1:]
    return out / (1 - rho * rho)


def toeplitz_fft_apply(col, x_sorted):
    """Symmetric Toeplitz matrix-vector product by circulant embedding (numpy FFT)."""
    n = x_sorted.size
    c = np.concatenate([col, [0.0], col[:0:-1]])
    xp = np.concatenate([x_sorted, np.zeros(n)])
    return np.fft.ifft(np.fft.fft(c) * np.fft.fft(xp)).real[:n]


@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_kms_rowsums_closed_form(fn):
    n = 300
    a, sigma, rho = kms_case(n)
    ones = np.ones(n, dtype=np.float32)
    y = oracle.apply_dense(a, ones) if fn == "dense" else oracle.apply_sweep(a, ones)
    # element with grid rank sigma[i] has the row sum of row sigma[i]
    ref = kms_rowsums(n, rho)[sigma]
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_kms_inverse_recovers_x(fn):
    n = 257
    a, sigma, rho = kms_case(n, seed=2)
    x = RNG.standard_normal(n).astype(np.float32)
    y = oracle.apply_dense(a, x) if fn == "dense" else oracle.apply_sweep(a, x)
    order = np.argsort(sigma)  # positions in grid order
    rec = kms_inverse_apply(y[order], rho)
    np.testing.assert_allclose(rec, x[order].astype(np.float64), rtol=0, atol=1e-11)


@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_toeplitz_fft(fn):
    n = 500
    a, sigma, rho = kms_case(n, h=2.0 ** -3, seed=3)
    x = RNG.standard_normal(n).astype(np.float32)
    y = oracle.apply_dense(a, x) if fn == "dense" else oracle.apply_sweep(a, x)
    order = np.argsort(sigma)
    ref = toeplitz_fft_apply(rho ** np.arange(n), x[order].astype(np.float64))
    np.testing.assert_allclose(y[order], ref, rtol=0, atol=1e-11 * np.abs(ref).max())


@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_phased_toeplitz_fft(fn):
    """phi_i = omega a_i, psi_j = omega a_j on a grid: K_ij = rho^|i-j| cos(omega h (i-j))."""
    n = 400
    h = 2.0 ** -4
    a, sigma, rho = kms_case(n, h=h, seed=4)
    omega = 0.5
    phi = (omega * a).astype(np.float32)
    assert np.array_equal(phi.astype(np.float64), omega * h * sigma)
    x = RNG.standard_normal(n).astype(np.float32)
    if fn == "dense":
        y = oracle.apply_dense(a, x, phi=phi, psi=phi)
    else:
        y = oracle.apply_sweep(a, x, phi=phi, psi=phi)
    order = np.argsort(sigma)
    m = np.arange(n)
    ref = toeplitz_fft_apply(rho ** m * np.cos(omega * h * m), x[order].astype(np.float64))
    np.testing.assert_allclose(y[order], ref, rtol=0, atol=1e-11 * np.abs(ref).max())


# ---------------------------------------------------- zero-temperature pins

def load_golden(name):
    cases, cur = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "a" and cur:
                cases.append(cur)
                cur = {}
            cur[key] = np.array([float(v) for v in vals])
    if cur:
        cases.append(cur)
    return cases


@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_zero_temperature_golden(fn):
    cases = load_golden("zero_temperature_routing.txt")
    assert len(cases) == 3
    f = oracle.apply_dense if fn == "dense" else oracle.apply_sweep
    for c in cases:
        if "x" in c:
            y = f(c["a"], c["x"], b=c["b"])
            assert np.array_equal(y, c["y"]), (c, y)
        else:
            z = f(c["a"], c["w"], b=c["b"], transpose=True)
            assert np.array_equal(z, c["z"]), (c, z)


@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_zero_temperature_identity_symmetric(fn):
    n = 500
    a = (1024.0 * RNG.permutation(n) - 200000.0).astype(np.float32)
    x = RNG.standard_normal((3, n)).astype(np.float32)
    y = oracle.apply_dense(a, x) if fn == "dense" else oracle.apply_sweep(a, x)
    assert np.array_equal(y, x.astype(np.float64))


@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_zero_temperature_random_permutation(fn):
    n = 700
    a = (1024.0 * RNG.permutation(n)).astype(np.float32)
    sigma = RNG.permutation(n)
    b = a[sigma]
    x = RNG.standard_normal(n).astype(np.float32)
    f = oracle.apply_dense if fn == "dense" else oracle.apply_sweep
    y = f(a, x, b=b)
    # b_j == a_sigma[j]  =>  y_sigma[j] = x_j
    ref = np.empty(n)
    ref[sigma] = x
    assert np.array_equal(y, ref)
    z = f(a, x, b=b, transpose=True)
    assert np.array_equal(z, x[sigma].astype(np.float64))


@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_signed_countsketch(fn):
    """psi = 0, phi in {0, pi}: signed bucket sums (cos(float32(pi)) = -1 + 4e-15)."""
    n, k = 64, 500
    a = (1024.0 * np.arange(n)).astype(np.float32)
    h = RNG.integers(0, n, size=k)
    b = a[h]
    phi = np.where(RNG.random(n) < 0.5, 0.0, np.pi).astype(np.float32)
    psi = np.zeros(k, dtype=np.float32)
    x = RNG.integers(-8, 9, size=k).astype(np.float32)
    f = oracle.apply_dense if fn == "dense" else oracle.apply_sweep
    y = f(a, x, b=b, phi=phi, psi=psi)
    sign = np.where(phi == 0, 1.0, -1.0)
    ref = sign * np.bincount(h, weights=x.astype(np.float64), minlength=n)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13 * max(1.0, np.abs(ref).max()))


# ------------------------------------------------------------ invariants

@pytest.mark.parametrize("fn", ["dense", "sweep"])
def test_adjoint_identity_phased(fn):
    n, k = 300, 170
    a = (RNG.standard_normal(n) * 4).astype(np.float32)
    b = (RNG.standard_normal(k) * 4).astype(np.float32)
    phi = RNG.uniform(0, 6.28, n).astype(np.float32)
    psi = RNG.uniform(0, 6.28, k).astype(np.float32)
    x = RNG.standard_normal(k).astype(np.float32)
    w = RNG.standard_normal(n).astype(np.float32)
    f = oracle.apply_dense if fn == "dense" else oracle.apply_sweep
    lhs = np.dot(f(a, x, b=b, phi=phi, psi=psi), w.astype(np.float64))
    rhs = np.dot(x.astype(np.float64), f(a, w, b=b, phi=phi, psi=psi, transpose=True))
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1)


def test_symmetric_unphased_is_self_adjoint_and_translation_invariant():
    n = 256
    a = (np.round(RNG.standard_normal(n) * 64) / 16).astype(np.float32)  # dyadic, ties
    x = RNG.standard_normal(n).astype(np.float32)
    K = oracle.dense_matrix(a)
    assert np.array_equal(K, K.T)
    assert np.all(np.diag(K) == 1.0)
    shift = np.float32(37.5)
    y0 = oracle.apply_dense(a, x)
    y1 = oracle.apply_dense(a + shift, x)
    assert np.array_equal(y0, y1)  # differences of dyadic anchors are exact


def test_permutation_equivariance_and_linearity():
    n = 200
    a = (RNG.standard_normal(n) * 3).astype(np.float32)
    x1 = RNG.standard_normal(n).astype(np.float32)
    x2 = RNG.standard_normal(n).astype(np.float32)
    pi = RNG.permutation(n)
    y = oracle.apply_sweep(a, x1)
    yp = oracle.apply_sweep(a[pi], x1[pi])
    np.testing.assert_allclose(yp, y[pi], rtol=1e-13, atol=1e-13)
    lin = oracle.apply_sweep(a, np.stack([x1, x2, (2 * x1.astype(np.float64) - 3 * x2).astype(np.float32)]))
    np.testing.assert_allclose(lin[2], 2 * lin[0] - 3 * lin[1], rtol=0, atol=1e-5)


# ------------------------------------------- sweep vs dense (brute force)

@pytest.mark.parametrize("n", [1, 2, 3, 17, 1000, 4096])
@pytest.mark.parametrize("phased", [False, True])
def test_sym_sweep_vs_dense(n, phased):
    a = (RNG.standard_normal(n) * 8).astype(np.float32)
    if n > 10:
        a[RNG.integers(0, n, n // 10)] = a[RNG.integers(0, n, n // 10)]  # exact ties
    x = RNG.standard_normal((2, n)).astype(np.float32)
    kw = {}
    if phased:
        kw = dict(phi=RNG.uniform(0, 6.3, n).astype(np.float32),
                  psi=RNG.uniform(0, 6.3, n).astype(np.float32))
    for tr in (False, True):
        ys = oracle.apply_sweep(a, x, transpose=tr, **kw)
        yd = oracle.apply_dense(a, x, transpose=tr, **kw)
        assert oracle.rel_l2(ys, yd) < 1e-12


@pytest.mark.parametrize("n,k", [(1, 1), (5, 3), (300, 1024), (1024, 300), (2000, 2000)])
@pytest.mark.parametrize("phased", [False, True])
def test_general_sweep_vs_dense(n, k, phased):
    a = (RNG.standard_normal(n) * 20).astype(np.float32)
    b = RNG.uniform(-60, 60, k).astype(np.float32)   # b reaches beyond the range of a
    m = min(n, k) // 4
    if m:
        b[RNG.integers(0, k, m)] = a[RNG.integers(0, n, m)]  # b equal to some a
    kw = {}
    if phased:
        kw = dict(phi=RNG.uniform(0, 6.3, n).astype(np.float32),
                  psi=RNG.uniform(0, 6.3, k).astype(np.float32))
    x = RNG.standard_normal((2, k)).astype(np.float32)
    w = RNG.standard_normal((2, n)).astype(np.float32)
    assert oracle.rel_l2(oracle.apply_sweep(a, x, b=b, **kw), oracle.apply_dense(a, x, b=b, **kw)) < 1e-12
    assert oracle.rel_l2(oracle.apply_sweep(a, w, b=b, transpose=True, **kw),
                         oracle.apply_dense(a, w, b=b, transpose=True, **kw)) < 1e-12


def test_dense_rows_subset_matches_full():
    n = 333
    a = (RNG.standard_normal(n) * 2).astype(np.float32)
    x = RNG.standard_normal((2, n)).astype(np.float32)
    rows = np.array([0, 5, 332, 17, 5])
    full = oracle.apply_dense(a, x)
    sub = oracle.apply_dense(a, x, rows=rows)   # few rows: the sum is split over threads
    np.testing.assert_allclose(sub, full[:, rows], rtol=1e-14, atol=1e-14)


def test_workload_inputs_reduced_sizes():
    inp = wl.config_inputs(2, n=1 << 16, batch=2)
    a = inp["a"]
    assert a.dtype == np.float32 and a.min() >= 0 and a.max() <= 0.05 * (1 << 24)
    assert np.unique(a).size < a.size  # duplicates injected
    inp3 = wl.config_inputs(3, n=4096, k=128, batch=2)
    assert inp3["x"].shape == (2, 128) and inp3["w"].shape == (2, 4096)
    assert inp3["phi"].size == 4096 and inp3["psi"].size == 128


# ------------------------------------------------------------------ Gram pins

def test_gram_zero_temperature_is_permuted_diagonal():
    n = 50
    a = (1024.0 * RNG.permutation(n)).astype(np.float32)
    sigma = RNG.permutation(n)
    b = a[sigma]          # A = K(a, b) is a permutation matrix: A[sigma[j], j] = 1
    D = RNG.uniform(0, 1, n).astype(np.float32)
    M = oracle.gram_direct(a, b, D)
    ref = np.zeros((n, n))
    ref[sigma, sigma] = D
    assert np.array_equal(M, ref)


def test_gram_countsketch_diagonal_sums():
    n, k = 16, 300
    a = (1024.0 * np.arange(n)).astype(np.float32)
    h = RNG.integers(0, n, k)
    D = RNG.integers(0, 5, k).astype(np.float32)
    M = oracle.gram_direct(a, a[h], D)
    assert np.array_equal(M, np.diag(np.bincount(h, weights=D.astype(np.float64), minlength=n)))


def test_gram_kms_inverse_both_sides():
    """a = b on a grid: M = K diag(D) K with K Kac-Murdock-Szego, so
    K^{-1} M K^{-1} = diag(D) with the closed-form tridiagonal inverse."""
    n = 120
    a, sigma, rho = kms_case(n, h=2.0 ** -3, seed=5)
    D = RNG.uniform(0, 1, n).astype(np.float32)
    M = oracle.gram_direct(a, a, D)
    order = np.argsort(sigma)
    Ms = M[np.ix_(order, order)]
    X = kms_inverse_apply(kms_inverse_apply(Ms, rho).T, rho)
    np.testing.assert_allclose(X, np.diag(D[order].astype(np.float64)), rtol=0, atol=1e-9)


def test_gram_matches_apply_composition_and_is_psd():
    n, k = 64, 900
    a = (RNG.standard_normal(n) * 5).astype(np.float32)
    b = (RNG.standard_normal(k) * 5).astype(np.float32)
    D = RNG.uniform(0, 1, k).astype(np.float32)
    M = oracle.gram_direct(a, b, D)
    assert np.allclose(M, M.T, rtol=1e-14, atol=0)
    for j in (0, 13, 63):
        e = np.zeros(n, dtype=np.float32)
        e[j] = 1
        col_in = oracle.apply_dense(a, e, b=b, transpose=True) * D      # D * A^T e_j (float64)
        col = oracle.dense_matrix(a, b=b) @ col_in                       # A (D * A^T e_j)
        np.testing.assert_allclose(M[:, j], col, rtol=1e-12, atol=1e-300)
    assert np.linalg.eigvalsh(M).min() > -1e-10 * np.abs(M).max()


def test_gram_subset_matches_full():
    n, k = 40, 500
    a = (RNG.standard_normal(n) * 5).astype(np.float32)
    b = (RNG.standard_normal(k) * 5).astype(np.float32)
    D = RNG.uniform(0, 1, k).astype(np.float32)
    full = oracle.gram_direct(a, b, D)
    rows, cols = np.array([3, 0, 39]), np.array([7, 3])
    assert np.array_equal(oracle.gram_direct(a, b, D, rows=rows, cols=cols), full[np.ix_(rows, cols)])


def test_phased_gram_zero_phases_is_unphased():
    n, k = 30, 400
    a = (RNG.standard_normal(n) * 3).astype(np.float32)
    b = (RNG.standard_normal(k) * 3).astype(np.float32)
    D = RNG.uniform(-1, 1, k).astype(np.float32)
    z_n, z_k = np.zeros(n, np.float32), np.zeros(k, np.float32)
    assert np.array_equal(oracle.gram_direct(a, b, D, phi=z_n, psi=z_k), oracle.gram_direct(a, b, D))


def test_phased_gram_zero_temperature_signed_diagonal():
    """A = K(a, phi; b, psi) with b = a[sigma] far apart: A[sigma_j, j] = cos(phi - psi),
    so M is diagonal with D_j cos^2(phi_sigma_j - psi_j) (float64 cos of float32 phases)."""
    n = 40
    a = (1024.0 * RNG.permutation(n)).astype(np.float32)
    sigma = RNG.permutation(n)
    phi = RNG.uniform(0, 6.28, n).astype(np.float32)
    psi = RNG.uniform(0, 6.28, n).astype(np.float32)
    D = RNG.uniform(0, 1, n).astype(np.float32)
    M = oracle.gram_direct(a, a[sigma], D, phi=phi, psi=psi)
    ref = np.zeros((n, n))
    ref[sigma, sigma] = D * np.cos(phi[sigma].astype(np.float64) - psi.astype(np.float64)) ** 2
    np.testing.assert_allclose(M, ref, rtol=1e-15, atol=1e-300)


def test_phased_gram_matches_apply_composition():
    n, k = 50, 700
    a = (RNG.standard_normal(n) * 5).astype(np.float32)
    b = (RNG.standard_normal(k) * 5).astype(np.float32)
    phi = RNG.uniform(0, 6.28, n).astype(np.float32)
    psi = RNG.uniform(0, 6.28, k).astype(np.float32)
    D = RNG.uniform(0, 1, k).astype(np.float32)
    M = oracle.gram_direct(a, b, D, phi=phi, psi=psi)
    A = oracle.dense_matrix(a, b=b, phi=phi, psi=psi)
    for j in (0, 7, 49):
        e = np.zeros(n, dtype=np.float32)
        e[j] = 1
        col_in = oracle.apply_dense(a, e, b=b, phi=phi, psi=psi, transpose=True) * D
        np.testing.assert_allclose(M[:, j], A @ col_in, rtol=1e-12, atol=1e-14)
