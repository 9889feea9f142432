"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar (the operator's own precision claim is float32; tolerances from the
arithmetic): sort permutations bit-exact; float32 outputs within relative L2
1e-5 per vector (max over the batch); zero-temperature routing bit-exact.
Sizes span several sort tiles (8192) and scan tiles (4096) with ragged tails.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from laplace_matvec_amd import laplex as lx
from laplace_matvec_amd import workloads as wl

pytestmark = pytest.mark.gpu
TOL = 1e-5
RNG = np.random.default_rng(7)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def max_rel(y, ref):
    y = np.atleast_2d(y)
    ref = np.atleast_2d(ref)
    return max(oracle.rel_l2(y[i], ref[i]) for i in range(y.shape[0]))


def anchors_with_ties(n, scale, rng=RNG):
    a = (rng.standard_normal(n) * scale).astype(np.float32)
    if n > 10:
        m = n // 20
        a[rng.integers(0, n, m)] = a[rng.integers(0, n, m)]
    return a


# ----------------------------------------------------------------- symmetric

@pytest.mark.parametrize("n", [1, 2, 3, 63, 4096, 8193, 50001])
def test_symmetric_perm_and_apply(gpu, n):
    say(f"[sym] n={n}")
    a = anchors_with_ties(n, 8.0)
    x = RNG.standard_normal((3, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a)) as plan:
        perm = host(lx.laplex_plan_perm(plan))
        assert np.array_equal(perm, oracle.argsort(a).astype(np.int64))
        srt = host(lx.laplex_plan_sorted(plan))
        assert np.array_equal(srt, a[perm])
        y = host(lx.laplex_apply(plan, dev(x)))
    ref = oracle.apply_dense(a, x) if n <= 50001 else oracle.apply_sweep(a, x)
    assert max_rel(y, ref) < TOL


@pytest.mark.parametrize("n", [5, 4097, 30000])
def test_symmetric_phased_both_directions(gpu, n):
    say(f"[sym phased] n={n}")
    a = anchors_with_ties(n, 4.0)
    phi = RNG.uniform(0, 6.3, n).astype(np.float32)
    psi = RNG.uniform(0, 6.3, n).astype(np.float32)
    x = RNG.standard_normal((2, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a), phi=dev(phi), psi=dev(psi)) as plan:
        for tr in (False, True):
            y = host(lx.laplex_apply(plan, dev(x), transpose=tr))
            ref = oracle.apply_dense(a, x, phi=phi, psi=psi, transpose=tr)
            assert max_rel(y, ref) < TOL, tr


def test_symmetric_config1_n4096(gpu):
    """Configuration 1: n = 4096, a ~ 8 N(0,1), x ~ N(0,1), one vector, vs the dense definition."""
    say("[sym] config 1")
    inp = wl.config_inputs(1)
    a, x = inp["a"], inp["x"]
    with lx.laplex_plan_create(dev(a)) as plan:
        assert np.array_equal(host(lx.laplex_plan_perm(plan)), oracle.argsort(a).astype(np.int64))
        y = host(lx.laplex_apply(plan, dev(x)))
    assert max_rel(y, oracle.apply_dense(a, x)) < TOL


def test_symmetric_larger_vs_sweep(gpu):
    n = 1_000_003
    say(f"[sym] n={n} vs sweep")
    a = anchors_with_ties(n, 50.0)
    x = RNG.standard_normal((2, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a)) as plan:
        assert np.array_equal(host(lx.laplex_plan_perm(plan)), oracle.argsort(a).astype(np.int64))
        y = host(lx.laplex_apply(plan, dev(x)))
    assert max_rel(y, oracle.apply_sweep(a, x)) < TOL


@pytest.mark.parametrize("n,batch,phased", [(1 << 20, 1, False), (1_500_001, 3, False), (1_234_567, 2, True)])
def test_symmetric_replay_path(gpu, n, batch, phased):
    """Sides of 2^20 or more move x into sorted order (and y back) by
    replaying the radix passes instead of gathering through the permutation."""
    say(f"[sym replay] n={n} batch={batch} phased={phased}")
    rng = np.random.default_rng(n)
    a = anchors_with_ties(n, 300.0, rng)
    x = rng.standard_normal((batch, n)).astype(np.float32)
    kw = {}
    if phased:
        kw = dict(phi=rng.uniform(0, 6.3, n).astype(np.float32), psi=rng.uniform(0, 6.3, n).astype(np.float32))
    with lx.laplex_plan_create(dev(a), **{k: dev(v) for k, v in kw.items()}) as plan:
        y = host(lx.laplex_apply(plan, dev(x)))
        yt = host(lx.laplex_apply(plan, dev(x), transpose=True)) if phased else None
        perm = host(lx.laplex_plan_perm(plan))
    assert np.array_equal(perm, oracle.argsort(a).astype(np.int64))
    assert max_rel(y, oracle.apply_sweep(a, x, **kw)) < TOL
    if phased:
        assert max_rel(yt, oracle.apply_sweep(a, x, transpose=True, **kw)) < TOL


def test_replay_zero_temperature_bitwise(gpu):
    """Replayed permutation moves every value exactly (K = I at zero temperature)."""
    n = (1 << 21) + 77
    a = (128.0 * np.random.default_rng(5).permutation(n) - 1.0e8).astype(np.float32)
    x = np.random.default_rng(6).standard_normal((2, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a)) as plan:
        y = host(lx.laplex_apply(plan, dev(x)))
    assert np.array_equal(y, x)


def test_zero_temperature_identity_bitwise(gpu):
    n = 20000
    a = (128.0 * RNG.permutation(n) - 1.0e6).astype(np.float32)
    x = RNG.standard_normal((2, n)).astype(np.float32)
    with lx.laplex_plan_create(dev(a)) as plan:
        y = host(lx.laplex_apply(plan, dev(x)))
    assert np.array_equal(y, x)


def test_special_values_sort_order(gpu):
    a = np.array([0.0, -0.0, 1e-45, -1e-45, 5.0, -5.0, 0.0, -0.0, 5.0, 3.4e38, -3.4e38] * 1000,
                 dtype=np.float32)
    with lx.laplex_plan_create(dev(a)) as plan:
        assert np.array_equal(host(lx.laplex_plan_perm(plan)), oracle.argsort(a).astype(np.int64))


def test_nonfinite_anchor_rejected(gpu):
    for bad in (np.nan, np.inf, -np.inf):
        a = RNG.standard_normal(10000).astype(np.float32)
        a[777] = bad
        with pytest.raises(lx.LaplexError) as e:
            lx.laplex_plan_create(dev(a))
        assert e.value.status == lx.ERR_NONFINITE_ANCHOR
    a = RNG.standard_normal(100).astype(np.float32)
    phi = np.zeros(100, np.float32)
    phi[3] = np.nan
    with pytest.raises(lx.LaplexError) as e:
        lx.laplex_plan_create(dev(a), phi=dev(phi), psi=dev(np.zeros(100, np.float32)))
    assert e.value.status == lx.ERR_NONFINITE_ANCHOR


def test_determinism_repeated(gpu):
    n = 70000
    a = anchors_with_ties(n, 3.0)
    x = dev(RNG.standard_normal((2, n)))
    outs, perms = [], []
    for _ in range(3):
        with lx.laplex_plan_create(dev(a)) as plan:
            perms.append(host(lx.laplex_plan_perm(plan)))
            outs.append(host(lx.laplex_apply(plan, x)))
    assert all(np.array_equal(perms[0], p) for p in perms)
    assert all(np.array_equal(outs[0], o) for o in outs)


def test_profile_only_one_label(gpu):
    """Kernel timing limited to one label: the same launches of that label
    are timed, and no other label is."""
    n = 70000
    a = dev(RNG.standard_normal(n))
    x = dev(RNG.standard_normal((2, n)))

    def timed(label):
        lx.profile_only(label)
        lx.profile_reset()
        lx.profile_enable(True)
        try:
            with lx.laplex_plan_create(a) as plan:
                lx.laplex_apply(plan, x)
            torch.cuda.synchronize()
            return lx.profile_read()
        finally:
            lx.profile_enable(False)
            lx.profile_only(None)

    every = timed(None)
    assert len(every) >= 2
    label = max(every, key=lambda k: every[k][1])
    only = timed(label)
    assert set(only) == {label}
    assert only[label][0] == every[label][0] and only[label][1] > 0


def test_apply_overlap_rejected(gpu):
    a = dev(RNG.standard_normal(100))
    buf = torch.zeros(300, device="cuda")
    with lx.laplex_plan_create(a) as plan:
        st = lx.load().laplex_apply(plan.handle, lx._ptr(buf), lx._ptr(buf[50:]), 1, 0, None)
        assert st == lx.ERR_INVALID_ARGUMENT
        st = lx.load().laplex_apply(plan.handle, lx._ptr(buf), lx._ptr(buf[100:]), 1, 2, None)
        assert st == lx.ERR_INVALID_ARGUMENT


# ------------------------------------------------------------------- general

GENERAL_CASES = [(1, 1), (7, 3), (5000, 1024), (1024, 5000), (20001, 300), (300, 20001)]


@pytest.mark.parametrize("n,k", GENERAL_CASES)
@pytest.mark.parametrize("phased", [False, True])
@pytest.mark.parametrize("algo", [lx.ALGO_AUTO, lx.ALGO_BUCKET, lx.ALGO_EVALUATE])
def test_general_both_directions(gpu, n, k, phased, algo):
    say(f"[general] n={n} k={k} phased={phased} algo={algo}")
    rng = np.random.default_rng(n * 31 + k)
    a = (rng.standard_normal(n) * 20).astype(np.float32)
    b = rng.uniform(-60, 60, k).astype(np.float32)
    m = min(n, k) // 4
    if m:
        b[rng.integers(0, k, m)] = a[rng.integers(0, n, m)]  # inputs on top of outputs
    kw = {}
    if phased:
        kw = dict(phi=rng.uniform(0, 6.3, n).astype(np.float32), psi=rng.uniform(0, 6.3, k).astype(np.float32))
    x = rng.standard_normal((3, k)).astype(np.float32)
    w = rng.standard_normal((3, n)).astype(np.float32)
    dkw = {key: dev(v) for key, v in kw.items()}
    with lx.laplex_plan_create(dev(a), b=dev(b), **dkw) as plan:
        lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, algo)
        assert np.array_equal(host(lx.laplex_plan_perm(plan, 0)), oracle.argsort(a).astype(np.int64))
        assert np.array_equal(host(lx.laplex_plan_perm(plan, 1)), oracle.argsort(b).astype(np.int64))
        y = host(lx.laplex_apply(plan, dev(x)))
        z = host(lx.laplex_apply(plan, dev(w), transpose=True))
    assert max_rel(y, oracle.apply_dense(a, x, b=b, **kw)) < TOL
    assert max_rel(z, oracle.apply_dense(a, w, b=b, transpose=True, **kw)) < TOL


@pytest.mark.parametrize("algo", [lx.ALGO_BUCKET, lx.ALGO_EVALUATE])
def test_general_repeat_bitwise(gpu, algo):
    """A small sorted side (1024 anchors, the bucketing in LDS or the
    evaluation): the same products three times, on the same plan and on a
    new one, give the same bits (no atomics; fixed summation order)."""
    rng = np.random.default_rng(1024)
    n, k = 200000, 1024
    a = (rng.standard_normal(n) * 100).astype(np.float32)
    b = rng.uniform(-300, 300, k).astype(np.float32)
    kw = dict(phi=rng.uniform(0, 6.3, n).astype(np.float32), psi=rng.uniform(0, 6.3, k).astype(np.float32))
    x = dev(rng.standard_normal((5, k)))
    w = dev(rng.standard_normal((5, n)))
    ys, zs = [], []
    for rep in range(2):
        with lx.laplex_plan_create(dev(a), b=dev(b), **{key: dev(v) for key, v in kw.items()}) as plan:
            lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, algo)
            for _ in range(2 if rep == 0 else 1):
                ys.append(host(lx.laplex_apply(plan, x)))
                zs.append(host(lx.laplex_apply(plan, w, transpose=True)))
    assert all(np.array_equal(ys[0], y) for y in ys[1:])
    assert all(np.array_equal(zs[0], z) for z in zs[1:])
    assert max_rel(ys[0], oracle.apply_sweep(a, host(x), b=b, **kw)) < TOL
    assert max_rel(zs[0], oracle.apply_sweep(a, host(w), b=b, transpose=True, **kw)) < TOL


@pytest.mark.parametrize("phased", [False, True])
@pytest.mark.parametrize("algo", [lx.ALGO_BUCKET, lx.ALGO_EVALUATE])
def test_general_partial_vector_groups(gpu, phased, algo):
    """11 vectors: the evaluation and bucketing kernels run them as groups
    of 6 and 5 (and 8 + 3), so the last group is partial; ragged sizes and
    outputs outside the input range on both sides."""
    n, k, B = 30011, 777, 11
    say(f"[general groups] n={n} k={k} B={B} phased={phased} algo={algo}")
    rng = np.random.default_rng(4242 + phased)
    a = (rng.standard_normal(n) * 20).astype(np.float32)
    b = rng.uniform(-45, 45, k).astype(np.float32)
    b[:40] = a[rng.integers(0, n, 40)]
    kw = {}
    if phased:
        kw = dict(phi=rng.uniform(0, 6.3, n).astype(np.float32), psi=rng.uniform(0, 6.3, k).astype(np.float32))
    x = rng.standard_normal((B, k)).astype(np.float32)
    w = rng.standard_normal((B, n)).astype(np.float32)
    dkw = {key: dev(v) for key, v in kw.items()}
    with lx.laplex_plan_create(dev(a), b=dev(b), **dkw) as plan:
        lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, algo)
        y = host(lx.laplex_apply(plan, dev(x)))
        z = host(lx.laplex_apply(plan, dev(w), transpose=True))
    assert max_rel(y, oracle.apply_dense(a, x, b=b, **kw)) < TOL
    assert max_rel(z, oracle.apply_dense(a, w, b=b, transpose=True, **kw)) < TOL


@pytest.mark.parametrize("algo", [lx.ALGO_BUCKET, lx.ALGO_EVALUATE])
def test_general_zero_temperature_permutation_bitwise(gpu, algo):
    n = 9000
    a = (1024.0 * RNG.permutation(n)).astype(np.float32)
    sigma = RNG.permutation(n)
    b = a[sigma]
    x = RNG.standard_normal(n).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b)) as plan:
        lx.laplex_plan_set_option(plan, lx.OPT_GENERAL_ALGO, algo)
        y = host(lx.laplex_apply(plan, dev(x)))
        z = host(lx.laplex_apply(plan, dev(x), transpose=True))
    ref = np.empty(n, np.float32)
    ref[sigma] = x
    assert np.array_equal(y, ref)
    assert np.array_equal(z, x[sigma])


def test_general_golden_countsketch(gpu):
    import os
    from test_oracle_pins import load_golden
    for c in load_golden("zero_temperature_routing.txt"):
        with lx.laplex_plan_create(dev(c["a"]), b=dev(c["b"])) as plan:
            if "x" in c:
                assert np.array_equal(host(lx.laplex_apply(plan, dev(c["x"]))), c["y"].astype(np.float32))
            else:
                assert np.array_equal(host(lx.laplex_apply(plan, dev(c["w"]), transpose=True)),
                                      c["z"].astype(np.float32))


# ---------------------------------------------------------------------- Gram

@pytest.mark.parametrize("n,k", [(1, 1), (5, 17), (300, 5000), (1000, 70000)])
def test_gram_general(gpu, n, k):
    say(f"[gram] n={n} k={k}")
    rng = np.random.default_rng(n + k)
    a = (rng.standard_normal(n) * 20).astype(np.float32)
    b = (rng.standard_normal(k) * 20).astype(np.float32)
    m = min(n, k) // 5
    if m:
        b[rng.integers(0, k, m)] = a[rng.integers(0, n, m)]
        a[rng.integers(0, n, m)] = a[rng.integers(0, n, m)]
    D = rng.uniform(0, 1, k).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b)) as plan:
        M = host(lx.laplex_gram(plan, dev(D)))
    ref = oracle.gram_direct(a, b, D)
    assert oracle.rel_l2(M, ref) < TOL


def test_gram_repeated_calls_and_temperature(gpu):
    """One plan, several Gram calls: the interval bounds the first call
    makes are reused, also after a temperature change and with new weights;
    inputs outside the anchor range and many inputs per interval."""
    rng = np.random.default_rng(77)
    n, k = 300, 30001
    a = (rng.standard_normal(n) * 15).astype(np.float32)
    b = (rng.standard_normal(k) * 25).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b)) as plan:
        for t, seed in ((1.0, 1), (0.5, 2), (2.0, 3)):
            lx.laplex_plan_set_temperature(plan, t)
            D = np.random.default_rng(seed).uniform(-1, 1, k).astype(np.float32)
            M = host(lx.laplex_gram(plan, dev(D)))
            ref = oracle.gram_direct(a, b, D, t=t)
            assert oracle.rel_l2(M, ref) < TOL, (t, seed)


@pytest.mark.parametrize("phased", [False, True])
def test_gram_wide_anchor_span(gpu, phased):
    """Anchors spanning 2500 t, in ascending original order: no centre
    serves all the anchors, so tiles near the diagonal (64 neighbouring
    anchors, about 230 t) split the decay about their own centre and tiles
    far from it take a decay per entry."""
    rng = np.random.default_rng(2500 + phased)
    n, k = 700, 6000
    a = np.sort(rng.uniform(0, 2500, n)).astype(np.float32)
    b = rng.uniform(-100, 2600, k).astype(np.float32)
    phi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    psi = rng.uniform(-np.pi, np.pi, k).astype(np.float32) if phased else None
    D = rng.uniform(0, 1, k).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        M = host(lx.laplex_gram(plan, dev(D)))
    ref = oracle.gram_direct(a, b, D, phi=phi, psi=psi)
    assert oracle.rel_l2(M, ref) < TOL
    near = np.abs(np.subtract.outer(np.arange(n), np.arange(n))) < 64
    assert oracle.rel_l2(M[near], ref[near]) < TOL


@pytest.mark.parametrize("n,k,phased", [(5037, 6000, False), (2531, 4000, True)])
def test_gram_scan_over_several_rounds(gpu, n, k, phased):
    """More intervals than one round of the scan (4096 per round, 2048 with
    three weight sets), with a ragged last round: 64 sampled rows of M
    against the definition."""
    say(f"[gram rounds] n={n} k={k} phased={phased}")
    rng = np.random.default_rng(n + 3 * k)
    a = (rng.standard_normal(n) * 20).astype(np.float32)
    b = (rng.standard_normal(k) * 20).astype(np.float32)
    b[rng.integers(0, k, 100)] = a[rng.integers(0, n, 100)]
    phi = rng.uniform(-np.pi, np.pi, n).astype(np.float32) if phased else None
    psi = rng.uniform(-np.pi, np.pi, k).astype(np.float32) if phased else None
    D = rng.uniform(-1, 1, k).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=None if phi is None else dev(phi),
                               psi=None if psi is None else dev(psi)) as plan:
        M = host(lx.laplex_gram(plan, dev(D)))
    rows = np.unique(np.concatenate([[0, n - 1, n // 2, 4095, 4096, 2047, 2048],
                                     rng.integers(0, n, 64)]))
    rows = rows[rows < n]
    ref = oracle.gram_direct(a, b, D, phi=phi, psi=psi, rows=rows, cols=np.arange(n))
    assert oracle.rel_l2(M[rows], ref) < TOL


@pytest.mark.parametrize("phased", [False, True])
def test_gram_repeat_bitwise(gpu, phased):
    """Gram calls on one plan and on a new plan give the same bits: the
    per-plan grouping of the inputs is stable, and the slices, intervals and
    lanes are added in a fixed order."""
    rng = np.random.default_rng(31 + phased)
    n, k = 900, 120000
    a = (rng.standard_normal(n) * 20).astype(np.float32)
    b = (rng.standard_normal(k) * 20).astype(np.float32)
    kw = {}
    if phased:
        kw = dict(phi=rng.uniform(0, 6.3, n).astype(np.float32), psi=rng.uniform(0, 6.3, k).astype(np.float32))
    D = dev(rng.uniform(-1, 1, k))
    outs = []
    for rep in range(2):
        with lx.laplex_plan_create(dev(a), b=dev(b), **{key: dev(v) for key, v in kw.items()}) as plan:
            for _ in range(2 if rep == 0 else 1):
                outs.append(host(lx.laplex_gram(plan, D)))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    rows = np.arange(0, n, 37)
    ref = oracle.gram_direct(a, b, host(D), rows=rows, cols=np.arange(n), **kw)
    assert oracle.rel_l2(outs[0][rows], ref) < TOL


def test_gram_symmetric_plan(gpu):
    n = 2000
    a = anchors_with_ties(n, 10.0)
    D = RNG.uniform(0, 1, n).astype(np.float32)
    with lx.laplex_plan_create(dev(a)) as plan:
        M = host(lx.laplex_gram(plan, dev(D)))
    assert oracle.rel_l2(M, oracle.gram_direct(a, a, D)) < TOL


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (300, 5000), (400, 40000)])
def test_gram_phased_general(gpu, n, k):
    say(f"[gram phased] n={n} k={k}")
    rng = np.random.default_rng(7 * n + k)
    a = (rng.standard_normal(n) * 20).astype(np.float32)
    b = (rng.standard_normal(k) * 20).astype(np.float32)
    m = min(n, k) // 5
    if m:
        b[rng.integers(0, k, m)] = a[rng.integers(0, n, m)]
    phi = rng.uniform(-np.pi, np.pi, n).astype(np.float32)
    psi = rng.uniform(-np.pi, np.pi, k).astype(np.float32)
    D = rng.uniform(-1, 1, k).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(b), phi=dev(phi), psi=dev(psi)) as plan:
        M = host(lx.laplex_gram(plan, dev(D)))
    ref = oracle.gram_direct(a, b, D, phi=phi, psi=psi)
    assert oracle.rel_l2(M, ref) < TOL


def test_gram_phased_symmetric_plan(gpu):
    n = 2000
    a = anchors_with_ties(n, 10.0)
    phi = RNG.uniform(-np.pi, np.pi, n).astype(np.float32)
    psi = RNG.uniform(-np.pi, np.pi, n).astype(np.float32)
    D = RNG.uniform(0, 1, n).astype(np.float32)
    with lx.laplex_plan_create(dev(a), phi=dev(phi), psi=dev(psi)) as plan:
        M = host(lx.laplex_gram(plan, dev(D)))
    ref = oracle.gram_direct(a, a, D, phi=phi, psi=psi)
    assert oracle.rel_l2(M, ref) < TOL
    # a phased symmetric plan is still a real Gram: M = M^T
    assert np.allclose(M, M.T, rtol=1e-5, atol=1e-6 * np.abs(M).max())


def test_gram_phased_zero_temperature_diagonal(gpu):
    # anchors 1024 apart: A is a signed permutation, M diagonal with
    # M_ii = D_l cos^2(phi_i - psi_l) for the partner l of i
    n = 3000
    a = (1024.0 * RNG.permutation(n)).astype(np.float32)
    sigma = RNG.permutation(n)
    phi = RNG.uniform(-np.pi, np.pi, n).astype(np.float32)
    psi = RNG.uniform(-np.pi, np.pi, n).astype(np.float32)
    D = RNG.uniform(0, 1, n).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(a[sigma]), phi=dev(phi), psi=dev(psi)) as plan:
        M = host(lx.laplex_gram(plan, dev(D)))
    inv = np.argsort(sigma)  # b_l = a_{sigma_l}: partner of row i is l = inv[i]
    diag = D[inv].astype(np.float64) * np.cos(phi.astype(np.float64) - psi[inv].astype(np.float64)) ** 2
    off = M - np.diag(np.diag(M))
    assert np.all(off == 0)
    assert np.allclose(np.diag(M), diag, rtol=1e-5, atol=1e-7)


def test_gram_zero_temperature_diagonal(gpu):
    n = 3000
    a = (1024.0 * RNG.permutation(n)).astype(np.float32)
    sigma = RNG.permutation(n)
    D = RNG.uniform(0, 1, n).astype(np.float32)
    with lx.laplex_plan_create(dev(a), b=dev(a[sigma])) as plan:
        M = host(lx.laplex_gram(plan, dev(D)))
    ref = np.zeros((n, n), np.float32)
    ref[sigma, sigma] = D
    assert np.array_equal(M, ref)
