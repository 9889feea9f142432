"""The bucketed dense rows used at full size equal the oracle's full dense
rows (CPU)."""
import numpy as np

import oracle
from dense_near import dense_rows_near


def test_dense_rows_near_is_the_dense_row():
    """2^16 anchors spread so that most pairs are more than 746 apart: the
    bucketed rows equal the full dense rows to float64 rounding, also with a
    bucket width that needs eight neighbouring buckets on each side."""
    rng = np.random.default_rng(8)
    a = (rng.standard_normal(1 << 16) * 3000).astype(np.float32)
    x = rng.standard_normal(1 << 16).astype(np.float32)
    rows = np.array([0, 5, 777, 40000, 65535, int(np.argmin(a)), int(np.argmax(a))])
    full = oracle.apply_dense(a, x, rows=rows)
    for width in (100.0, 256.0, 1000.0):
        near = dense_rows_near(a, x, rows, width=width)
        assert np.allclose(near, full, rtol=1e-13, atol=1e-13 * np.abs(full).max()), width


def test_reach_is_where_the_terms_vanish():
    """Anchors 744 apart still interact (e^-744 is a nonzero subnormal) and
    the bucketed row keeps that term; 747 apart the dense term is exactly 0."""
    x = np.array([0.0, 1.0], dtype=np.float32)
    near_pair = np.array([0.0, 744.0], dtype=np.float32)
    full = oracle.apply_dense(near_pair, x, rows=np.array([0]))
    assert full[0] > 0.0
    assert np.array_equal(dense_rows_near(near_pair, x, np.array([0])), full)
    far_pair = np.array([0.0, 747.0], dtype=np.float32)
    assert oracle.apply_dense(far_pair, x, rows=np.array([0]))[0] == 0.0
