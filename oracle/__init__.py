"""fp64 CPU oracle for the LAPLEX operator -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in the package entry module and the
CPU-baseline leg of the benchmark may import this package.  The GPU product
path never imports it and shares no code with it.

The arithmetic lives in ``laplex_oracle.c`` (plain C, double precision); this
module only builds that file with gcc and marshals numpy arrays through
ctypes.  Semantics follow the technical summary of "LAPLEX: The FFT of
Learnable Laplace Kernels" (§2.1 operator, §2.2 scan algebra and Gram):

* symmetric operator (``b is None``): K = LAPLEX(a, phi; a, psi), n x n;
  ``transpose=True`` applies K^T, i.e. swaps the roles of phi and psi;
* general operator: K = LAPLEX(a, phi; b, psi), n x k; ``transpose=False``
  maps x in R^k to y in R^n, ``transpose=True`` maps w in R^n to z in R^k.

Every function takes the temperature ``t`` (entries exp(-|a - b| / t));
``t = 1`` is the printed operator, ``t = 0`` the equality-routing limit.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "laplex_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liblaplex_oracle.so")
_lib = None

OK, NONFINITE, BADARG, NOMEM = 0, 1, 2, 3


class OracleError(RuntimeError):
    pass


def build() -> str:
    """Compile the oracle with gcc (no HIP headers, no GPU code)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.lo_argsort.argtypes = [vp, i64, vp]
    f64 = ctypes.c_double
    lib.lo_apply_dense.argtypes = [vp, vp, i64, vp, vp, i64, vp, i64, vp, i64, f64, vp]
    lib.lo_dense_matrix.argtypes = [vp, vp, i64, vp, vp, i64, f64, vp]
    lib.lo_apply_sym_sweep.argtypes = [vp, vp, vp, i64, vp, i64, f64, vp]
    lib.lo_apply_general_sweep.argtypes = [vp, vp, i64, vp, vp, i64, vp, i64, f64, vp]
    lib.lo_gram_direct.argtypes = [vp, vp, i64, vp, vp, i64, vp, vp, i64, vp, i64, f64, vp]
    lib.lo_grad_dense.argtypes = [vp, vp, i64, vp, vp, i64, f64, vp, vp, i64, vp, i64, vp, i64,
                                  vp, vp, vp, vp]
    for f in (lib.lo_argsort, lib.lo_apply_dense, lib.lo_dense_matrix, lib.lo_apply_sym_sweep,
              lib.lo_apply_general_sweep, lib.lo_gram_direct, lib.lo_grad_dense, lib.lo_num_threads):
        f.restype = ctypes.c_int
    lib.lo_num_threads.argtypes = []
    _lib = lib
    return lib


def _f32(v):
    if v is None:
        return None
    return np.ascontiguousarray(np.asarray(v, dtype=np.float32))


def _ptr(arr):
    return None if arr is None else arr.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != OK:
        names = {NONFINITE: "non-finite anchor", BADARG: "bad argument", NOMEM: "out of memory"}
        raise OracleError(f"{what}: {names.get(rc, rc)}")


def num_threads() -> int:
    return int(_load().lo_num_threads())


def argsort(a) -> np.ndarray:
    """Stable ascending argsort under the IEEE total order (-0.0 < +0.0)."""
    a = _f32(a)
    perm = np.empty(a.size, dtype=np.uint32)
    _check(_load().lo_argsort(_ptr(a), a.size, _ptr(perm)), "argsort")
    return perm


def _sides(a, b, phi, psi, transpose):
    """(out_anchor, out_phase, in_anchor, in_phase) for K or K^T."""
    if b is None:
        b = a
    if transpose:
        return b, psi, a, phi
    return a, phi, b, psi


def _temp(t) -> float:
    t = float(t)
    if not (t >= 0.0) or t == float("inf"):
        raise ValueError("temperature must be finite and >= 0")
    return t


def apply_dense(a, x, b=None, phi=None, psi=None, transpose=False, rows=None, t=1.0) -> np.ndarray:
    """Definition (summary §2.1): y = K x entry by entry, O(n k) per vector.

    x is [batch][n_in] (or 1-D); returns float64 [batch][n_rows] (or 1-D).
    ``rows`` restricts the computation to the listed output indices."""
    a, b, phi, psi = _f32(a), _f32(b), _f32(phi), _f32(psi)
    if (phi is None) != (psi is None):
        raise ValueError("phases: give both phi and psi or neither")
    oa, op, ia, ip = _sides(a, b, phi, psi, transpose)
    x = _f32(x)
    one = x.ndim == 1
    x2 = x.reshape(1, -1) if one else x
    if x2.shape[1] != ia.size:
        raise ValueError("x has the wrong length")
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    m = oa.size if r is None else r.size
    y = np.empty((x2.shape[0], m), dtype=np.float64)
    rc = _load().lo_apply_dense(_ptr(oa), _ptr(op), oa.size, _ptr(ia), _ptr(ip), ia.size,
                                _ptr(x2), x2.shape[0], _ptr(r), 0 if r is None else r.size,
                                _temp(t), _ptr(y))
    _check(rc, "apply_dense")
    return y[0] if one else y


def dense_matrix(a, b=None, phi=None, psi=None, transpose=False, t=1.0) -> np.ndarray:
    """The full matrix K (or K^T) by its definition, float64."""
    a, b, phi, psi = _f32(a), _f32(b), _f32(phi), _f32(psi)
    oa, op, ia, ip = _sides(a, b, phi, psi, transpose)
    K = np.empty((oa.size, ia.size), dtype=np.float64)
    _check(_load().lo_dense_matrix(_ptr(oa), _ptr(op), oa.size, _ptr(ia), _ptr(ip), ia.size,
                                   _temp(t), _ptr(K)), "dense_matrix")
    return K


def apply_sweep(a, x, b=None, phi=None, psi=None, transpose=False, t=1.0) -> np.ndarray:
    """Sort + prefix/suffix recurrences (summary §2.2), float64 result.

    Symmetric operators use the two-sweep form (L + U - x); general ones the
    interval bucketing into u, v followed by the same two recurrences."""
    a, b, phi, psi = _f32(a), _f32(b), _f32(phi), _f32(psi)
    if (phi is None) != (psi is None):
        raise ValueError("phases: give both phi and psi or neither")
    x = _f32(x)
    one = x.ndim == 1
    x2 = x.reshape(1, -1) if one else x
    lib = _load()
    if b is None:
        po, pi = (psi, phi) if transpose else (phi, psi)
        if x2.shape[1] != a.size:
            raise ValueError("x has the wrong length")
        y = np.empty((x2.shape[0], a.size), dtype=np.float64)
        rc = lib.lo_apply_sym_sweep(_ptr(a), _ptr(po), _ptr(pi), a.size, _ptr(x2), x2.shape[0],
                                    _temp(t), _ptr(y))
        _check(rc, "apply_sym_sweep")
    else:
        oa, op, ia, ip = _sides(a, b, phi, psi, transpose)
        if x2.shape[1] != ia.size:
            raise ValueError("x has the wrong length")
        y = np.empty((x2.shape[0], oa.size), dtype=np.float64)
        rc = lib.lo_apply_general_sweep(_ptr(oa), _ptr(op), oa.size, _ptr(ia), _ptr(ip), ia.size,
                                        _ptr(x2), x2.shape[0], _temp(t), _ptr(y))
        _check(rc, "apply_general_sweep")
    return y[0] if one else y


def gram_direct(a, b, D, rows=None, cols=None, phi=None, psi=None, t=1.0) -> np.ndarray:
    """M = A diag(D) A^T with A = K(a, phi; b, psi), entry by entry in O(k)
    (summary §2.2, Gram operators).  rows/cols select original indices of a."""
    a, b, D, phi, psi = _f32(a), _f32(b), _f32(D), _f32(phi), _f32(psi)
    if (phi is None) != (psi is None):
        raise ValueError("phases: give both phi and psi or neither")
    if D.size != b.size:
        raise ValueError("D must have one weight per b anchor")
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    c = None if cols is None else np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    mr = a.size if r is None else r.size
    mc = a.size if c is None else c.size
    M = np.empty((mr, mc), dtype=np.float64)
    rc = _load().lo_gram_direct(_ptr(a), _ptr(phi), a.size, _ptr(b), _ptr(psi), b.size, _ptr(D), _ptr(r),
                                0 if r is None else r.size, _ptr(c), 0 if c is None else c.size,
                                _temp(t), _ptr(M))
    _check(rc, "gram_direct")
    return M


def grad_dense(a, u, w, b=None, phi=None, psi=None, t=1.0, rows=None, cols=None) -> dict:
    """Gradients of F = sum_v <u_v, K w_v> with respect to the anchors and
    phases, from the entrywise derivatives of the definition (summary §2.1).

    u is [batch][n] (row side), w is [batch][k] (column side).  For y = K x
    with upstream gradient g pass u = g, w = x; for y = K^T x pass u = x,
    w = g.  Returns float64 arrays {"da", "db", "dphi", "dpsi"} (phase
    entries only for a phased operator).  Symmetric operator (b is None):
    b := a, so the anchor gradient is the sum of both sides and "db" is
    absent; "dpsi" is still its own parameter.  rows/cols select indices of
    a (da, dphi) and of b (db, dpsi); symmetric: rows selects both."""
    sym = b is None
    a, phi, psi = _f32(a), _f32(phi), _f32(psi)
    b = a if sym else _f32(b)
    if (phi is None) != (psi is None):
        raise ValueError("phases: give both phi and psi or neither")
    u, w = _f32(u), _f32(w)
    u2 = u.reshape(1, -1) if u.ndim == 1 else u
    w2 = w.reshape(1, -1) if w.ndim == 1 else w
    if u2.shape[1] != a.size or w2.shape[1] != b.size or u2.shape[0] != w2.shape[0]:
        raise ValueError("u must be [batch][n] and w [batch][k]")
    r = None if rows is None else np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    if sym:
        c = r
    else:
        c = None if cols is None else np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    mr = a.size if r is None else r.size
    mc = b.size if c is None else c.size
    phased = phi is not None
    da, db = np.empty(mr), np.empty(mc)
    dphi = np.empty(mr) if phased else None
    dpsi = np.empty(mc) if phased else None
    rc = _load().lo_grad_dense(_ptr(a), _ptr(phi), a.size, _ptr(b), _ptr(psi), b.size, _temp(t),
                               _ptr(u2), _ptr(w2), u2.shape[0], _ptr(r), 0 if r is None else r.size,
                               _ptr(c), 0 if c is None else c.size, _ptr(da), _ptr(db),
                               _ptr(dphi), _ptr(dpsi))
    _check(rc, "grad_dense")
    out = {"da": da + db if sym else da}
    if not sym:
        out["db"] = db
    if phased:
        out["dphi"] = dphi
        out["dpsi"] = dpsi
    return out


def rel_l2(y, ref) -> float:
    """Relative L2 error ||y - ref|| / ||ref||, accumulated in float64."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((y - ref).ravel())
    return float(num / den) if den > 0 else float(num)
