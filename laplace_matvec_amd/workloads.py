"""Seeded synthetic inputs for the LAPLEX workloads.

This module holds only random-number generation and the workload recipes; it
contains none of the operator's arithmetic and imports neither the GPU
library's compute path nor the oracle, so both sides can consume what it
produces.

Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
numbers: as easy as 1, 2, 3", SC'11), counter-based.  Element ``i`` of a
stream keyed ``(key0, key1)`` takes word ``i % 4`` of the block computed for
counter ``(i // 4) = (c0 | c1 << 32), c2 = c3 = 0``.  The same definition is
implemented on the device in ``csrc/inputs_philox.hip`` for arrays too large
to generate on the host; both follow the conversions below:

* uniform u32 word w  -> u = w * 2^-32 in [0, 1) (exact in float64),
  value = float32(lo + (hi - lo) * u);
* normal: words (w0, w1) of one block give z0, z1 and (w2, w3) give z2, z3 by
  Box-Muller in float64: r = sqrt(-2 ln((w0 + 1) 2^-32)),
  t = 2 pi w1 2^-32, z0 = r cos t, z1 = r sin t; value = float32(mean + scale z).

Workloads (the benchmark's five configurations; sizes and distributions as
stated there) are built by :func:`config_inputs`.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85

# stream ids (second key word)
S_A, S_B, S_X, S_PHI, S_PSI, S_D, S_DUP_POS, S_DUP_SRC, S_W = 0, 1, 2, 3, 4, 5, 6, 7, 8

_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Vectorised Philox4x32 with 10 rounds.  Counters are uint32 arrays (or
    scalars); returns four uint32 arrays."""
    x0 = np.asarray(c0, dtype=np.uint64)
    x1 = np.asarray(c1, dtype=np.uint64)
    x2 = np.asarray(c2, dtype=np.uint64)
    x3 = np.asarray(c3, dtype=np.uint64)
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    x0, x1, x2, x3 = (v.copy() for v in (x0, x1, x2, x3))
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    key0, key1 = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for _ in range(10):
        p0 = m0 * x0
        p1 = m1 * x2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        x0, x1, x2, x3 = (hi1 ^ x1 ^ np.uint64(key0), lo1, hi0 ^ x3 ^ np.uint64(key1), lo0)
        key0 = (key0 + PHILOX_W0) & 0xFFFFFFFF
        key1 = (key1 + PHILOX_W1) & 0xFFFFFFFF
    return tuple(v.astype(np.uint32) for v in (x0, x1, x2, x3))


def _blocks(offset: int, n: int):
    """Philox blocks covering elements [offset, offset + n)."""
    b0 = offset // 4
    b1 = (offset + n + 3) // 4
    idx = np.arange(b0, b1, dtype=np.uint64)
    return b0, (idx & _MASK32).astype(np.uint32), (idx >> np.uint64(32)).astype(np.uint32)


def uniform_u32(n: int, key0: int, key1: int, offset: int = 0) -> np.ndarray:
    """Raw uint32 words of elements [offset, offset + n) of a stream."""
    b0, lo, hi = _blocks(offset, n)
    w = philox4x32_10(lo, hi, 0, 0, key0, key1)
    words = np.stack(w, axis=1).reshape(-1)
    s = offset - 4 * b0
    return words[s:s + n]


def uniform(n: int, key0: int, key1: int, lo: float, hi: float, offset: int = 0) -> np.ndarray:
    u = uniform_u32(n, key0, key1, offset).astype(np.float64) * 2.0 ** -32
    return (lo + (hi - lo) * u).astype(np.float32)


def normal(n: int, key0: int, key1: int, mean: float = 0.0, scale: float = 1.0,
           offset: int = 0) -> np.ndarray:
    b0, lo, hi = _blocks(offset, n)
    w0, w1, w2, w3 = (v.astype(np.float64) for v in philox4x32_10(lo, hi, 0, 0, key0, key1))
    two32 = 2.0 ** -32
    r01 = np.sqrt(-2.0 * np.log((w0 + 1.0) * two32))
    t01 = 2.0 * math.pi * (w1 * two32)
    r23 = np.sqrt(-2.0 * np.log((w2 + 1.0) * two32))
    t23 = 2.0 * math.pi * (w3 * two32)
    z = np.stack([r01 * np.cos(t01), r01 * np.sin(t01), r23 * np.cos(t23), r23 * np.sin(t23)],
                 axis=1).reshape(-1)
    s = offset - 4 * b0
    z = z[s:s + n]
    return (mean + scale * z).astype(np.float32)


def inject_duplicates(a: np.ndarray, key0: int, frac: float = 0.01) -> np.ndarray:
    """Overwrite floor(frac * n) seeded positions with copies of seeded other
    entries of the original array (later draws win on repeated positions)."""
    n = a.size
    m = int(math.floor(frac * n))
    if m == 0 or n < 2:
        return a.copy()
    pos = (uniform_u32(m, key0, S_DUP_POS).astype(np.uint64) * np.uint64(n)) >> np.uint64(32)
    src = (uniform_u32(m, key0, S_DUP_SRC).astype(np.uint64) * np.uint64(n)) >> np.uint64(32)
    # keep the last draw of each repeated position, explicitly
    pos = pos.astype(np.int64)
    src = src.astype(np.int64)
    _, first_in_reversed = np.unique(pos[::-1], return_index=True)
    last = m - 1 - first_in_reversed
    out = a.copy()
    out[pos[last]] = a[src[last]]
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark configuration: sizes and input distributions."""
    cfg: int
    name: str
    kind: str            # "sym", "general" or "gram"
    n: int
    k: int = 0
    batch: int = 1
    a_dist: tuple = ("normal", 0.0, 1.0)
    b_dist: tuple | None = None
    phased: bool = False
    dup_frac: float = 0.0
    note: str = ""


TWO_PI = 2.0 * math.pi

WORKLOADS = {
    1: Workload(1, "sym_n4096", "sym", 4096, batch=1, a_dist=("normal", 0.0, 8.0),
                note="symmetric, a ~ 8 N(0,1), x ~ N(0,1), one vector"),
    2: Workload(2, "sym_n2^24_b16_ties", "sym", 1 << 24, batch=16,
                a_dist=("uniform", 0.0, 0.05 * (1 << 24)), dup_frac=0.01,
                note="symmetric, a ~ U[0, 0.05 n] plus 1% exact duplicates, 16 vectors"),
    3: Workload(3, "general_n2^26_k1024_b64_phased", "general", 1 << 26, k=1024, batch=64,
                a_dist=("normal", 0.0, 100.0), b_dist=("uniform", -300.0, 300.0), phased=True,
                note="a ~ N(0,100^2), b ~ U[-300,300], phases U[0,2pi), 64 vectors, y=Kx and z=K^T w"),
    4: Workload(4, "gram_n4096_k3x2^20", "gram", 4096, k=3 << 20,
                a_dist=("normal", 0.0, 20.0), b_dist=("normal", 0.0, 20.0),
                note="weighted Gram, a, b ~ 20 N(0,1), D ~ U[0,1]"),
    5: Workload(5, "sym_n2^30", "sym", 1 << 30, batch=1, a_dist=("normal", 0.0, 1.0e4),
                note="symmetric, a ~ 1e4 N(0,1), x ~ N(0,1), one vector, end to end"),
}


def draw(dist: tuple, n: int, key0: int, key1: int, offset: int = 0) -> np.ndarray:
    kind, p, q = dist
    if kind == "normal":
        return normal(n, key0, key1, mean=p, scale=q, offset=offset)
    if kind == "uniform":
        return uniform(n, key0, key1, p, q, offset=offset)
    raise ValueError(kind)


def config_inputs(cfg: int, n: int | None = None, k: int | None = None,
                  batch: int | None = None) -> dict:
    """Host (numpy) inputs of a configuration, optionally at reduced sizes
    with the same distributions (for tests that the oracle must finish).

    Returns a dict with float32 arrays: ``a`` and, as the workload needs,
    ``b``, ``phi``, ``psi``, ``x`` ([batch][k or n]), ``w`` ([batch][n]), ``D``."""
    wl = WORKLOADS[cfg]
    n = wl.n if n is None else n
    k = wl.k if k is None else k
    batch = wl.batch if batch is None else batch
    out = {"a": draw(wl.a_dist, n, cfg, S_A)}
    if wl.dup_frac:
        out["a"] = inject_duplicates(out["a"], cfg, wl.dup_frac)
    if wl.kind == "sym":
        out["x"] = normal(batch * n, cfg, S_X).reshape(batch, n)
    elif wl.kind == "general":
        out["b"] = draw(wl.b_dist, k, cfg, S_B)
        out["x"] = normal(batch * k, cfg, S_X).reshape(batch, k)
        out["w"] = normal(batch * n, cfg, S_W).reshape(batch, n)
    elif wl.kind == "gram":
        out["b"] = draw(wl.b_dist, k, cfg, S_B)
        out["D"] = uniform(k, cfg, S_D, 0.0, 1.0)
    if wl.phased:
        out["phi"] = uniform(n, cfg, S_PHI, 0.0, TWO_PI)
        out["psi"] = uniform(k if wl.kind == "general" else n, cfg, S_PSI, 0.0, TWO_PI)
    return out


# --------------------------------------------------------------- device side

_gen_lib = None


def _gen():
    """liblaplex_inputs.so: the same Philox streams drawn on the GPU."""
    global _gen_lib
    if _gen_lib is None:
        import ctypes
        import os
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblaplex_inputs.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build the package first")
        lib = ctypes.CDLL(path)
        lib.laplex_inputs_generate.restype = ctypes.c_int
        lib.laplex_inputs_generate.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int,
                                               ctypes.c_double, ctypes.c_double, ctypes.c_void_p]
        lib.laplex_inputs_copy.restype = ctypes.c_int
        lib.laplex_inputs_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        _gen_lib = lib
    return _gen_lib


def device_copy(src, dst) -> None:
    """dst[:] = src through the input library's plain copy kernel (one
    dispatch, 4-byte accesses): the known-size reference of the HBM traffic
    counters.  Both are contiguous device tensors of 4-byte elements."""
    import ctypes
    import torch
    if src.numel() != dst.numel() or src.element_size() != 4 or dst.element_size() != 4:
        raise ValueError("device_copy: same number of 4-byte elements needed")
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("device_copy: contiguous tensors needed")
    rc = _gen().laplex_inputs_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                   src.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"laplex_inputs_copy failed ({rc})")


def _device_draw(shape, key0, key1, kind, p, q, device, dtype=None):
    import ctypes
    import torch
    dtype = dtype or torch.float32
    out = torch.empty(shape, dtype=dtype, device=device)
    if out.numel():
        rc = _gen().laplex_inputs_generate(ctypes.c_void_p(out.data_ptr()), out.numel(), 0, key0, key1,
                                           kind, float(p), float(q),
                                           ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream))
        if rc != 0:
            raise RuntimeError(f"device input generator failed ({rc})")
    return out


def device_normal(shape, key0, key1, mean=0.0, scale=1.0, device="cuda"):
    return _device_draw(shape, key0, key1, 0, mean, scale, device)


def device_uniform(shape, key0, key1, lo, hi, device="cuda"):
    return _device_draw(shape, key0, key1, 1, lo, hi, device)


def device_u32(shape, key0, key1, device="cuda"):
    import torch
    return _device_draw(shape, key0, key1, 2, 0.0, 0.0, device, dtype=torch.int32)


def device_draw(dist, shape, key0, key1, device="cuda"):
    kind, p, q = dist
    if kind == "normal":
        return device_normal(shape, key0, key1, p, q, device)
    return device_uniform(shape, key0, key1, p, q, device)


def device_config_inputs(cfg: int, n: int | None = None, k: int | None = None,
                         batch: int | None = None, device="cuda", with_w: bool = True) -> dict:
    """The inputs of :func:`config_inputs`, drawn on the GPU (same streams).

    Duplicate injection (config 2) runs on the host copy of the anchors."""
    import torch
    wl = WORKLOADS[cfg]
    n = wl.n if n is None else n
    k = wl.k if k is None else k
    batch = wl.batch if batch is None else batch
    out = {"a": device_draw(wl.a_dist, (n,), cfg, S_A, device)}
    if wl.dup_frac:
        host = inject_duplicates(out["a"].cpu().numpy(), cfg, wl.dup_frac)
        out["a"] = torch.from_numpy(host).to(device)
    if wl.kind == "sym":
        out["x"] = device_normal((batch, n), cfg, S_X, device=device)
    elif wl.kind == "general":
        out["b"] = device_draw(wl.b_dist, (k,), cfg, S_B, device)
        out["x"] = device_normal((batch, k), cfg, S_X, device=device)
        if with_w:
            out["w"] = device_normal((batch, n), cfg, S_W, device=device)
    elif wl.kind == "gram":
        out["b"] = device_draw(wl.b_dist, (k,), cfg, S_B, device)
        out["D"] = device_uniform((k,), cfg, S_D, 0.0, 1.0, device)
    if wl.phased:
        out["phi"] = device_uniform((n,), cfg, S_PHI, 0.0, TWO_PI, device)
        out["psi"] = device_uniform((k if wl.kind == "general" else n,), cfg, S_PSI, 0.0, TWO_PI, device)
    return out
