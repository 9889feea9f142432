"""Thin ctypes binding of liblaplex.so (C ABI in include/laplex.h).

Argument marshalling only: every step of the operator runs in the HIP
library.  PyTorch supplies device memory and the current stream.  If the
library is missing this module raises on import of any entry point; there
is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblaplex.so")

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_NONFINITE_ANCHOR = 2
ERR_OUT_OF_MEMORY = 3
ERR_UNSUPPORTED = 4
ERR_DEVICE = 5
ERR_NO_DEVICE = 6

OPT_GENERAL_ALGO = 1
ALGO_AUTO, ALGO_BUCKET, ALGO_EVALUATE = 0, 1, 2
PLAN_SYMMETRIC, PLAN_PHASED = 1, 2

# every entry point of include/laplex.h: name -> (restype, argtypes)
_VP, _I64, _I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "laplex_plan_create": (_I32, [ctypes.POINTER(_VP), _VP, _I64, _VP, _I64, _VP, _VP, _VP]),
    "laplex_plan_create_apply": (_I32, [ctypes.POINTER(_VP), _VP, _I64, _VP, _VP, _VP, _VP, _I64, _VP]),
    "laplex_apply": (_I32, [_VP, _VP, _VP, _I64, _I32, _VP]),
    "laplex_apply_noalloc": (_I32, [_VP, _VP, _VP, _I64, _I32, _VP]),
    "laplex_gram": (_I32, [_VP, _VP, _VP, _VP]),
    "laplex_plan_destroy": (_I32, [_VP]),
    "laplex_plan_perm": (_I32, [_VP, _I32, ctypes.POINTER(_VP)]),
    "laplex_plan_sorted": (_I32, [_VP, _I32, ctypes.POINTER(_VP)]),
    "laplex_plan_info": (_I32, [_VP, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I32)]),
    "laplex_plan_set_option": (_I32, [_VP, _I32, _I64]),
    "laplex_plan_set_temperature": (_I32, [_VP, ctypes.c_double]),
    "laplex_backward": (_I32, [_VP, _VP, _VP, _I64, _I32, _VP, _VP, _VP, _VP, _VP, _VP]),
    "laplex_profile_enable": (_I32, [_I32]),
    "laplex_profile_only": (_I32, [ctypes.c_char_p]),
    "laplex_profile_reset": (_I32, []),
    "laplex_profile_collect": (_I32, []),
    "laplex_profile_entry": (_I32, [_I32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(_I64),
                                    ctypes.POINTER(ctypes.c_double)]),
    "laplex_status_str": (ctypes.c_char_p, [_I32]),
    "laplex_last_error": (ctypes.c_char_p, []),
}

_lib = None


class LaplexError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        lib = load()
        msg = lib.laplex_status_str(status).decode()
        detail = lib.laplex_last_error().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))


def load():
    """Load liblaplex.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run laplace_matvec_amd/build.py "
                               "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _check(st: int, where: str):
    if st != OK:
        raise LaplexError(st, where)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _dev_f32(t, name):
    if t is None:
        return None
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous float32 CUDA tensor")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class Plan:
    """A sorted LAPLEX operator K = LAPLEX(a, phi; b, psi) (n x k)."""

    def __init__(self, handle, n, k, symmetric, phased, device):
        self.handle = handle
        self.n, self.k = n, k
        self.symmetric, self.phased = symmetric, phased
        self.device = device

    def destroy(self):
        if self.handle:
            _check(load().laplex_plan_destroy(self.handle), "laplex_plan_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()


def laplex_plan_create(a, b=None, phi=None, psi=None, stream=None) -> Plan:
    a = _dev_f32(a, "a")
    b = _dev_f32(b, "b")
    phi = _dev_f32(phi, "phi")
    psi = _dev_f32(psi, "psi")
    h = ctypes.c_void_p()
    st = load().laplex_plan_create(ctypes.byref(h), _ptr(a), a.numel(), _ptr(b),
                                   0 if b is None else b.numel(), _ptr(phi), _ptr(psi), _stream(stream))
    _check(st, "laplex_plan_create")
    k = a.numel() if b is None else b.numel()
    return Plan(h, a.numel(), k, b is None, phi is not None, a.device)


def laplex_plan_create_apply(a, x, y=None, phi=None, psi=None, stream=None):
    """Symmetric plan and y = K x in one call; returns (plan, y)."""
    a = _dev_f32(a, "a")
    phi = _dev_f32(phi, "phi")
    psi = _dev_f32(psi, "psi")
    x = _dev_f32(x, "x")
    n = a.numel()
    one = x.dim() == 1
    batch = 1 if one else x.shape[0]
    if x.shape[-1] != n or x.dim() > 2:
        raise ValueError(f"x must have shape [batch][{n}]")
    if y is None:
        y = torch.empty_like(x)
    y = _dev_f32(y, "y")
    if y.numel() != batch * n:
        raise ValueError("y has the wrong size")
    h = ctypes.c_void_p()
    st = load().laplex_plan_create_apply(ctypes.byref(h), _ptr(a), n, _ptr(phi), _ptr(psi), _ptr(x), _ptr(y),
                                         batch, _stream(stream))
    _check(st, "laplex_plan_create_apply")
    return Plan(h, n, n, True, phi is not None, a.device), y


def laplex_apply(plan: Plan, x, y=None, transpose: bool = False, stream=None):
    """y = K x (transpose False) or K^T x; x is [batch][in] or 1-D."""
    x = _dev_f32(x, "x")
    n_in, n_out = (plan.n, plan.k) if transpose else (plan.k, plan.n)
    one = x.dim() == 1
    batch = 1 if one else x.shape[0]
    if x.shape[-1] != n_in or x.dim() > 2:
        raise ValueError(f"x must have shape [batch][{n_in}]")
    if y is None:
        y = torch.empty((n_out,) if one else (batch, n_out), dtype=torch.float32, device=x.device)
    y = _dev_f32(y, "y")
    if y.numel() != batch * n_out:
        raise ValueError("y has the wrong size")
    _check(load().laplex_apply(plan.handle, _ptr(x), _ptr(y), batch, int(bool(transpose)), _stream(stream)),
           "laplex_apply")
    return y


def laplex_apply_noalloc(plan: Plan, x, y, transpose: bool = False, stream=None):
    """laplex_apply into a caller-provided y, with the library's fixed
    scratch instead of any allocation (see include/laplex.h)."""
    x = _dev_f32(x, "x")
    y = _dev_f32(y, "y")
    n_in, n_out = (plan.n, plan.k) if transpose else (plan.k, plan.n)
    batch = 1 if x.dim() == 1 else x.shape[0]
    if x.shape[-1] != n_in or x.dim() > 2 or y.numel() != batch * n_out:
        raise ValueError(f"x must be [batch][{n_in}] and y [batch][{n_out}]")
    _check(load().laplex_apply_noalloc(plan.handle, _ptr(x), _ptr(y), batch, int(bool(transpose)),
                                       _stream(stream)), "laplex_apply_noalloc")
    return y


def laplex_gram(plan: Plan, D, M=None, stream=None):
    D = _dev_f32(D, "D")
    if D.numel() != plan.k:
        raise ValueError(f"D must have {plan.k} entries")
    if M is None:
        M = torch.empty((plan.n, plan.n), dtype=torch.float32, device=D.device)
    M = _dev_f32(M, "M")
    _check(load().laplex_gram(plan.handle, _ptr(D), _ptr(M), _stream(stream)), "laplex_gram")
    return M


def laplex_plan_set_option(plan: Plan, option: int, value: int):
    _check(load().laplex_plan_set_option(plan.handle, option, value), "laplex_plan_set_option")


def laplex_plan_set_temperature(plan: Plan, t: float):
    """Entries exp(-|a_i - b_j| / t); t = 0 routes by exact anchor equality."""
    _check(load().laplex_plan_set_temperature(plan.handle, float(t)), "laplex_plan_set_temperature")


def laplex_backward(plan: Plan, x, g, transpose: bool = False, want=("dx", "da", "db", "dphi", "dpsi"),
                    stream=None) -> dict:
    """Gradients of a step through y = K x (or K^T x): x the forward input
    (None for a plan from laplex_plan_create_apply, which kept it), g = dL/dy.  Returns the requested tensors among dx ([batch][in]), da [n],
    db [k] (general plans), dphi [n], dpsi [k] (phased plans); entries a plan
    does not have are left out."""
    g = _dev_f32(g, "g")
    n_in, n_out = (plan.n, plan.k) if transpose else (plan.k, plan.n)
    if x is None:  # the input kept by laplex_plan_create_apply
        shape = (n_in,) if g.dim() == 1 else (g.shape[0], n_in)
    else:
        x = _dev_f32(x, "x")
        shape = tuple(x.shape)
        if x.shape[-1] != n_in or x.dim() > 2:
            raise ValueError(f"x must have shape [batch][{n_in}]")
    batch = 1 if len(shape) == 1 else shape[0]
    if g.numel() != batch * n_out or g.shape[-1] != n_out:
        raise ValueError(f"g must have shape [batch][{n_out}]")
    dev = g.device
    out = {}
    if "dx" in want:
        out["dx"] = torch.empty(shape, dtype=torch.float32, device=dev)
    if "da" in want:
        out["da"] = torch.empty(plan.n, dtype=torch.float32, device=dev)
    if "db" in want and not plan.symmetric:
        out["db"] = torch.empty(plan.k, dtype=torch.float32, device=dev)
    if plan.phased:
        if "dphi" in want:
            out["dphi"] = torch.empty(plan.n, dtype=torch.float32, device=dev)
        if "dpsi" in want:
            out["dpsi"] = torch.empty(plan.k, dtype=torch.float32, device=dev)
    p = [_ptr(out.get(k)) for k in ("dx", "da", "db", "dphi", "dpsi")]
    _check(load().laplex_backward(plan.handle, _ptr(x), _ptr(g), batch, int(bool(transpose)), *p,
                                  _stream(stream)), "laplex_backward")
    return out


def _copy_device(dst: torch.Tensor, src_ptr: int, nbytes: int, stream=None):
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.restype = ctypes.c_int
    hip.hipMemcpyAsync.argtypes = [_VP, _VP, ctypes.c_size_t, ctypes.c_int, _VP]
    rc = hip.hipMemcpyAsync(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src_ptr), nbytes, 3,  # D2D
                            _stream(stream))
    if rc != 0:
        raise RuntimeError(f"hipMemcpyAsync failed ({rc})")


def laplex_plan_perm(plan: Plan, side: int = 0, stream=None) -> torch.Tensor:
    """Copy of the plan's permutation (rank -> original index) as int64."""
    p = ctypes.c_void_p()
    _check(load().laplex_plan_perm(plan.handle, side, ctypes.byref(p)), "laplex_plan_perm")
    m = plan.n if side == 0 else plan.k
    out = torch.empty(m, dtype=torch.int32, device=plan.device)
    _copy_device(out, p.value, 4 * m, stream)
    return out.to(torch.int64)  # indices are below 2^31


def laplex_plan_sorted(plan: Plan, side: int = 0, stream=None) -> torch.Tensor:
    p = ctypes.c_void_p()
    _check(load().laplex_plan_sorted(plan.handle, side, ctypes.byref(p)), "laplex_plan_sorted")
    m = plan.n if side == 0 else plan.k
    out = torch.empty(m, dtype=torch.float32, device=plan.device)
    _copy_device(out, p.value, 4 * m, stream)
    return out


def laplex_plan_info(plan: Plan):
    n, k, f = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
    _check(load().laplex_plan_info(plan.handle, ctypes.byref(n), ctypes.byref(k), ctypes.byref(f)),
           "laplex_plan_info")
    return n.value, k.value, f.value


def laplex_plan_destroy(plan: Plan):
    plan.destroy()


# ---- kernel timing -------------------------------------------------------

def profile_enable(on: bool = True):
    load().laplex_profile_enable(int(on))


def profile_only(label: str | None = None):
    """Bracket only launches labelled `label` (None: every launch)."""
    load().laplex_profile_only(None if label is None else label.encode())


def profile_reset():
    load().laplex_profile_reset()


def profile_read() -> dict:
    """Collect pending events; returns {kernel name: (launches, total ms)}."""
    lib = load()
    _check(lib.laplex_profile_collect(), "laplex_profile_collect")
    out = {}
    i = 0
    while True:
        name, cnt, ms = ctypes.c_char_p(), ctypes.c_int64(), ctypes.c_double()
        if lib.laplex_profile_entry(i, ctypes.byref(name), ctypes.byref(cnt), ctypes.byref(ms)) != OK:
            break
        out[name.value.decode()] = (cnt.value, ms.value)
        i += 1
    return out
