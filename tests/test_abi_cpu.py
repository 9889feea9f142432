"""CPU-only checks of the C ABI: the library loads, exports every entry point
that include/laplex.h declares, and rejects invalid arguments on the host
before any HIP call.  Also checks that the product path does not reach the
oracle."""
import ctypes
import os
import re

import pytest

from laplace_matvec_amd import laplex as lx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "laplex.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(laplex_[a-z_]+)\s*\(", text)))


def test_header_lists_expected_calls():
    names = header_functions()
    for required in ("laplex_plan_create", "laplex_apply", "laplex_gram", "laplex_plan_destroy"):
        assert required in names


def test_library_exports_every_header_function():
    lib = lx.load()
    for name in header_functions():
        assert hasattr(lib, name), name
        assert name in lx.SIGNATURES, f"binding lacks {name}"


def test_inputs_library_exports_generator():
    lib = ctypes.CDLL(os.path.join(ROOT, "laplace_matvec_amd", "liblaplex_inputs.so"))
    assert hasattr(lib, "laplex_inputs_generate")


def _create(a, n, b, k, phi, psi):
    lib = lx.load()
    h = ctypes.c_void_p(12345)
    st = lib.laplex_plan_create(ctypes.byref(h), a, n, b, k, phi, psi, None)
    return st, h.value


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: checks run first


@pytest.mark.parametrize("args", [
    (None, 10, None, 0, None, None),                 # a NULL
    (FAKE, 0, None, 0, None, None),                  # n < 1
    (FAKE, 1 << 31, None, 0, None, None),            # n too large for uint32 permutations
    (FAKE, (1 << 30) + 1, None, 0, None, None),      # n past 2^30 (32-bit byte offsets)
    (FAKE, 10, None, 5, None, None),                 # symmetric with k != n
    (FAKE, 10, FAKE, 0, None, None),                 # general with k < 1
    (FAKE, 10, FAKE, 1 << 31, None, None),           # k too large
    (FAKE, 10, FAKE, (1 << 30) + 1, None, None),     # k past 2^30
    (FAKE, (1 << 30) + 1, FAKE, 10, None, None),     # general plan, n past 2^30
    (FAKE, 10, None, 0, FAKE, None),                 # phi without psi
    (FAKE, 10, None, 0, None, FAKE),                 # psi without phi
])
def test_plan_create_rejects_bad_arguments(args):
    st, h = _create(*args)
    assert st == lx.ERR_INVALID_ARGUMENT
    assert h is None  # *out set to NULL on error
    assert lx.load().laplex_last_error()


def test_plan_create_null_out():
    assert lx.load().laplex_plan_create(None, FAKE, 10, None, 0, None, None, None) == lx.ERR_INVALID_ARGUMENT


def test_apply_and_gram_reject_bad_arguments():
    lib = lx.load()
    assert lib.laplex_apply(None, FAKE, FAKE, 1, 0, None) == lx.ERR_INVALID_ARGUMENT
    assert lib.laplex_gram(None, FAKE, FAKE, None) == lx.ERR_INVALID_ARGUMENT
    assert lib.laplex_plan_destroy(None) == lx.OK
    assert lib.laplex_plan_set_option(None, 1, 0) == lx.ERR_INVALID_ARGUMENT
    assert lib.laplex_plan_info(None, None, None, None) == lx.ERR_INVALID_ARGUMENT
    assert lib.laplex_plan_set_temperature(None, 1.0) == lx.ERR_INVALID_ARGUMENT
    h = ctypes.c_void_p(1)
    assert lib.laplex_plan_create_apply(ctypes.byref(h), FAKE, 10, None, None, None, FAKE, 1, None) == \
        lx.ERR_INVALID_ARGUMENT and h.value is None
    assert lib.laplex_plan_create_apply(ctypes.byref(h), FAKE, 10, None, None, FAKE, FAKE, 1, None) == \
        lx.ERR_INVALID_ARGUMENT  # x and y overlap
    assert lib.laplex_plan_create_apply(ctypes.byref(h), FAKE, 10, None, None, FAKE, ctypes.c_void_p(0x9000), 0,
                                        None) == lx.ERR_INVALID_ARGUMENT
    big = (1 << 30) + 1  # past the longest side
    assert lib.laplex_plan_create_apply(ctypes.byref(h), FAKE, big, None, None, ctypes.c_void_p(1 << 44),
                                        ctypes.c_void_p(1 << 45), 1, None) == lx.ERR_INVALID_ARGUMENT
    assert lib.laplex_backward(None, FAKE, FAKE, 1, 0, FAKE, None, None, None, None, None) == \
        lx.ERR_INVALID_ARGUMENT
    for s in range(7):
        assert lib.laplex_status_str(s)


def test_profile_label_filter_host_side():
    # host state only: no launch, no event; set, clear, and read back nothing
    lx.profile_only("sort_pass")
    lx.profile_only(None)
    lx.profile_only("")
    lib = lx.load()
    assert lib.laplex_profile_enable(0) == lx.OK
    assert lib.laplex_profile_reset() == lx.OK
    assert lx.profile_read() == {}


def test_valid_arguments_without_gpu_report_no_device():
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is visible here")
    except Exception:
        pass
    st, h = _create(FAKE, 10, None, 0, None, None)
    assert st == lx.ERR_NO_DEVICE and h is None


def test_product_path_never_imports_oracle():
    pkg = os.path.join(ROOT, "laplace_matvec_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "laplex_oracle" not in text, f
                assert "lo_apply" not in text and "lo_argsort" not in text, f


def test_oracle_shares_no_code_with_gpu_path():
    src = open(os.path.join(ROOT, "oracle", "laplex_oracle.c")).read()
    assert '#include "lx_' not in src and "#include <hip" not in src
