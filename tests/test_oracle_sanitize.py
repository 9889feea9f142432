"""The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer
(host code only): a driver calls every oracle entry point on small inputs
with ties, signed zeros, phases and temperatures 1, 1/2, 0, and checks the
sweeps against the dense definition.  A copy of the oracle with a planted
out-of-bounds read must be caught, so the build really is instrumented."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "oracle_sanitize_main.c")
ORACLE = os.path.join(ROOT, "oracle", "laplex_oracle.c")
FLAGS = ["-g", "-O1", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-fopenmp", "-Wall", "-Wextra"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")


def build(tmp_path, oracle_src):
    exe = str(tmp_path / "oracle_san")
    r = subprocess.run(["gcc", *FLAGS, "-o", exe, DRIVER, oracle_src, "-lm"], capture_output=True, text=True)
    if r.returncode != 0 and ("asan" in r.stderr.lower() or "ubsan" in r.stderr.lower()):
        pytest.skip("sanitizer runtimes not installed: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    return exe


@pytest.fixture(scope="module", autouse=True)
def need_gcc():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")


def test_oracle_clean_under_sanitizers(tmp_path):
    exe = build(tmp_path, ORACLE)
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout


def test_planted_overread_is_caught(tmp_path):
    src = open(ORACLE).read()
    needle = "for (int64_t i = 0; i < n; ++i)\n        if (!isfinite(a[i]))"
    assert src.count(needle) == 1
    bad = tmp_path / "oracle_overread.c"
    bad.write_text(src.replace(needle, needle.replace("i < n", "i <= n")))
    exe = build(tmp_path, str(bad))
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr
