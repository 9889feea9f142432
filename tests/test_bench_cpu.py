"""Host logic of bench.py, on the CPU: the one-GPU refusal, the byte model
of a symmetric step, and the pinning of committed rocprofv3 counter records
to the hash of the kernel source they were taken from."""
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_step_byte_model_symmetric_one_vector():
    b = load_bench()
    n = 1 << 30
    # histogram 4; four radix passes with x as a value row: 10 + 8 + the tile
    # table (6 B x 256 per 8192 keys); scans 8 + 12; four backward replays
    # 2 + 8 + the tile table
    table = 6.0 * 256 / 8192
    per = 4 + 4 * (10 + 8 + table) + 8 + 12 + 4 * (2 + 8 + table)
    assert per == pytest.approx(137.5)
    assert b.model_step_bytes(n, 1) == pytest.approx(per * n)
    assert b.model_bytes("no_such_kernel", n) is None


def test_counter_record_applies_only_to_the_source_it_was_taken_from(tmp_path):
    b = load_bench()
    src_dir = tmp_path / "laplace_matvec_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = src_dir / "k.hip"
    src.write_text("kernel source, first version\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    (tmp_path / "profiles" / "k_w_counters.txt").write_text(
        "# a record\nkernel=k\nworkload=w\nsource=k.hip\n"
        f"source_sha={sha}\nhbm_bytes_per_launch=12345\n")
    (tmp_path / "profiles" / "step_w_counters.txt").write_text(
        f"kernel=step\nworkload=w\nsource=k.hip\nsource_sha={sha}\nhbm_bytes_per_step=777\n")
    b.ROOT = str(tmp_path)
    assert b.counter_traffic("k", "w") == 12345.0
    assert b.counter_traffic("k", "other") is None
    assert b.counter_traffic("other", "w") is None
    assert b.counter_step_bytes("w") == 777.0
    src.write_text("kernel source, changed since the counters were taken\n")
    assert b.counter_traffic("k", "w") is None
    assert b.counter_step_bytes("w") is None
