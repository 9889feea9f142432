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
    # design bytes: histogram 4; four radix passes with x as a value row:
    # 10 + 8 + the tile table (6 B x 256 per 8192 keys); scans 8 + 12; four
    # backward replays 2 + 8 + the tile table
    table = 6.0 * 256 / 8192
    per = 4 + 4 * (10 + 8 + table) + 8 + 12 + 4 * (2 + 8 + table)
    assert per == pytest.approx(137.5)
    assert b.model_step_bytes(n, 1) == pytest.approx(per * n)
    assert b.model_bytes("no_such_kernel", n) is None
    # the scope table's bytes: sort 68, gather 12, scan 20, scatter 12 at B = 1
    assert b.survey_step_bytes(n, 1) == pytest.approx(112.0 * n)
    # a radix pass launch: 12 B (first pass) or 16 B (later passes), 15 B on average
    assert b.survey_bytes("sort_pass", n) == pytest.approx(15.0 * n)
    four = sum(b.survey_bytes(k, n) * c for k, c in b.SYM_STEP.items())
    # the step's kernels at the table's per-launch figures: histogram 4,
    # passes 12 + 3 x 16, scans 8 + 12, scatter 12 (the gather rides in the
    # sort; the table's sort total of 68 is 4 more than its listed items)
    assert four == pytest.approx(96.0 * n)
    # x travelling through the passes: the four launches carry the gather's
    # 4 + 8B bytes per element between them, on top of the sort's 15 each
    for batch in (1, 16):
        with_rows = b.survey_bytes("sort_pass", n, batch, carried_rows=batch)
        assert 4 * (with_rows - b.survey_bytes("sort_pass", n, batch)) == pytest.approx((4.0 + 8.0 * batch) * n)
    # general case, 64 phased vectors: the bucketing reads w, its layout the
    # anchors and phase factors, the evaluation those and writes y
    assert b.survey_bytes("bucket_sorted", n, 64, 2) == pytest.approx(256.0 * n)
    assert b.survey_bytes("bucket_layout", n, 64, 2) == pytest.approx(12.0 * n)
    assert b.survey_bytes("eval", n, 64, 2) == pytest.approx(268.0 * n)
    assert b.gram_bytes("gram_tile", 4096, 3 << 20) == 4.0 * 4096 * 4096


def _tree(tmp_path):
    src_dir = tmp_path / "laplace_matvec_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "include").mkdir()
    (tmp_path / "profiles").mkdir()
    (src_dir / "k.hip").write_text("kernel source, first version\n")
    (src_dir / "k.h").write_text("device helpers\n")
    (tmp_path / "include" / "lib.h").write_text("the C ABI\n")
    return src_dir


def test_counter_record_applies_only_to_the_sources_it_was_taken_from(tmp_path):
    from laplace_matvec_amd import counters
    b = load_bench()
    src_dir = _tree(tmp_path)
    sha = counters.source_digest(str(tmp_path))
    (tmp_path / "profiles" / "w_counters.txt").write_text(
        f"# a record\nworkload=w\nsource_sha={sha}\nsteps=3\nlabel.k=4 12345\nlabel.j=1 7\nstep_bytes=49387\n")
    b.ROOT = str(tmp_path)
    rec = b.counter_record("w")
    assert rec is not None and rec["labels"]["k"] == (4.0, 12345.0) and float(rec["step_bytes"]) == 49387.0
    assert b.counter_record("other") is None
    # any library source changing makes the record stale: a kernel file, a
    # device header, the C ABI header
    for f in (src_dir / "k.hip", src_dir / "k.h", tmp_path / "include" / "lib.h"):
        old = f.read_text()
        f.write_text(old + "changed since the counters were taken\n")
        assert b.counter_record("w") is None, f
        f.write_text(old)
        assert b.counter_record("w") is not None
    (src_dir / "new.hip").write_text("a new kernel file\n")
    assert b.counter_record("w") is None


def test_counter_labels_follow_the_library_timing_names():
    from laplace_matvec_amd import counters
    assert counters.label_of("void lx::lx_sort_pass<true, false, true>(float const*)") == "sort_pass"
    assert counters.label_of("lx::lx_replay_bwd2<float>(float const*, long)") == "replay_backward"
    assert counters.label_of("lx::lx_replay_fwd2<unsigned int, true>(unsigned int const*)") == "perm_replay"
    assert counters.label_of("lx::lx_scan_reduce<1, 0, false, 1>(lx::ScanArgs)") == "scan_reduce"
    assert counters.label_of("lx::lx_scan_apply<2, 0, true, 8>(lx::ScanArgs)") == "scan_apply_scatter"
    assert counters.label_of("lx::lx_scan_apply<1, 2, true, 8>(lx::ScanArgs)") == "scan_apply_tables"
    assert counters.label_of("lx::lx_eval_rows<2>(lx::EvalArgs, int, int, long)") == "eval"
    assert counters.label_of("__amd_rocclr_copyBuffer") is None
    assert counters.label_of("(anonymous namespace)::lx_calib_copy(unsigned int const*, unsigned int*, long)") is None
    assert counters.label_of("(anonymous namespace)::lx_gen(void*, long, long, unsigned int)") is None
    assert counters.label_of("void lx::(anonymous namespace)::lx_small_sym<4>(lx::SmallSymArgs)") == "small_sym"


def test_calibration_uses_the_plain_copy_kernel():
    """The factor comes from the input library's copy kernel (1 GiB each
    way per dispatch), not from the runtime's blits, whose counters scale
    differently."""
    from laplace_matvec_amd import counters
    copy = "(anonymous namespace)::lx_calib_copy(unsigned int const*, unsigned int*, long)"
    disp = [("__amd_rocclr_copyBuffer", 524308.0), (copy, 524288.0), (copy, 524290.0),
            ("lx::lx_sort_hist(float const*)", 2.0e6)]
    f = counters.calibration_factor(disp, counters.COPY_BYTES)
    assert abs(f - (1 << 30) / (524289.0 * 1024.0)) < 1e-12
    with pytest.raises(ValueError):
        counters.calibration_factor([("__amd_rocclr_copyBuffer", 524308.0)], counters.COPY_BYTES)
    # every launch label in the sources is reachable from some kernel
    import re
    labels = set()
    for f in counters.source_files():
        labels |= set(re.findall(r'LX_LAUNCH\(\s*"([a-z_]+)"', open(f).read()))
    assert "sort_pass" in labels and "replay_backward" in labels
