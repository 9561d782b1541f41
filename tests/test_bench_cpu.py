"""Host logic of bench.py (no GPU): the profile summaries it writes and reads,
the stale-source check on committed counter summaries, the rotation size and
the single-GPU refusal."""
from __future__ import annotations

import csv
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_stats_summary_keys_shapes_on_both_grid_dimensions(bench, tmp_path):
    d = tmp_path / "trace"
    d.mkdir()
    _write_csv(d / "run_kernel_stats.csv", ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [["k_a", "3", "2000", "1000", "3000"], ["k_b", "1", "500", "500", "500"]])
    head = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X", "Grid_Size_Y"]
    _write_csv(d / "run_kernel_trace.csv", head,
               [["k_a", "0", "1000", "256", "2816", "73"],      # same kernel, two grids in y
                ["k_a", "0", "3000", "256", "2816", "193"],
                ["k_a", "0", "2000", "256", "2816", "193"],
                ["k_b", "0", "500", "512", "81920", "1"]])
    out = tmp_path / "summary.txt"
    out.write_text("# header kept\n")
    bench.stats_summary(str(d), str(out))
    text = out.read_text()
    assert text.startswith("# header kept\n")  # appended after the caller's header
    lines = text.splitlines()
    shape = {tuple(ln.split()[:2]): ln.split() for ln in lines if ln.startswith(("k_a ", "k_b "))
             and len(ln.split()) == 6}
    # per-shape rows: kernel, grid, wg, calls, avg_us, median_us
    assert shape[("k_a", "2816x73")][3:] == ["1", "1.000", "1.000"]
    assert shape[("k_a", "2816x193")][3:5] == ["2", "2.500"]
    assert shape[("k_b", "81920")][2:4] == ["512", "1"]


def test_read_summary_rejects_a_stale_source_hash(bench, tmp_path):
    srcs = bench.MFMA_SOURCES
    good = tmp_path / "good.txt"
    good.write_text("source_sha256: %s\nmfma_busy_fraction: 0.4536   (ratio)\n" % bench.source_hash(srcs))
    assert bench.read_summary(str(good), "mfma_busy_fraction", srcs) == pytest.approx(0.4536)
    stale = tmp_path / "stale.txt"
    stale.write_text("source_sha256: 0000000000000000\nmfma_busy_fraction: 0.4536\n")
    assert bench.read_summary(str(stale), "mfma_busy_fraction", srcs) is None
    assert bench.read_summary(str(tmp_path / "missing.txt"), "mfma_busy_fraction", srcs) is None


def test_committed_counter_summaries_match_the_sources(bench):
    """The figures bench.py reports from profiles/ belong to the kernels as
    they are now (otherwise it reports null for them)."""
    assert bench.read_summary(bench.TRAFFIC_FILE, "traffic_bytes_per_launch", bench.KERNEL_SOURCES) is not None
    assert bench.read_summary(bench.MFMA_FILE, "mfma_busy_fraction", bench.MFMA_SOURCES) is not None
    text = open(bench.MOE_TRAFFIC_FILE).read()
    assert "source_sha256: %s" % bench.source_hash(bench.MOE_SOURCES) in text


def test_rotation_covers_a_gibibyte(bench):
    for nbytes in (1, 5 << 20, 56_770_560, 1 << 30, 3 << 30):
        n = bench.n_copies(nbytes)
        assert n >= 2 and n * nbytes >= min(bench.ROTATE_BYTES, 2 * nbytes)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert "one GPU" in (r.stdout + r.stderr)
