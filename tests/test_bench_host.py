"""Host logic of bench.py (no GPU): the kernel-source hash and the counter summary it
gates, and the refusal of more than one GPU."""

import pathlib
import subprocess
import sys

import bench

ROOT = pathlib.Path(__file__).resolve().parent.parent


def test_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    a.write_text("int x = 1;  // one\n\n// note\nint y = 2;\n")
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [a])
    h1 = bench.kernel_source_hash()
    a.write_text("// header\nint x = 1;\nint y = 2;  // two\n")
    assert bench.kernel_source_hash() == h1
    a.write_text("int x = 1;\nint y = 3;\n")
    assert bench.kernel_source_hash() != h1


def test_counter_traffic_needs_a_matching_hash(tmp_path, monkeypatch):
    summary = tmp_path / "counters.md"
    monkeypatch.setattr(bench, "COUNTERS", summary)
    summary.write_text(f"- hbm bytes per launch: 123\n- kernel source hash: `{bench.kernel_source_hash()}`\n")
    assert bench.counter_traffic() == 123
    summary.write_text("- hbm bytes per launch: 123\n- kernel source hash: `0000000000000000`\n")
    assert bench.counter_traffic() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr


def test_clock_reading_reports_instead_of_raising():
    """Without a GPU (or amdsmi) the clock reading reports the error and the bench goes on."""
    import torch

    calls = []
    rep = bench.clocks_under_load(torch, torch.device("cuda:0"), calls.append, seconds=0.1)
    assert "error" in rep or "readings" in rep
