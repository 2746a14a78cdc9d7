"""bench.py's host-side helpers, on the CPU: the one-GPU refusal, and how committed profiles are
attached to a bench line (only while the kernel source they were taken on is unchanged).
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_counter_entries_follow_their_source(tmp_path, monkeypatch):
    with open(bench.COUNTERS_FILE) as fh:
        table = json.load(fh)["kernels"]
    fields = {"avg_us", "hbm_read_gb", "hbm_write_gb", "l2_hit", "mfma_busy",
              "mfma_busy_at_2400mhz", "bf16_mfma_tflops", "clock_ghz"}
    allc = bench.counters_for()
    assert set(allc) == set(table)
    for key, e in allc.items():
        # an entry is attached exactly when its source file still hashes as when it was taken
        src = os.path.join(ROOT, "frame_wise_gated_libgdn_amd", "csrc", table[key]["source"])
        current = bench.source_sha(src) == table[key]["source_sha256"]
        assert (e is not None) == current, key
        if e is not None:
            assert set(e) == fields
            assert bench.counters_for(key) == e
    assert bench.counters_for("no such kernel") is None
    # a changed source (here: every hash differs) detaches every entry
    monkeypatch.setattr(bench, "source_sha", lambda path=None: "0" * 64)
    assert all(v is None for v in bench.counters_for().values())
    # a missing or unreadable table gives None
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(tmp_path / "missing.json"))
    assert bench.counters_for() is None


def test_kernel_against_its_ceiling(monkeypatch):
    ceiling = {"kind": "copy", "gb_s": 5000.0}
    monkeypatch.setattr(bench, "counters_for",
                        lambda key=None: {"hbm_read_gb": 30.0, "hbm_write_gb": 20.0})
    # 40 GB algorithmic, 50 GB moved, in 10 ms
    out = bench.kernel_vs_ceiling(40e9, 10.0, "bwd", ceiling)
    assert out["achieved_gb_s"] == pytest.approx(4000.0)
    assert out["frac"] == pytest.approx(4000.0 / bench.HBM_PEAK_GBS)
    assert out["hbm_gb_per_launch"] == pytest.approx(50.0)
    assert out["hbm_gb_s"] == pytest.approx(5000.0)
    assert out["frac_of_ceiling"] == pytest.approx(1.0)
    assert out["ceiling"] is ceiling
    # without counters for the current source: no HBM figures, the algorithmic ones stay
    monkeypatch.setattr(bench, "counters_for", lambda key=None: None)
    out = bench.kernel_vs_ceiling(40e9, 10.0, "bwd", ceiling)
    assert out["hbm_gb_s"] is None and out["frac_of_ceiling"] is None
    assert out["achieved_gb_s"] == pytest.approx(4000.0)
    assert bench.kernel_vs_ceiling(40e9, None, "bwd", ceiling) is None


def test_streaming_ceiling_kinds_name_their_mix():
    assert set(bench.CEILING_KINDS) == {1, 2, 3}
    for nread, kind in bench.CEILING_KINDS.items():
        assert "%d tensor" % nread in kind and "1 written" in kind
