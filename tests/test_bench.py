"""The benchmark's contract on the host: one GPU only, the roofline arithmetic,
and traffic records that resolve only while their kernel sources are unchanged."""
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
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_roofline_entry():
    kt = {"k": dict(avg_us=100.0)}
    hbm = bench.roofline_entry(kt, "k", bytes_per_launch=4e8)      # 4 TB/s
    assert hbm["bound"] == "hbm" and hbm["achieved"] == 4000.0
    assert hbm["frac"] == pytest.approx(4000.0 / bench.HBM_PEAK_GBS)
    mf = bench.roofline_entry(kt, "k", flops_per_launch=1e9, mfma_peak=bench.MFMA_FP64_PEAK_TFLOPS)
    assert mf["bound"] == "mfma" and mf["achieved"] == pytest.approx(10.0)
    assert mf["frac"] == pytest.approx(10.0 / 78.6, abs=1e-4)
    assert bench.roofline_entry(kt, "missing", bytes_per_launch=1.0) is None


def test_measured_traffic_follows_the_source_digest(monkeypatch):
    """A committed record resolves to its read + write bytes while the kernel's
    digest matches, and to None once the sources change (or for no record)."""
    import json

    from particle_cell_grid_amd import profsummary

    rec = json.load(open(bench.TRAFFIC_FILE))["kernels"]["cic3d_128_ppc32"]["deposit_regroup"]
    monkeypatch.setattr(profsummary, "source_digest", lambda k: rec["source_sha1"])
    t = bench.measured_traffic("deposit_regroup", "cic3d_128_ppc32")
    assert t == int(rec["read_bytes"] + rec["write_bytes"]) and 4e9 < t < 6e9
    assert bench.measured_traffic("deposit_regroup", "no_such_workload") is None
    monkeypatch.setattr(profsummary, "source_digest", lambda k: "changed")
    assert bench.measured_traffic("deposit_regroup", "cic3d_128_ppc32") is None


def test_kernel_table_marks_gated_launches():
    """Launches of the general sort that a step enqueues behind the incremental
    one carry no bytes, so no per-kernel rate can exceed the HBM peak by
    counting work a gated launch never did."""
    kt = {"deposit_regroup": dict(avg_us=1000.0, launches=20),
          "sort_permute": dict(avg_us=6.0, launches=20),
          "sort_hist": dict(avg_us=6.0, launches=40)}
    alg = {"deposit_regroup": 4.3e9, "sort_permute": 4.5e9}
    tab = bench.kernel_table(kt, 20, alg, gated=True)
    assert "GBps" not in tab["sort_permute"] and "gated" in tab["sort_permute"]
    assert tab["sort_hist"]["launches_per_step"] == 2.0
    assert tab["deposit_regroup"]["GBps"] == 4300.0
    for e in tab.values():
        assert e.get("GBps", 0.0) <= bench.HBM_PEAK_GBS
