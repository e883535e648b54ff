"""Host logic of the profile summaries: kernel symbols map to the library's launch
names (the benchmark looks traffic records up by them), and a record's digest
covers the source file that holds the kernel."""
import os

import pytest

from particle_cell_grid_amd import profsummary as ps


@pytest.mark.parametrize("symbol,name", [
    ("k_deposit_tiled<3, 1, 0, 11, true>", "deposit_regroup"),
    ("k_deposit_tiled<3, 1, 0, 11, false>", "deposit_tiled"),
    ("k_deposit_flat<3, 1>", "deposit_flat"),
    ("k_inc_count<3, 1, 4>", "sort_inc_count"),
    ("k_inc_move<3, 1, 4>", "sort_inc_move"),
    ("k_mass_column<true, false, float>", "mass_mfma"),
    ("k_mass_column<false, false, float>", "mass_valu"),
    ("k_mass_column<true, true, float>", "mass_scalar_mfma"),
    ("k_mass_column<true, false, double>", "mass_mfma_f64"),
    ("k_mass_column<false, true, double>", "mass_scalar_valu_f64"),
    ("k_mass_flat<false, float>", "mass_flat"),
    ("k_mass_strays<true, double>", "mass_scalar_strays_f64"),
    ("k_mass_tsc_brick<false>", "mass_tsc_mfma"),
    ("k_mass_tsc_brick<true>", "mass_tsc_tensor_mfma"),
    ("k_mass_tsc_valu", "mass_tsc_valu"),
    ("k_mass_tsc_tensor_valu", "mass_tsc_tensor_valu"),
    ("k_mass_tsc_flat", "mass_tsc_flat"),
    ("k_mass_tsc_tensor_flat", "mass_tsc_tensor_flat"),
    ("k_sweep1d", "sweep1d"),
    ("k_sweep1d_grad<true>", "sweep1d_grad"),
    ("k_zigzag_tiled<true, 13>", "zigzag_tiled"),
    ("k_zigzag_tiled<false, 0>", "zigzag_tiled_f32"),
    ("k_zigzag_flat", "zigzag_flat"),
])
def test_tap_names(symbol, name):
    assert ps.tap_name(symbol) == name


def test_short_names_drop_the_parameter_list():
    sym = "void pcg::(anonymous namespace)::k_inc_move<3, 1, 4>(pcg::(anonymous namespace)::IncGeom)"
    assert ps.short(sym) == "k_inc_move<3, 1, 4>"


@pytest.mark.parametrize("name,src", [("deposit_regroup", "deposit.hip"),
                                      ("sort_inc_count", "sort.hip"),
                                      ("mass_mfma", "mass.hip"),
                                      ("mass_tsc_tensor_mfma", "mass_tsc.hip"),
                                      ("sweep1d_grad", "sweep.hip")])
def test_digest_covers_the_kernel_source(name, src, tmp_path, monkeypatch):
    """Changing the kernel's own file changes its digest; another kernel file does not."""
    import shutil
    csrc = tmp_path / "csrc"
    shutil.copytree(ps.CSRC, csrc, ignore=shutil.ignore_patterns("_build"))
    monkeypatch.setattr(ps, "CSRC", str(csrc))
    before = ps.source_digest(name)
    other = "sweep.hip" if src != "sweep.hip" else "mass.hip"
    with open(os.path.join(csrc, other), "a") as f:
        f.write("\n// touched\n")
    assert ps.source_digest(name) == before
    with open(os.path.join(csrc, src), "a") as f:
        f.write("\n// touched\n")
    assert ps.source_digest(name) != before


def test_calibration_uses_the_large_copy():
    """Small copies of the workload's own (bins, read-backs) go through the same
    copy kernel; the calibration reading is the 1 GiB copy's."""
    big = [524300.0, 524315.0, 524290.0]
    small = [7.0, 162.0, 524.0, 524.0, 524.0, 524.0, 524.0]
    assert ps.calibration_reading(big + small) in big
    assert ps.calibration_reading(big) == 524300.0
