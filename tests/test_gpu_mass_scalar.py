"""GPU scalar mass matrix (coefficient q w; MFMA, VALU and flat variants) vs the
fp64 oracle.

Tolerance as for the tensor matrix: ||M_gpu - M_oracle||_F <= 1e-4
||M_oracle||_F over the 27-offset store (the mass-matrix paper, §5 "Exactness
and precision": the per-cell contraction is exact up to fp32 rounding), and
max |M_gpu - M_oracle| <= 1e-4 max |M_oracle|.
"""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import (DEV, block_row_sums, check_row_sums, dev, full_workload, node_row_sums,
                      rel_frob_err, say, seam_cells)

pytestmark = pytest.mark.gpu
TOL = 1e-4
VARIANTS = [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU, pcg.PCG_MASS_FLAT]


def _run(wl, perm, off, variant, n_part=None, use_layout=True):
    s = wl.take(perm.astype(np.int64)) if perm is not None else wl
    M = torch.zeros(wl.n[2], wl.n[1], wl.n[0], 27, dtype=torch.float32, device=DEV)
    cells = None
    if use_layout:
        cells = pcg.Layout(T=1, order=1, tile_offsets=dev(off.view(np.int32)),
                           n_partitioned=wl.count if n_part is None else n_part, drift=0)
    say("mass scalar", wl.n, wl.count, variant, n_part, use_layout)
    pcg.assemble_mass_matrix_scalar(wl.n, [dev(a) for a in s.x], dev(s.q), dev(s.w), M, cells,
                                    variant)
    torch.cuda.synchronize()
    return M.cpu().numpy()


def _check(M, ref):
    assert rel_frob_err(M, ref) <= TOL
    assert np.abs(M - ref).max() <= 1e-4 * np.abs(ref).max()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n,ppc", [([8, 8, 8], 16), ([6, 5, 7], 64), ([4, 4, 4], 100),
                                   ([9, 3, 5], 7)])
def test_scalar_mass_matches_oracle(orc, variant, n, ppc):
    """Uniform loading; ppc = 100 takes a second, partial 64-particle batch, ppc = 7
    a partial 8-particle product."""
    wl = synthetic.mass_workload(n, ppc, w_uniform=True, seed=600 + ppc)
    _, perm, off = orc.tile_sort(3, n, 1, 1, wl.x)
    M = _run(wl, perm, off, variant)
    _check(M, orc.mass_matrix_scalar(n, wl.x, wl.q, wl.w))


@pytest.mark.parametrize("variant", VARIANTS)
def test_scalar_mass_ragged_cells(orc, variant):
    """Random positions: empty cells, cells of 1-3 particles and cells far above 64."""
    r = np.random.default_rng(61)
    n = [10, 9, 8]
    cnt = 6000
    x = [r.uniform(0, n[k], cnt).astype(np.float32) for k in range(3)]
    x[0][:1500] = r.uniform(2, 3, 1500).astype(np.float32)   # a crowded column
    x[1][:1500] = r.uniform(4, 5, 1500).astype(np.float32)
    q = np.where(r.random(cnt) < 0.5, 1.0, -1.0).astype(np.float32)
    w = r.uniform(0.5, 1.5, cnt).astype(np.float32)
    z = np.zeros(cnt, np.float32)
    wl = synthetic.Workload(3, n, x, x, [z] * 3, q, w, [z] * 3, z)
    _, perm, off = orc.tile_sort(3, n, 1, 1, x)
    M = _run(wl, perm, off, variant)
    _check(M, orc.mass_matrix_scalar(n, x, q, w))


@pytest.mark.parametrize("variant", [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU])
def test_scalar_mass_stale_layout_and_tail(orc, variant):
    """Particles moved after the cell sort lie outside their slice's cell and go
    through the flat path; so does the unsorted tail."""
    wl = synthetic.mass_workload([8, 8, 8], 20, seed=63)
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    s = wl.take(perm.astype(np.int64))
    s.x[0] = synthetic.periodic_shift(s.x[0], np.where(np.arange(s.count) % 7 == 0, 0.6, 0.0), 8)
    M = _run(s, None, off, variant, n_part=s.count - 500)
    _check(M, orc.mass_matrix_scalar(wl.n, s.x, s.q, s.w))


def test_scalar_mass_no_layout_is_flat(orc):
    wl = synthetic.mass_workload([5, 6, 7], 9, seed=64)
    M = _run(wl, None, None, pcg.PCG_MASS_AUTO, use_layout=False)
    _check(M, orc.mass_matrix_scalar(wl.n, wl.x, wl.q, wl.w))


@pytest.mark.parametrize("variant", [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU])
def test_scalar_mass_z_seams(orc, variant):
    """A grid of several 8-node work-group columns in z and two in y: every row
    against the oracle."""
    wl = synthetic.mass_workload([8, 10, 36], 24, w_uniform=True, seed=611)
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    _check(_run(wl, perm, off, variant), orc.mass_matrix_scalar(wl.n, wl.x, wl.q, wl.w))


def test_scalar_mass_full_size_64(orc):
    """64^3, 64 ppc (16.8M particles), the launch the benchmark times.  The
    oracle runs on the particles of the cell planes on both sides of every z
    plane 4k (the wrap included) and the node rows only they reach are
    compared entry by entry; every row's sum equals sum_p q w W_pg (Eq.(11),
    numpy); entries (g, o) and (g + o, -o) agree (symmetry) to fp32 rounding."""
    wl = full_workload("mass_64_ppc64")
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    M = _run(wl, perm, off, pcg.PCG_MASS_MFMA)
    s = wl.take(perm.astype(np.int64))
    cells, rows = seam_cells(wl.n[2], 4)
    sub = s.take(np.nonzero(cells[np.floor(s.x[2]).astype(np.int64)])[0])
    ref = orc.mass_matrix_scalar(wl.n, sub.x, sub.q, sub.w)
    _check(M[rows], ref[rows])
    qw = s.q.astype(np.float64) * s.w
    want = node_row_sums(wl.n, s.x, 1, [qw])
    scale = node_row_sums(wl.n, s.x, 1, [np.abs(qw)])
    say("row sums: worst error / bound", check_row_sums(block_row_sums(M), want, scale, TOL))
    offs = [(dx, dy, dz) for dz in (-1, 0, 1) for dy in (-1, 0, 1) for dx in (-1, 0, 1)]
    scale = np.abs(M).max()
    for o, (dx, dy, dz) in enumerate(offs):
        mo = offs.index((-dx, -dy, -dz))
        rolled = np.roll(M[..., mo], shift=(-dz, -dy, -dx), axis=(0, 1, 2))
        assert np.abs(M[..., o] - rolled).max() <= 1e-5 * scale


@pytest.mark.parametrize("variant", [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_FLAT])
def test_scalar_mass_overwrite(orc, variant):
    """PCG_MASS_OVERWRITE on the scalar matrix: M's previous values are gone,
    a tail still adds after the rows are set."""
    wl = synthetic.mass_workload([9, 8, 10], 12, seed=68)
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    s = wl.take(perm.astype(np.int64))
    M = torch.from_numpy(np.random.default_rng(69).standard_normal(
        (10, 8, 9, 27)).astype(np.float32)).to(DEV)
    cells = pcg.Layout(T=1, order=1, tile_offsets=dev(off.view(np.int32)),
                       n_partitioned=s.count - 200, drift=0)
    pcg.assemble_mass_matrix_scalar(wl.n, [dev(a) for a in s.x], dev(s.q), dev(s.w), M, cells,
                                    variant | pcg.PCG_MASS_OVERWRITE)
    torch.cuda.synchronize()
    _check(M.cpu().numpy(), orc.mass_matrix_scalar(wl.n, s.x, s.q, s.w))


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", ["empty", "all_tail"])
def test_scalar_mass_empty_and_all_tail(orc, variant, case):
    """No particles: M keeps its values when added to and is all zeros with
    PCG_MASS_OVERWRITE; a layout that covers none of the particles (all in the
    unsorted tail) still gives the whole matrix, on every path."""
    wl = synthetic.mass_workload([7, 6, 5], 12, seed=122)
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    s = wl.take(perm.astype(np.int64))
    if case == "empty":
        s = s.take(np.arange(0))
        off = np.zeros_like(off)
    init = np.random.default_rng(123).standard_normal((5, 6, 7, 27)).astype(np.float32)
    cells = pcg.Layout(T=1, order=1, tile_offsets=dev(off.view(np.int32)), n_partitioned=0,
                       drift=0)
    for flags in (0, pcg.PCG_MASS_OVERWRITE):
        M = torch.from_numpy(init.copy()).to(DEV)
        say("mass scalar", case, variant, flags)
        pcg.assemble_mass_matrix_scalar(wl.n, [dev(a) for a in s.x], dev(s.q), dev(s.w), M, cells,
                                        variant | flags)
        torch.cuda.synchronize()
        got = M.cpu().numpy().astype(np.float64)
        if not s.count:
            assert np.array_equal(got, np.zeros_like(got) if flags else init)
        else:
            _check(got if flags else got - init, orc.mass_matrix_scalar(wl.n, s.x, s.q, s.w))
