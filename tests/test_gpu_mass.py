"""GPU ECSIM mass matrix (MFMA, VALU and flat variants) vs the fp64 oracle.

Tolerance: ||M_gpu - M_oracle||_F <= 1e-4 ||M_oracle||_F over the 27 x 9 store
(the mass-matrix paper, §5 "Exactness and precision": the reformulation is exact
up to the tile's rounding).  A tighter max-abs check guards single entries.
"""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import DEV, dev, full_size_checks, full_workload, rel_frob_err, say

pytestmark = pytest.mark.gpu
TOL = 1e-4
VARIANTS = [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU, pcg.PCG_MASS_FLAT]


def _run(wl, perm, off, variant, n_part=None, use_layout=True, M0=None):
    s = wl.take(perm.astype(np.int64)) if perm is not None else wl
    M = torch.zeros(wl.n[2], wl.n[1], wl.n[0], 27, 3, 3, dtype=torch.float32, device=DEV)
    if M0 is not None:
        M.copy_(torch.from_numpy(M0))
    cells = None
    if use_layout:
        cells = pcg.Layout(T=1, order=1, tile_offsets=dev(off.view(np.int32)),
                           n_partitioned=wl.count if n_part is None else n_part, drift=0)
    say("mass", wl.n, wl.count, variant, n_part, use_layout)
    pcg.assemble_mass_matrix(wl.n, [dev(a) for a in s.x], [dev(b) for b in s.B], dev(s.beta),
                             dev(s.q), dev(s.w), M, cells, variant)
    torch.cuda.synchronize()
    return M.cpu().numpy()


def _check(M, ref):
    assert rel_frob_err(M, ref) <= TOL
    assert np.abs(M - ref).max() <= 1e-4 * np.abs(ref).max()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n,ppc", [([8, 8, 8], 16), ([6, 5, 7], 64), ([4, 4, 4], 100)])
def test_mass_matches_oracle(orc, variant, n, ppc):
    """Uniform loading; ppc = 100 exercises a second (partial) 64-particle batch."""
    wl = synthetic.mass_workload(n, ppc, w_uniform=True, seed=500 + ppc)
    _, perm, off = orc.tile_sort(3, n, 1, 1, wl.x)
    M = _run(wl, perm, off, variant)
    ref = orc.mass_matrix(n, wl.x, wl.B, wl.q, wl.w, wl.beta)
    _check(M, ref)


@pytest.mark.parametrize("variant", VARIANTS)
def test_mass_ragged_cells(orc, variant):
    """Random positions: empty cells, cells with 1-3 particles (padded batches),
    and cells far above 64."""
    r = np.random.default_rng(51)
    n = [10, 9, 8]
    cnt = 6000
    x = [r.uniform(0, n[k], cnt).astype(np.float32) for k in range(3)]
    x[0][:1500] = r.uniform(2, 3, 1500).astype(np.float32)   # a crowded column
    x[1][:1500] = r.uniform(4, 5, 1500).astype(np.float32)
    B = [r.normal(0, 1, cnt).astype(np.float32) for _ in range(3)]
    q = np.where(r.random(cnt) < 0.5, 1.0, -1.0).astype(np.float32)
    w = r.uniform(0.5, 1.5, cnt).astype(np.float32)
    beta = (q * 0.05).astype(np.float32)
    wl = synthetic.Workload(3, n, x, x, [np.zeros(cnt, np.float32)] * 3, q, w, B, beta)
    _, perm, off = orc.tile_sort(3, n, 1, 1, x)
    M = _run(wl, perm, off, variant)
    _check(M, orc.mass_matrix(n, x, B, q, w, beta))


@pytest.mark.parametrize("variant", [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU])
def test_mass_stale_layout_and_tail(orc, variant):
    """Particles moved after the cell sort are found in the wrong cell's slice and
    deposited by the flat path; the unsorted tail likewise."""
    wl = synthetic.mass_workload([8, 8, 8], 20, seed=53)
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    s = wl.take(perm.astype(np.int64))
    moved = synthetic.periodic_shift(s.x[0], np.where(np.arange(s.count) % 7 == 0, 0.6, 0.0), 8)
    s.x[0] = moved
    M = _run(s, None, off, variant, n_part=s.count - 500)
    _check(M, orc.mass_matrix(wl.n, s.x, s.B, s.q, s.w, s.beta))


def test_mass_zero_field_reduces_to_scalar(orc):
    wl = synthetic.mass_workload([6, 6, 6], 16, seed=54)
    wl.B = [np.zeros_like(b) for b in wl.B]
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    M = _run(wl, perm, off, pcg.PCG_MASS_MFMA)
    assert np.abs(M[..., 0, 1]).max() <= 1e-6 * np.abs(M[..., 0, 0]).max()
    assert np.allclose(M[..., 0, 0], M[..., 2, 2], rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("variant", [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU])
@pytest.mark.parametrize("n,ppc", [([8, 8, 40], 16), ([10, 9, 36], 24)])
def test_mass_z_seams(orc, variant, n, ppc):
    """Grids taller than one work-group column of nodes in z: every row, the
    rows on both sides of each column boundary and of the periodic wrap
    included, against the oracle.  Weights w ~ U[0.5, 1.5]."""
    wl = synthetic.mass_workload(n, ppc, w_uniform=True, seed=510 + ppc)
    _, perm, off = orc.tile_sort(3, n, 1, 1, wl.x)
    M = _run(wl, perm, off, variant)
    _check(M, orc.mass_matrix(n, wl.x, wl.B, wl.q, wl.w, wl.beta))


def test_mass_full_size_64(orc):
    """64^3, 64 ppc (16.8M particles), the launch the benchmark times."""
    wl = full_workload("mass_64_ppc64")
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    M = _run(wl, perm, off, pcg.PCG_MASS_MFMA)
    full_size_checks(orc, wl.take(perm.astype(np.int64)), M, TOL)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", ["layout", "stale_tail", "all_tail", "empty"])
def test_mass_overwrite(orc, variant, case):
    """PCG_MASS_OVERWRITE: M holding other values ends as the matrix alone, on
    every path (the column kernels store each row without reading it; the
    others clear M first), with stray and tail particles still added, and as
    zeros for no particles."""
    wl = synthetic.mass_workload([8, 7, 6], 20, seed=58)
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    s = wl.take(perm.astype(np.int64))
    n_part = s.count
    if case == "stale_tail":
        s.x[0] = synthetic.periodic_shift(s.x[0], np.where(np.arange(s.count) % 7 == 0, 0.6, 0.0),
                                          wl.n[0])
        n_part = s.count - 300
    elif case == "all_tail":
        n_part = 0
    elif case == "empty":
        s = s.take(np.arange(0))
        off = np.zeros_like(off)
        n_part = 0
    M0 = np.random.default_rng(59).standard_normal((6, 7, 8, 27, 3, 3)).astype(np.float32)
    if variant == pcg.PCG_MASS_FLAT and case != "layout":
        return  # the flat path ignores the layout: one case covers it
    M = _run(s, None, off, variant | pcg.PCG_MASS_OVERWRITE, n_part=n_part, M0=M0)
    ref = orc.mass_matrix(wl.n, s.x, s.B, s.q, s.w, s.beta) if s.count else np.zeros_like(M)
    if s.count:
        _check(M, ref)
    else:
        assert not M.any()
