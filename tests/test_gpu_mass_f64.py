"""GPU fp64 mass matrices (ECSIM tensor and scalar; MFMA on v_mfma_f64_16x16x4f64,
VALU and flat variants) vs the fp64 oracle.

Tolerance: every product and sum is fp64 on both sides and the inputs are the
same fp32 values, so the two differ only in summation order: ||M_gpu -
M_oracle||_F <= 1e-12 ||M_oracle||_F and max |M_gpu - M_oracle| <= 1e-12 max
|M_oracle| (the mass-matrix paper, §5 "Exactness and precision": no rounding
error seen with its FP64 tile).
"""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import (DEV, block_row_sums, check_row_sums, dev, full_size_checks,
                      full_workload, node_row_sums, rel_frob_err, say, seam_cells)

pytestmark = pytest.mark.gpu
TOL = 1e-12
VARIANTS = [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU, pcg.PCG_MASS_FLAT]


def _run(wl, perm, off, variant, scalar, n_part=None, M0=None):
    s = wl.take(perm.astype(np.int64)) if perm is not None else wl
    shape = (wl.n[2], wl.n[1], wl.n[0], 27) + (() if scalar else (3, 3))
    M = torch.zeros(shape, dtype=torch.float64, device=DEV)
    if M0 is not None:
        M.copy_(torch.from_numpy(M0.reshape(shape)))
    cells = pcg.Layout(T=1, order=1, tile_offsets=dev(off.view(np.int32)),
                       n_partitioned=wl.count if n_part is None else n_part, drift=0)
    say("mass f64", "scalar" if scalar else "tensor", wl.n, wl.count, variant, n_part)
    if scalar:
        pcg.assemble_mass_matrix_scalar(wl.n, [dev(a) for a in s.x], dev(s.q), dev(s.w), M, cells,
                                        variant)
    else:
        pcg.assemble_mass_matrix(wl.n, [dev(a) for a in s.x], [dev(b) for b in s.B],
                                 dev(s.beta), dev(s.q), dev(s.w), M, cells, variant)
    torch.cuda.synchronize()
    return M.cpu().numpy()


def _ref(orc, n, s, scalar):
    if scalar:
        return orc.mass_matrix_scalar(n, s.x, s.q, s.w)
    return orc.mass_matrix(n, s.x, s.B, s.q, s.w, s.beta)


def _check(M, ref):
    assert M.dtype == np.float64
    assert rel_frob_err(M, ref) <= TOL
    assert np.abs(M - ref).max() <= TOL * np.abs(ref).max()


@pytest.mark.parametrize("scalar", [False, True])
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n,ppc", [([8, 8, 8], 16), ([6, 5, 7], 64), ([4, 4, 4], 100)])
def test_f64_mass_matches_oracle(orc, scalar, variant, n, ppc):
    """Uniform loading; ppc = 100 takes a second, partial 64-particle batch."""
    wl = synthetic.mass_workload(n, ppc, w_uniform=True, seed=700 + ppc)
    _, perm, off = orc.tile_sort(3, n, 1, 1, wl.x)
    _check(_run(wl, perm, off, variant, scalar), _ref(orc, n, wl, scalar))


@pytest.mark.parametrize("scalar", [False, True])
def test_f64_mass_ragged_stale_and_tail(orc, scalar):
    """Random positions (empty, sparse and crowded cells), a stale layout (every
    7th particle moved after the sort) and an unsorted tail of 500."""
    r = np.random.default_rng(71)
    n = [10, 9, 8]
    cnt = 6000
    x = [r.uniform(0, n[k], cnt).astype(np.float32) for k in range(3)]
    x[0][:1500] = r.uniform(2, 3, 1500).astype(np.float32)
    x[1][:1500] = r.uniform(4, 5, 1500).astype(np.float32)
    B = [r.normal(0, 1, cnt).astype(np.float32) for _ in range(3)]
    q = np.where(r.random(cnt) < 0.5, 1.0, -1.0).astype(np.float32)
    w = r.uniform(0.5, 1.5, cnt).astype(np.float32)
    beta = (q * 0.05).astype(np.float32)
    wl = synthetic.Workload(3, n, x, x, [np.zeros(cnt, np.float32)] * 3, q, w, B, beta)
    _, perm, off = orc.tile_sort(3, n, 1, 1, x)
    s = wl.take(perm.astype(np.int64))
    s.x[0] = synthetic.periodic_shift(s.x[0], np.where(np.arange(cnt) % 7 == 0, 0.6, 0.0), n[0])
    M = _run(s, None, off, pcg.PCG_MASS_MFMA, scalar, n_part=cnt - 500)
    _check(M, _ref(orc, n, s, scalar))


@pytest.mark.parametrize("scalar", [False, True])
@pytest.mark.parametrize("variant", [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU])
@pytest.mark.parametrize("n,ppc", [([8, 8, 40], 16), ([10, 9, 36], 24)])
def test_f64_mass_z_seams(orc, scalar, variant, n, ppc):
    """Grids taller than one work-group column of nodes in z (both matrices):
    every row, those on both sides of each column boundary and of the wrap
    included, against the oracle."""
    wl = synthetic.mass_workload(n, ppc, w_uniform=True, seed=710 + ppc)
    _, perm, off = orc.tile_sort(3, n, 1, 1, wl.x)
    _check(_run(wl, perm, off, variant, scalar), _ref(orc, n, wl, scalar))


def test_f64_mass_full_size_64(orc):
    """64^3, 64 ppc, the tensor matrix in fp64 on the matrix cores: the rows on
    both sides of every z plane 8k entry by entry, and every row's block sums."""
    wl = full_workload("mass_64_ppc64")
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    M = _run(wl, perm, off, pcg.PCG_MASS_MFMA, scalar=False)
    full_size_checks(orc, wl.take(perm.astype(np.int64)), M, TOL)


def test_f64_scalar_mass_full_size_64(orc):
    """64^3, 64 ppc, the scalar matrix in fp64 on the matrix cores: the rows on
    both sides of every z plane 4k (its work-group columns are 8 nodes tall)
    entry by entry, and every row's sum against sum_p q w W_pg."""
    wl = full_workload("mass_64_ppc64")
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    M = _run(wl, perm, off, pcg.PCG_MASS_MFMA, scalar=True)
    s = wl.take(perm.astype(np.int64))
    cells, rows = seam_cells(wl.n[2], 4)
    sub = s.take(np.nonzero(cells[np.floor(s.x[2]).astype(np.int64)])[0])
    ref = orc.mass_matrix_scalar(wl.n, sub.x, sub.q, sub.w)
    _check(M[rows], ref[rows])
    qw = s.q.astype(np.float64) * s.w
    want = node_row_sums(wl.n, s.x, 1, [qw])
    scale = node_row_sums(wl.n, s.x, 1, [np.abs(qw)])
    say("row sums: worst error / bound", check_row_sums(block_row_sums(M), want, scale, TOL))


@pytest.mark.parametrize("scalar", [False, True])
def test_f64_mass_overwrite(orc, scalar):
    """PCG_MASS_OVERWRITE in fp64: the column kernel stores every row of M
    without reading it."""
    wl = synthetic.mass_workload([8, 6, 7], 16, seed=78)
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    s = wl.take(perm.astype(np.int64))
    size = 7 * 6 * 8 * 27 * (1 if scalar else 9)
    M0 = np.random.default_rng(79).standard_normal(size)
    M = _run(s, None, off, pcg.PCG_MASS_MFMA | pcg.PCG_MASS_OVERWRITE, scalar, M0=M0)
    ref = _ref(orc, wl.n, s, scalar)
    assert rel_frob_err(M, ref) <= TOL


@pytest.mark.parametrize("scalar", [False, True])
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", ["empty", "all_tail"])
def test_f64_mass_empty_and_all_tail(orc, scalar, variant, case):
    """No particles: M keeps its values when added to and is all zeros with
    PCG_MASS_OVERWRITE; a layout that covers none of the particles (all in the
    unsorted tail) still gives the whole matrix, in fp64 on every path."""
    wl = synthetic.mass_workload([7, 6, 5], 12, seed=120)
    _, perm, off = orc.tile_sort(3, wl.n, 1, 1, wl.x)
    s = wl.take(perm.astype(np.int64))
    if case == "empty":
        s = s.take(np.arange(0))
        off = np.zeros_like(off)
    size = 5 * 6 * 7 * 27 * (1 if scalar else 9)
    M0 = np.random.default_rng(121).standard_normal(size)
    for flags in (0, pcg.PCG_MASS_OVERWRITE):
        M = _run(s, None, off, variant | flags, scalar, n_part=0, M0=M0)
        init = M0.reshape(M.shape)
        if not s.count:
            assert np.array_equal(M, np.zeros_like(M) if flags else init)
        else:
            ref = _ref(orc, wl.n, s, scalar)
            got = M if flags else M - init
            assert rel_frob_err(got, ref) <= TOL
            # adding to a non-zero M rounds against its values, not the matrix's
            bound = TOL * (np.abs(ref).max() + (0 if flags else np.abs(init).max()))
            assert np.abs(got - ref).max() <= bound
