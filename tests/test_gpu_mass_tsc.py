"""GPU mass matrices with TSC weights, scalar and ECSIM tensor (MFMA, VALU and
flat variants), vs the fp64 oracle.

Tolerance as for the fp32 CIC matrices: ||M_gpu - M_oracle||_F <= 1e-4
||M_oracle||_F over the 125-offset store and max |M_gpu - M_oracle| <= 1e-4
max |M_oracle| (fp32 products and sums, fp32 atomics into M; the mass-matrix
paper, §5 "Exactness and precision")."""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import (DEV, alpha_coefs, axis_weights, block_row_sums, check_row_sums, dev,
                      full_workload, node_row_sums, rel_frob_err, say)

pytestmark = pytest.mark.gpu
TOL = 1e-4
VARIANTS = [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU, pcg.PCG_MASS_FLAT]


def _run(n, s, off, variant, n_part=None, use_layout=True):
    M = torch.zeros(n[2], n[1], n[0], 125, dtype=torch.float32, device=DEV)
    groups = None
    if use_layout:
        groups = pcg.Layout(T=1, order=2, tile_offsets=dev(off.view(np.int32)),
                            n_partitioned=s.count if n_part is None else n_part, drift=0)
    say("mass tsc", n, s.count, variant, n_part, use_layout)
    pcg.assemble_mass_matrix_scalar_tsc(n, [dev(a) for a in s.x], dev(s.q), dev(s.w), M, groups,
                                        variant)
    torch.cuda.synchronize()
    return M.cpu().numpy()


def _check(M, ref):
    assert rel_frob_err(M, ref) <= TOL
    assert np.abs(M - ref).max() <= TOL * np.abs(ref).max()


def _grouped(orc, wl):
    _, perm, off = orc.tile_sort(3, wl.n, 2, 1, wl.x)   # order 2, T = 1
    return wl.take(perm.astype(np.int64)), off


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n,ppc", [([5, 5, 5], 16), ([7, 6, 8], 64), ([6, 6, 6], 100)])
def test_tsc_mass_matches_oracle(orc, variant, n, ppc):
    """Uniform loading: support groups of varied size (several above 64 at ppc 64
    and 100 take a second, partial batch)."""
    wl = synthetic.mass_workload(n, ppc, w_uniform=True, seed=800 + ppc)
    s, off = _grouped(orc, wl)
    _check(_run(n, s, off, variant), orc.mass_matrix_scalar_tsc(n, wl.x, wl.q, wl.w))


@pytest.mark.parametrize("variant", [pcg.PCG_MASS_MFMA, pcg.PCG_MASS_VALU])
def test_tsc_mass_ragged_stale_and_tail(orc, variant):
    """Random positions with a crowded column, every 7th particle moved after the
    sort (found in another group's slice), and an unsorted tail of 400."""
    r = np.random.default_rng(81)
    n = [9, 8, 10]
    cnt = 5000
    x = [r.uniform(0, n[k], cnt).astype(np.float32) for k in range(3)]
    x[0][:1200] = r.uniform(2, 3, 1200).astype(np.float32)
    x[1][:1200] = r.uniform(4, 5, 1200).astype(np.float32)
    q = np.where(r.random(cnt) < 0.5, 1.0, -1.0).astype(np.float32)
    w = r.uniform(0.5, 1.5, cnt).astype(np.float32)
    z = np.zeros(cnt, np.float32)
    wl = synthetic.Workload(3, n, x, x, [z] * 3, q, w, [z] * 3, z)
    s, off = _grouped(orc, wl)
    s.x[0] = synthetic.periodic_shift(s.x[0], np.where(np.arange(cnt) % 7 == 0, 0.6, 0.0), n[0])
    M = _run(n, s, off, variant, n_part=cnt - 400)
    _check(M, orc.mass_matrix_scalar_tsc(n, s.x, s.q, s.w))


@pytest.mark.parametrize("scale", [1e-20, 1e15])
def test_tsc_mass_charge_scale(orc, scale):
    """The matrix-core path sums each brick of support groups in fixed point
    whose unit follows the brick's sum |q w|: charges far from 1 keep their
    relative precision."""
    wl = synthetic.mass_workload([8, 7, 6], 24, seed=85)
    s, off = _grouped(orc, wl)
    s.w = (s.w.astype(np.float64) * scale).astype(np.float32)
    _check(_run(wl.n, s, off, pcg.PCG_MASS_MFMA), orc.mass_matrix_scalar_tsc(wl.n, s.x, s.q, s.w))


def test_tsc_mass_adds_to_M(orc):
    """M += the matrix: a non-zero M keeps its values under the additions."""
    wl = synthetic.mass_workload([6, 5, 7], 16, seed=86)
    s, off = _grouped(orc, wl)
    init = np.random.default_rng(87).standard_normal((7, 5, 6, 125)).astype(np.float32)
    M = torch.from_numpy(init.copy()).to(DEV)
    groups = pcg.Layout(T=1, order=2, tile_offsets=dev(off.view(np.int32)), n_partitioned=s.count,
                        drift=0)
    pcg.assemble_mass_matrix_scalar_tsc(wl.n, [dev(a) for a in s.x], dev(s.q), dev(s.w), M, groups,
                                        pcg.PCG_MASS_MFMA)
    torch.cuda.synchronize()
    ref = orc.mass_matrix_scalar_tsc(wl.n, s.x, s.q, s.w)
    _check(M.cpu().numpy().astype(np.float64) - init, ref)


@pytest.mark.parametrize("variant", VARIANTS)
def test_tsc_mass_overwrite(orc, variant):
    """PCG_MASS_OVERWRITE: M is cleared before the additions, on every path."""
    wl = synthetic.mass_workload([6, 7, 5], 16, seed=88)
    s, off = _grouped(orc, wl)
    M = torch.from_numpy(np.random.default_rng(89).standard_normal(
        (5, 7, 6, 125)).astype(np.float32)).to(DEV)
    groups = pcg.Layout(T=1, order=2, tile_offsets=dev(off.view(np.int32)), n_partitioned=s.count,
                        drift=0)
    pcg.assemble_mass_matrix_scalar_tsc(wl.n, [dev(a) for a in s.x], dev(s.q), dev(s.w), M, groups,
                                        variant | pcg.PCG_MASS_OVERWRITE)
    torch.cuda.synchronize()
    _check(M.cpu().numpy(), orc.mass_matrix_scalar_tsc(wl.n, s.x, s.q, s.w))


def test_tsc_mass_no_layout_is_flat(orc):
    wl = synthetic.mass_workload([5, 6, 7], 9, seed=82)
    _check(_run(wl.n, wl, None, pcg.PCG_MASS_AUTO, use_layout=False),
           orc.mass_matrix_scalar_tsc(wl.n, wl.x, wl.q, wl.w))


def test_tsc_mass_full_size_64(orc):
    """64^3, 64 ppc on the matrix cores: rows of a z-slab against the oracle on the
    particles whose support base lies in the slab (node plane z receives from
    bases z-2 .. z), and every row's sum against sum_p q w W_pg (Eq.(11),
    numpy)."""
    wl = full_workload("mass_64_ppc64")
    s, off = _grouped(orc, wl)
    M = _run(wl.n, s, off, pcg.PCG_MASS_MFMA)
    z = wl.x[2].astype(np.float64)
    fl = np.floor(z)
    bz = np.where(z - fl < 0.5, fl - 1, fl)
    z0, z1 = 20, 30
    sub = wl.take(np.nonzero((bz >= z0) & (bz < z1))[0])
    ref = orc.mass_matrix_scalar_tsc(wl.n, sub.x, sub.q, sub.w)
    _check(M[z0 + 2:z1], ref[z0 + 2:z1])
    qw = s.q.astype(np.float64) * s.w
    want = node_row_sums(wl.n, s.x, 2, [qw])
    scale = node_row_sums(wl.n, s.x, 2, [np.abs(qw)])
    say("row sums: worst error / bound", check_row_sums(block_row_sums(M), want, scale, TOL))


def _run_tensor(n, s, off, variant, n_part=None, use_layout=True):
    M = torch.zeros(n[2], n[1], n[0], 125, 3, 3, dtype=torch.float32, device=DEV)
    groups = None
    if use_layout:
        groups = pcg.Layout(T=1, order=2, tile_offsets=dev(off.view(np.int32)),
                            n_partitioned=s.count if n_part is None else n_part, drift=0)
    say("mass tsc tensor", n, s.count, variant, n_part, use_layout)
    pcg.assemble_mass_matrix_tsc(n, [dev(a) for a in s.x], [dev(b) for b in s.B], dev(s.beta),
                                 dev(s.q), dev(s.w), M, groups, variant)
    torch.cuda.synchronize()
    return M.cpu().numpy()


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("n,ppc", [([5, 5, 5], 16), ([7, 6, 8], 64), ([6, 6, 6], 100)])
def test_tsc_tensor_mass_matches_oracle(orc, variant, n, ppc):
    wl = synthetic.mass_workload(n, ppc, w_uniform=True, seed=900 + ppc)
    s, off = _grouped(orc, wl)
    _check(_run_tensor(n, s, off, variant), orc.mass_matrix_tsc(n, wl.x, wl.B, wl.q, wl.w,
                                                                wl.beta))


def test_tsc_tensor_mass_stale_layout_and_tail(orc):
    wl = synthetic.mass_workload([8, 7, 9], 20, seed=91)
    s, off = _grouped(orc, wl)
    s.x[0] = synthetic.periodic_shift(s.x[0], np.where(np.arange(s.count) % 7 == 0, 0.6, 0.0),
                                      wl.n[0])
    M = _run_tensor(wl.n, s, off, pcg.PCG_MASS_MFMA, n_part=s.count - 300)
    _check(M, orc.mass_matrix_tsc(wl.n, s.x, s.B, s.q, s.w, s.beta))


def test_tsc_tensor_zero_field_is_scalar(orc):
    """B = 0: each diagonal component equals the scalar TSC matrix's kernel output
    to fp32 rounding, and the off-diagonal components vanish."""
    wl = synthetic.mass_workload([6, 6, 6], 16, seed=92)
    wl.B = [np.zeros_like(b) for b in wl.B]
    s, off = _grouped(orc, wl)
    Mt = _run_tensor(wl.n, s, off, pcg.PCG_MASS_MFMA)
    Ms = _run(wl.n, s, off, pcg.PCG_MASS_MFMA)
    assert np.abs(Mt[..., 0, 1]).max() <= 1e-6 * np.abs(Ms).max()
    for i in range(3):
        assert np.abs(Mt[..., i, i] - Ms).max() <= 1e-5 * np.abs(Ms).max()


def test_tsc_tensor_mass_large(orc):
    """24^3, 64 ppc (885K particles) on the matrix cores, every row against the
    oracle: thousands of groups and both batch paths, small enough for the
    single-threaded fp64 oracle."""
    wl = synthetic.mass_workload([24, 24, 24], 64, seed=93)
    s, off = _grouped(orc, wl)
    M = _run_tensor(wl.n, s, off, pcg.PCG_MASS_MFMA)
    _check(M, orc.mass_matrix_tsc(wl.n, wl.x, wl.B, wl.q, wl.w, wl.beta))


def test_tsc_tensor_mass_full_size_64(orc):
    """64^3, 64 ppc (16.8M particles), the launch the benchmark times.
    (1) Element-wise: the oracle runs on the particles whose support base lies
    in a 10^3 box of nodes straddling the periodic wrap on every axis (bases
    59..63, 0..4); the 8^3 node rows that only those bases reach (node g
    receives from bases g-2 .. g) are compared entry by entry.
    (2) Every row: block row sums of the trace, of the skew pair (0,1)-(1,0) and
    of the symmetric pair (0,2)+(2,0) against sum_p c_p W_pg (Eq.(11), numpy)."""
    wl = full_workload("mass_64_ppc64")
    s, off = _grouped(orc, wl)
    M = _run_tensor(wl.n, s, off, pcg.PCG_MASS_MFMA)
    box = (np.arange(64) >= 59) | (np.arange(64) < 5)
    inside = np.ones(s.count, bool)
    for k in range(3):
        base, _ = axis_weights(s.x[k], 64, 2)
        inside &= box[base]
    sub = s.take(np.nonzero(inside)[0])
    ref = orc.mass_matrix_tsc(wl.n, sub.x, sub.B, sub.q, sub.w, sub.beta)
    rows = np.r_[61:64, 0:5]
    ix = np.ix_(rows, rows, rows)
    _check(M[ix], ref[ix])
    del ref
    c = alpha_coefs(s)
    combos = [c[0] + c[4] + c[8], c[1] - c[3], c[2] + c[6]]
    want = node_row_sums(wl.n, s.x, 2, combos)
    scale = node_row_sums(wl.n, s.x, 2, [np.abs(c[0]) + np.abs(c[4]) + np.abs(c[8]),
                                         np.abs(c[1]) + np.abs(c[3]),
                                         np.abs(c[2]) + np.abs(c[6])])
    rs = block_row_sums(M)
    got = np.stack([rs[0] + rs[4] + rs[8], rs[1] - rs[3], rs[2] + rs[6]])
    say("row sums: worst error / bound", check_row_sums(got, want, scale, TOL))


@pytest.mark.parametrize("scale", [1e-20, 1e15])
def test_tsc_tensor_mass_charge_scale(orc, scale):
    """The tensor bricks sum in fixed point whose unit follows the brick's
    sum |q w| as well: charges far from 1 keep their relative precision."""
    wl = synthetic.mass_workload([7, 6, 5], 24, seed=94)
    s, off = _grouped(orc, wl)
    s.w = (s.w.astype(np.float64) * scale).astype(np.float32)
    _check(_run_tensor(wl.n, s, off, pcg.PCG_MASS_MFMA),
           orc.mass_matrix_tsc(wl.n, s.x, s.B, s.q, s.w, s.beta))


@pytest.mark.parametrize("field", [0.05, 20.0])
def test_tsc_tensor_mass_field_strength(orc, field):
    """Weak and strong rotation (|omega| from about 0.05 to 20 times the
    default): the rotation and omega omega^T terms of alpha dominate in turn,
    and both halves of every packed patch word carry large values."""
    wl = synthetic.mass_workload([5, 7, 6], 32, seed=95)
    wl.B = [(b.astype(np.float64) * field).astype(np.float32) for b in wl.B]
    s, off = _grouped(orc, wl)
    _check(_run_tensor(wl.n, s, off, pcg.PCG_MASS_MFMA),
           orc.mass_matrix_tsc(wl.n, wl.x, wl.B, wl.q, wl.w, wl.beta))


@pytest.mark.parametrize("variant", VARIANTS)
def test_tsc_tensor_mass_overwrite_and_add(orc, variant):
    """M += the matrix on a non-zero M, and PCG_MASS_OVERWRITE clears it first,
    on every path; grid edges of 9, 7, 5 leave partial bricks on every axis."""
    wl = synthetic.mass_workload([9, 7, 5], 12, seed=96)
    s, off = _grouped(orc, wl)
    ref = orc.mass_matrix_tsc(wl.n, s.x, s.B, s.q, s.w, s.beta)
    init = np.random.default_rng(97).standard_normal((5, 7, 9, 125, 3, 3)).astype(np.float32)
    groups = pcg.Layout(T=1, order=2, tile_offsets=dev(off.view(np.int32)), n_partitioned=s.count,
                        drift=0)
    for flags in (0, pcg.PCG_MASS_OVERWRITE):
        M = torch.from_numpy(init.copy()).to(DEV)
        say("mass tsc tensor on a non-zero M", wl.n, s.count, variant, flags)
        pcg.assemble_mass_matrix_tsc(wl.n, [dev(a) for a in s.x], [dev(b) for b in s.B],
                                     dev(s.beta), dev(s.q), dev(s.w), M, groups, variant | flags)
        torch.cuda.synchronize()
        got = M.cpu().numpy().astype(np.float64)
        _check(got if flags else got - init, ref)


@pytest.mark.parametrize("tensor", [False, True])
def test_tsc_mass_long_x_graded_weights(orc, tensor):
    """41 nodes along x: 11 scalar bricks or 21 tensor ones per row, the last one
    partial, and weights that grow along x by a factor of 100, so that
    neighbouring bricks, which add to the same node pairs, sum in fixed point of
    different units; the light end holds the tolerance against its own largest
    value."""
    wl = synthetic.mass_workload([41, 6, 5], 12, seed=98)
    grow = 10.0 ** (2.0 * wl.x[0].astype(np.float64) / 41)
    wl.w = (wl.w.astype(np.float64) * grow).astype(np.float32)
    s, off = _grouped(orc, wl)
    if tensor:
        M = _run_tensor(wl.n, s, off, pcg.PCG_MASS_MFMA)
        ref = orc.mass_matrix_tsc(wl.n, s.x, s.B, s.q, s.w, s.beta)
    else:
        M = _run(wl.n, s, off, pcg.PCG_MASS_MFMA)
        ref = orc.mass_matrix_scalar_tsc(wl.n, s.x, s.q, s.w)
    _check(M, ref)
    lo = (slice(None), slice(None), slice(2, 8))  # node columns x = 2 .. 7
    assert np.abs(M[lo] - ref[lo]).max() <= TOL * np.abs(ref[lo]).max()


@pytest.mark.parametrize("tensor", [False, True])
@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("case", ["empty", "all_tail"])
def test_tsc_mass_empty_and_all_tail(orc, tensor, variant, case):
    """No particles: M keeps its values when added to and is all zeros with
    PCG_MASS_OVERWRITE.  A layout that covers none of the particles (every one
    in the unsorted tail): the matrix still comes out whole."""
    wl = synthetic.mass_workload([6, 5, 7], 10, seed=99)
    s, off = _grouped(orc, wl)
    n_part = 0
    if case == "empty":
        s = s.take(np.arange(0))
        off = np.zeros_like(off)
    shape = (7, 5, 6, 125, 3, 3) if tensor else (7, 5, 6, 125)
    init = np.random.default_rng(100).standard_normal(shape).astype(np.float32)
    groups = pcg.Layout(T=1, order=2, tile_offsets=dev(off.view(np.int32)), n_partitioned=n_part,
                        drift=0)
    if s.count:
        ref = (orc.mass_matrix_tsc(wl.n, s.x, s.B, s.q, s.w, s.beta) if tensor
               else orc.mass_matrix_scalar_tsc(wl.n, s.x, s.q, s.w))
    for flags in (0, pcg.PCG_MASS_OVERWRITE):
        M = torch.from_numpy(init.copy()).to(DEV)
        say("mass tsc", case, "tensor" if tensor else "scalar", variant, flags)
        if tensor:
            pcg.assemble_mass_matrix_tsc(wl.n, [dev(a) for a in s.x], [dev(b) for b in s.B],
                                         dev(s.beta), dev(s.q), dev(s.w), M, groups,
                                         variant | flags)
        else:
            pcg.assemble_mass_matrix_scalar_tsc(wl.n, [dev(a) for a in s.x], dev(s.q), dev(s.w),
                                                M, groups, variant | flags)
        torch.cuda.synchronize()
        got = M.cpu().numpy().astype(np.float64)
        if not s.count:
            assert np.array_equal(got, np.zeros_like(got) if flags else init)
        else:
            _check(got if flags else got - init, ref)
