"""GPU current deposit (tiled and flat) vs the fp64 oracle.

Tolerance: max |J_gpu - J_oracle| <= 1e-5 max |J_oracle| over the whole array.
Escape counts are compared bit-exactly with the oracle's classifier.
([TD] "How a tile deposit runs", "Correctness is independent of the halo",
"Coverage: the tail pass and the first step".)
"""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import DEV, component_errors, dev, full_workload, rel_max_err, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _J(n):
    n3 = list(n) + [1] * (3 - len(n))
    return torch.zeros(3, n3[2], n3[1], n3[0], dtype=torch.float32, device=DEV)


def _sorted_pushed(orc, wl, order, T):
    """Oracle-sorted on x, pushed to x_next (input preparation for the tiled path)."""
    k, p, o = orc.tile_sort(wl.dim, wl.n, order, T, wl.x)
    return wl.take(p.astype(np.int64)), o


def _run_tiled(wl, order, T, D, offsets, n_part=None, block=0):
    dim = wl.dim
    xs = [dev(a) for a in wl.x_next]
    vs = [dev(a) for a in wl.v]
    J = _J(wl.n)
    esc = torch.zeros(1, dtype=torch.int64, device=DEV)
    lay = pcg.Layout(T=T, order=order, tile_offsets=dev(offsets.view(np.int32)),
                     n_partitioned=wl.count if n_part is None else n_part, drift=D, block=block)
    say("deposit tiled", dim, wl.n, order, T, D, wl.count, n_part, block)
    pcg.deposit_currents(dim, wl.n, order, xs, vs, dev(wl.q), dev(wl.w), J, lay, esc)
    torch.cuda.synchronize()
    return J.cpu().numpy(), int(esc.item())


@pytest.mark.parametrize("dim,n,order,T,D,far", [
    (1, [512], 1, 8, 1, 0.05),
    (1, [512], 2, 4, 1, 0.05),
    (2, [64, 64], 1, 8, 1, 0.02),
    (2, [64, 48], 2, 8, 2, 0.02),
    (3, [32, 32, 32], 1, 8, 1, 0.02),
    (3, [32, 32, 32], 1, 4, 0, 0.0),
    (3, [32, 32, 32], 2, 4, 1, 0.02),
    (3, [32, 32, 32], 2, 8, 1, 0.02),
    (3, [32, 32, 32], 2, 16, 1, 0.02),
    (3, [24, 16, 32], 1, 8, 2, 0.05),
])
def test_tiled_matches_oracle(orc, dim, n, order, T, D, far):
    ppc = {1: 40, 2: 6, 3: 3}[dim]
    wl = synthetic.deposit_workload(dim, n, ppc=ppc, far_fraction=far, w_uniform=True,
                                    seed=200 + dim * 10 + order + T)
    s, off = _sorted_pushed(orc, wl, order, T)
    J, esc = _run_tiled(s, order, T, D, off)
    ref = orc.deposit(dim, wl.n, order, s.x_next, s.v, s.q, s.w)
    n_ref, _ = orc.escape(dim, wl.n, order, T, D, s.x_next, off)
    assert rel_max_err(J, ref) <= TOL
    assert esc == n_ref
    if D == 0 or far > 0:
        assert n_ref > 0  # the escape valve was exercised


@pytest.mark.parametrize("dim,order", [(2, 1), (3, 1), (3, 2), (1, 2)])
def test_flat_matches_oracle(orc, dim, order):
    n = {1: [300], 2: [40, 50], 3: [20, 24, 16]}[dim]
    wl = synthetic.deposit_workload(dim, n, ppc=3, w_uniform=True, seed=300 + dim + order)
    J = _J(n)
    say("deposit flat", dim, order, wl.count)
    pcg.deposit_currents(dim, n, order, [dev(a) for a in wl.x_next], [dev(a) for a in wl.v],
                         dev(wl.q), dev(wl.w), J, None)
    torch.cuda.synchronize()
    ref = orc.deposit(dim, n, order, wl.x_next, wl.v, wl.q, wl.w)
    assert rel_max_err(J.cpu().numpy(), ref) <= TOL


def test_tail_pass(orc):
    """Particles past n_partitioned are deposited by the flat kernel; escapes are
    counted among the partitioned slots only."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=3, far_fraction=0.03, seed=41)
    s, off = _sorted_pushed(orc, wl, 1, 8)
    npart = wl.count * 2 // 3
    J, esc = _run_tiled(s, 1, 8, 1, off, n_part=npart)
    ref = orc.deposit(3, wl.n, 1, s.x_next, s.v, s.q, s.w)
    n_ref, _ = orc.escape(3, wl.n, 1, 8, 1, s.x_next, off, n_part=npart)
    assert rel_max_err(J, ref) <= TOL and esc == n_ref


def test_stale_layout_still_correct(orc):
    """A layout that does not describe the particles (sorted on other positions):
    every misplaced particle takes the escape valve and J is still exact."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=3, seed=42)
    other = synthetic.deposit_workload(3, [32, 32, 32], ppc=3, seed=43)
    _, _, off = orc.tile_sort(3, wl.n, 1, 8, other.x)
    J, esc = _run_tiled(wl, 1, 8, 1, off)
    ref = orc.deposit(3, wl.n, 1, wl.x_next, wl.v, wl.q, wl.w)
    n_ref, _ = orc.escape(3, wl.n, 1, 8, 1, wl.x_next, off)
    assert rel_max_err(J, ref) <= TOL and esc == n_ref and n_ref > wl.count // 2


@pytest.mark.parametrize("block", [64, 128, 512, 1024])
def test_block_sizes(orc, block):
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=4, far_fraction=0.02, seed=44)
    s, off = _sorted_pushed(orc, wl, 2, 8)
    J, esc = _run_tiled(s, 2, 8, 1, off, block=block)
    ref = orc.deposit(3, wl.n, 2, s.x_next, s.v, s.q, s.w)
    n_ref, _ = orc.escape(3, wl.n, 2, 8, 1, s.x_next, off)
    assert rel_max_err(J, ref) <= TOL and esc == n_ref


def test_heavy_tiles_split_into_chunks(orc):
    """A dense blob: tiles far above the chunk size are split over several
    work-groups (each with its own scratch and flush); empty tiles own none."""
    wl = synthetic.deposit_workload(3, [64, 64, 64], count=400_000,
                                    blob=dict(sigma=3.0, overdensity=400.0), w_uniform=True,
                                    seed=45)
    s, off = _sorted_pushed(orc, wl, 2, 8)
    assert np.diff(off.astype(np.int64)).max() > 8 * 2048
    J, esc = _run_tiled(s, 2, 8, 1, off)
    ref = orc.deposit(3, wl.n, 2, s.x_next, s.v, s.q, s.w)
    assert rel_max_err(J, ref) <= TOL and esc == 0


def test_single_particle_and_empty(orc):
    x = [np.float32([31.75]), np.float32([0.25]), np.float32([16.5])]
    v = [np.float32([1.0]), np.float32([-2.0]), np.float32([0.5])]
    q, w = np.float32([1.0]), np.float32([3.0])
    wl = synthetic.Workload(3, [32, 32, 32], x, x, v, q, w)
    _, _, off = orc.tile_sort(3, wl.n, 2, 8, x)
    J, esc = _run_tiled(wl, 2, 8, 1, off)
    ref = orc.deposit(3, wl.n, 2, x, v, q, w)
    assert rel_max_err(J, ref) <= TOL and esc == 0
    e = [np.zeros(0, np.float32)] * 3
    wl0 = synthetic.Workload(3, [32, 32, 32], e, e, e, e[0], e[0])
    J0, esc0 = _run_tiled(wl0, 2, 8, 1, np.zeros(65, np.uint32))
    assert not J0.any() and esc0 == 0


# ---------------------------------------------------------------- full sizes

def _full(orc, name, order, T, D=1):
    wl = full_workload(name)
    s, off = _sorted_pushed(orc, wl, order, T)
    return wl, s, off


def test_full_size_cic2d_512(orc):
    wl, s, off = _full(orc, "cic2d_512_ppc16", 1, 8)
    J, esc = _run_tiled(s, 1, 8, 1, off)
    ref = orc.deposit(2, wl.n, 1, s.x_next, s.v, s.q, s.w)
    comp = component_errors(J, ref)
    say("cic2d_512 rel err", rel_max_err(J, ref), "per component", comp)
    assert rel_max_err(J, ref) <= TOL and max(comp) <= TOL and esc == 0


def test_full_size_cic3d_128(orc):
    """Headline workload: 128^3, 32 ppc, 67.1M particles, 2% displaced 2-4 cells."""
    wl, s, off = _full(orc, "cic3d_128_ppc32", 1, 8)
    J, esc = _run_tiled(s, 1, 8, 1, off)
    ref = orc.deposit(3, wl.n, 1, s.x_next, s.v, s.q, s.w)
    n_ref, _ = orc.escape(3, wl.n, 1, 8, 1, s.x_next, off)
    err = rel_max_err(J, ref)
    comp = component_errors(J, ref)
    say("cic3d_128 rel err", err, "per component", comp, "escaped", esc, n_ref)
    assert err <= TOL and max(comp) <= TOL and esc == n_ref and n_ref > 0


_TSC_REF = {}


@pytest.mark.parametrize("T", [4, 8, 16])
def test_full_size_tsc3d_blob(orc, T):
    """Clustered TSC workload (33.5M particles), tile edge swept over {4, 8, 16}."""
    wl = full_workload("tsc3d_128_blob")
    s, off = _sorted_pushed(orc, wl, 2, T)
    J, esc = _run_tiled(s, 2, T, 1, off)
    if "ref" not in _TSC_REF:
        _TSC_REF["ref"] = orc.deposit(3, wl.n, 2, wl.x_next, wl.v, wl.q, wl.w)
    err, comp = rel_max_err(J, _TSC_REF["ref"]), component_errors(J, _TSC_REF["ref"])
    say("tsc3d_128_blob T", T, "rel err", err, "per component", comp)
    assert err <= TOL and max(comp) <= TOL and esc == 0


# ---------------------------------------------------------------- magnitudes

def test_tiny_charges_keep_relative_precision(orc):
    """SI-like scales (q w ~ 1e-19): the per-work-group fixed-point scale adapts,
    so the relative error stays at fp32 level."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=3, far_fraction=0.02, seed=46)
    wl.q = (wl.q * np.float32(1.6e-19)).astype(np.float32)
    s, off = _sorted_pushed(orc, wl, 1, 8)
    J, esc = _run_tiled(s, 1, 8, 1, off)
    ref = orc.deposit(3, wl.n, 1, s.x_next, s.v, s.q, s.w)
    n_ref, _ = orc.escape(3, wl.n, 1, 8, 1, s.x_next, off)
    assert rel_max_err(J, ref) <= TOL and esc == n_ref


def test_mixed_magnitudes_in_one_tile(orc):
    """Particles 1e6 x larger or 1e-9 x smaller than a tile's first batch, and a
    first batch with zero velocity: they leave the fixed-point range and are
    deposited through the valve (not counted as escapes); J stays exact."""
    wl = synthetic.deposit_workload(3, [16, 16, 16], ppc=8, w_uniform=True, seed=47)
    s, off = _sorted_pushed(orc, wl, 1, 8)
    w = s.w.copy()
    v = [a.copy() for a in s.v]
    for t in range(len(off) - 1):
        lo, hi = int(off[t]), int(off[t + 1])
        n = hi - lo
        if t % 2 == 0:
            for c in range(3):
                v[c][lo:lo + min(256, n)] = 0.0          # all-zero first batch
        w[lo + n // 2: lo + n // 2 + 5] *= np.float32(1e6)
        w[lo + n // 3: lo + n // 3 + 5] *= np.float32(1e-9)
    s.w, s.v = w, v
    J, esc = _run_tiled(s, 1, 8, 1, off)
    ref = orc.deposit(3, wl.n, 1, s.x_next, s.v, s.q, s.w)
    n_ref, _ = orc.escape(3, wl.n, 1, 8, 1, s.x_next, off)
    assert rel_max_err(J, ref) <= TOL and esc == n_ref


def test_tiled_is_deterministic(orc):
    """In-tile sums are exact integers, so repeated deposits agree bit for bit
    wherever a node is covered by a single tile window."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=4, seed=48)
    s, off = _sorted_pushed(orc, wl, 1, 8)
    J1, e1 = _run_tiled(s, 1, 8, 1, off)
    J2, e2 = _run_tiled(s, 1, 8, 1, off)
    assert e1 == e2 == 0
    # with drift 1 the window of the tile at origin o spans nodes o-1 .. o+9;
    # nodes o+2 .. o+6 (local index 2..6 on every axis) lie in that window only
    a = J1.reshape(3, 4, 8, 4, 8, 4, 8)[:, :, 2:7, :, 2:7, :, 2:7]
    b = J2.reshape(3, 4, 8, 4, 8, 4, 8)[:, :, 2:7, :, 2:7, :, 2:7]
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- 32-bit sums

def _crowded_cell(n, order, count_bg, count_cell, cell, seed):
    """A sparse uniform background plus one cell holding `count_cell` particles
    that all carry the same current: the tile's mean density is low, so its
    32-bit sums are sized for few particles per cell and the per-cell count
    cannot rule out an overflow -- the work-group re-runs its chunk into wider
    sums."""
    r = np.random.default_rng(seed)
    dim = len(n)
    x = [r.uniform(0, n[k], count_bg).astype(np.float32) for k in range(dim)]
    for k in range(dim):
        x[k] = np.concatenate([x[k], (cell[k] + r.uniform(0.05, 0.95, count_cell))
                               .astype(np.float32)])
    cnt = count_bg + count_cell
    v = [np.concatenate([r.normal(0, 0.1, count_bg), np.full(count_cell, 0.45)])
         .astype(np.float32) for _ in range(3)]
    q = np.ones(cnt, np.float32)
    w = np.ones(cnt, np.float32)
    return synthetic.Workload(dim, list(n), x, [a.copy() for a in x], v, q, w)


@pytest.mark.parametrize("dim,n,order,T,crowd", [
    (3, [16, 16, 16], 1, 8, 400),    # runs again at a lower scale
    (3, [16, 16, 16], 1, 8, 3000),   # runs again into 64-bit sums
    (2, [32, 32], 1, 8, 3000),
    (3, [32, 32, 32], 2, 16, 3000),  # 64-bit sums do not fit the LDS: fp32 sums
])
def test_overflow_guard_reruns_the_chunk(orc, dim, n, order, T, crowd):
    cell = [T // 2] * dim
    wl = _crowded_cell(n, order, 400, crowd, cell, seed=49 + dim + order)
    s, off = _sorted_pushed(orc, wl, order, T)
    J, esc = _run_tiled(s, order, T, 1, off)
    ref = orc.deposit(dim, wl.n, order, s.x_next, s.v, s.q, s.w)
    n_ref, _ = orc.escape(dim, wl.n, order, T, 1, s.x_next, off)
    assert rel_max_err(J, ref) <= TOL and esc == n_ref
    # the crowded cell's nodes carry ~crowd x 0.45 / 2^dim each: far beyond
    # the range the 32-bit sums were first sized for
    assert np.abs(ref).max() > crowd * 0.45 / 2 ** dim / 2
