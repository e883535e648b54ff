"""GPU charge-conserving zigzag deposit (tiled and flat) vs the fp64 oracle.

Tolerance: max |J_gpu - J_oracle| <= 1e-5 max |J_oracle| over the whole array
(fp32 products and atomics against fp64).  Escape counts are compared exactly
with a classifier written here from the window's definition.  ([TD] "Halo
sizing" for the scheme and its stencil, "How a tile deposit runs" for the tiled
form, "Correctness is independent of the halo" for the escape valve.)
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
    return torch.zeros(3, n[2], n[1], n[0], dtype=torch.float32, device=DEV)


def _inputs(n, ppc, seed, max_step=0.95):
    wl = synthetic.deposit_workload(3, n, ppc=ppc, w_uniform=True, seed=seed)
    x = wl.x
    xp = synthetic.previous_positions(x, max_step=max_step, seed=seed + 1)
    return x, xp, wl.q, wl.w


def _sorted(orc, n, T, key, arrays):
    """Oracle tile sort (order 1) keyed on `key`; returns the permuted arrays
    and the tile offsets."""
    _, p, off = orc.tile_sort(3, n, 1, T, key)
    p = p.astype(np.int64)
    return [a[p] for a in arrays], off


def _expected_escapes(n, T, D, key, x, xp):
    """Particles whose stencil min(i1, i2) .. max(i1, i2) + 1 per axis does not
    fit the window of TE = T + 2D + 3 nodes starting D + 1 below the origin of
    the tile holding `key`."""
    TE = T + 2 * D + 3
    esc = np.zeros(x[0].size, dtype=bool)
    for k in range(3):
        i1 = np.floor(xp[k].astype(np.float64)).astype(np.int64)
        i2 = np.floor(x[k].astype(np.float64)).astype(np.int64)
        lo = np.minimum(i1, i2)
        ext = np.maximum(i1, i2) + 1 - lo
        ws = (np.floor(key[k].astype(np.float64)).astype(np.int64) // T) * T - D - 1
        l0 = np.mod(lo - ws, n[k])
        esc |= (l0 + ext >= TE) | (ext > 2)
    return int(esc.sum())


def _run(n, x, xp, q, w, layout=None):
    J = _J(n)
    esc = torch.zeros(1, dtype=torch.int64, device=DEV)
    pcg.deposit_currents_zigzag(n, [dev(a) for a in x], [dev(a) for a in xp], dev(q), dev(w), J,
                                layout, esc)
    torch.cuda.synchronize()
    return J.cpu().numpy(), int(esc.item())


def _layout(T, D, off, n_part):
    return pcg.Layout(T=T, order=1, tile_offsets=dev(off.view(np.int32)), n_partitioned=n_part,
                      drift=D)


@pytest.mark.parametrize("n,T,D", [
    ([32, 32, 32], 8, 1),
    ([32, 32, 32], 4, 0),
    ([24, 16, 32], 8, 2),
    ([16, 16, 16], 16, 1),   # the int64 window exceeds the LDS: fp32 sums
])
def test_tiled_matches_oracle(orc, n, T, D):
    x, xp, q, w = _inputs(n, 3, seed=700 + T + D)
    (x0, x1, x2, p0, p1, p2, q, w), off = _sorted(orc, n, T, x, [*x, *xp, q, w])
    x, xp = [x0, x1, x2], [p0, p1, p2]
    say("zigzag tiled", n, T, D, x0.size)
    J, esc = _run(n, x, xp, q, w, _layout(T, D, off, x0.size))
    ref = orc.deposit_zigzag(n, x, xp, q, w)
    assert rel_max_err(J, ref) <= TOL
    assert esc == 0  # keyed on the new positions: every move under a cell fits


@pytest.mark.parametrize("D", [0, 1, 2])
def test_stale_layout_escapes(orc, D):
    """A layout keyed on positions up to 2.5 cells off for 10% of the particles:
    those whose stencil leaves the window take the valve and are counted."""
    n, T = [32, 32, 32], 8
    x, xp, q, w = _inputs(n, 2, seed=720 + D)
    key = synthetic.stale_keys(x, n, fraction=0.1, span=2.5, seed=730 + D)
    (x0, x1, x2, p0, p1, p2, k0, k1, k2, q, w), off = _sorted(orc, n, T, key,
                                                             [*x, *xp, *key, q, w])
    x, xp, key = [x0, x1, x2], [p0, p1, p2], [k0, k1, k2]
    say("zigzag stale", n, T, D, x0.size)
    J, esc = _run(n, x, xp, q, w, _layout(T, D, off, x0.size))
    ref = orc.deposit_zigzag(n, x, xp, q, w)
    assert rel_max_err(J, ref) <= TOL
    expect = _expected_escapes(n, T, D, key, x, xp)
    assert esc == expect
    assert expect > 0  # the valve was exercised


@pytest.mark.parametrize("heavy_w", [40.0, 1e5])
def test_scale_redo_with_escapes(orc, heavy_w):
    """The fixed-point scale comes from the first particle of each thread; a
    tile holding a later particle with |q w| above twice that is deposited
    again at its true maximum.  One heavy particle per tile past its first 256,
    on a stale layout so that the same tiles also send particles to the valve
    (which the second pass must not deposit or count again).  At w = 40 a
    window not cleared or an escape deposited twice shows at 1e-3 or more; at
    w = 1e5 the first scale would overflow int64 had the tile not been redone."""
    n, T, D = [16, 16, 16], 8, 1
    x, xp, q, w = _inputs(n, 4, seed=760)
    key = synthetic.stale_keys(x, n, fraction=0.1, span=2.5, seed=761)
    (x0, x1, x2, p0, p1, p2, k0, k1, k2, q, w), off = _sorted(orc, n, T, key,
                                                             [*x, *xp, *key, q, w])
    x, xp, key = [x0, x1, x2], [p0, p1, p2], [k0, k1, k2]
    w = np.full_like(w, 0.5)
    heavy = [int(off[t]) + 300 for t in range(off.size - 1) if off[t + 1] - off[t] > 300]
    assert len(heavy) == off.size - 1
    w[heavy] = heavy_w
    say("zigzag scale redo", n, T, D, x0.size)
    J, esc = _run(n, x, xp, q, w, _layout(T, D, off, x0.size))
    ref = orc.deposit_zigzag(n, x, xp, q, w)
    assert rel_max_err(J, ref) <= TOL
    expect = _expected_escapes(n, T, D, key, x, xp)
    assert esc == expect and expect > 0


def test_flat_and_tail(orc):
    """No layout (flat kernel), and a layout over a prefix with the ragged rest
    sent to the flat kernel."""
    n, T = [24, 20, 16], 4
    x, xp, q, w = _inputs(n, 2, seed=740)
    say("zigzag flat", n, x[0].size)
    J, esc = _run(n, x, xp, q, w)
    ref = orc.deposit_zigzag(n, x, xp, q, w)
    assert rel_max_err(J, ref) <= TOL and esc == 0
    m = x[0].size - 1237
    head, off = _sorted(orc, n, T, [a[:m] for a in x], [a[:m] for a in [*x, *xp, q, w]])
    rest = [a[m:] for a in [*x, *xp, q, w]]
    x0, x1, x2, p0, p1, p2, qq, ww = [np.concatenate([h, r]) for h, r in zip(head, rest)]
    say("zigzag tail", n, T, m, x0.size)
    J, esc = _run(n, [x0, x1, x2], [p0, p1, p2], qq, ww, _layout(T, 1, off, m))
    assert rel_max_err(J, ref) <= TOL and esc == 0


def test_edge_cases(orc):
    """No particles; one particle on a 1x1x1-tile grid whose move crosses the
    periodic boundary on every axis; particles at rest (no current)."""
    n = [8, 8, 8]
    e = np.zeros(0, np.float32)
    say("zigzag empty")
    J, esc = _run(n, [e] * 3, [e] * 3, e, e)
    assert not J.any() and esc == 0
    x = [np.array([0.2], np.float32)] * 3
    xp = [np.array([-0.4], np.float32)] * 3
    q = np.array([-1.0], np.float32)
    w = np.array([1.25], np.float32)
    off = np.array([0] + [1] * 8, np.uint32)   # 2x2x2 tiles of T = 4; the particle in tile 0
    say("zigzag boundary crossing")
    J, esc = _run(n, x, xp, q, w, _layout(4, 0, off, 1))
    ref = orc.deposit_zigzag(n, x, xp, q, w)
    assert rel_max_err(J, ref) <= TOL and esc == 0
    xs, _, q2, w2 = _inputs(n, 1, seed=750)
    say("zigzag at rest")
    J, _ = _run(n, xs, xs, q2, w2)
    assert not J.any()


@pytest.mark.parametrize("D", [0, 1])
def test_full_size_parity(orc, D):
    """3-D 128^3 with 32 per cell (the headline loading), each particle moved by
    its velocity: the tiled launch (T = 8; drift 0 as benchmarked, and 1)
    against the oracle over the whole array, and the total current
    sum_g J_c = sum_p q w (x - x_prev)_c."""
    wl = full_workload("cic3d_128_ppc32")
    n, T = wl.n, 8
    x = wl.x
    xp = synthetic.previous_positions(x, scale_v=1.0, v=wl.v)
    # grouped by the previous positions (wrapped into the grid), as a step
    # finds them after the last sort
    key = [np.mod(a, np.float32(n[k])).astype(np.float32) for k, a in enumerate(xp)]
    key = [np.where(a >= n[k], np.float32(0), a) for k, a in enumerate(key)]
    _, p, off = orc.tile_sort(3, n, 1, T, key)
    p = p.astype(np.int64)
    x, xp = [a[p] for a in x], [a[p] for a in xp]
    q, w = wl.q[p], wl.w[p]
    say("zigzag full", n, T, D, x[0].size)
    J, esc = _run(n, x, xp, q, w, _layout(T, D, off, x[0].size))
    assert esc == 0
    ref = orc.deposit_zigzag(n, x, xp, q, w)
    assert rel_max_err(J, ref) <= TOL
    qw = q.astype(np.float64) * w
    for c in range(3):
        tot = float((qw * (x[c].astype(np.float64) - xp[c])).sum())
        scale = float(np.abs(qw * (x[c].astype(np.float64) - xp[c])).sum())
        assert abs(float(J[c].astype(np.float64).sum()) - tot) <= 1e-6 * scale


# ---------------------------------------------------------------- fused pass

def _run_fused(n, T, D, x, xp, q, w, off, n_part=None, arrays=None):
    """deposit_currents_zigzag_regroup with the layout `off` (the particles'
    current grouping): J, escapes, the new offsets and the regrouped arrays."""
    xs, xps = [dev(a) for a in x], [dev(a) for a in xp]
    qd, wd = dev(q), dev(w)
    arrs = xs + xps + [qd, wd] if arrays is None else [dev(a) for a in arrays]
    J = _J(n)
    esc = torch.zeros(1, dtype=torch.int64, device=DEV)
    lay = _layout(T, D, off, x[0].size if n_part is None else n_part)
    say("zigzag fused", n, T, D, x[0].size, n_part, len(arrs))
    off_new, outs = pcg.deposit_currents_zigzag_regroup(n, xs, xps, qd, wd, J, lay, arrs,
                                                        n_escaped=esc)
    torch.cuda.synchronize()
    return (J.cpu().numpy(), int(esc.item()), off_new.cpu().numpy().view(np.uint32),
            [o.cpu().numpy() for o in outs])


def _check_fused(orc, n, T, D, key, x, xp, q, w, off, got, arrays=None):
    """J vs the oracle; escapes vs the window rule; the new layout and every
    regrouped array bit for bit against the oracle's stable sort of x."""
    J, esc, off_new, outs = got
    ref = orc.deposit_zigzag(n, x, xp, q, w)
    comp = component_errors(J, ref)
    say("zigzag fused: rel err", rel_max_err(J, ref), "per component", comp)
    assert rel_max_err(J, ref) <= TOL and max(comp) <= TOL
    assert esc == _expected_escapes(n, T, D, key, x, xp)
    _, p, o = orc.tile_sort(3, n, 1, T, x)
    assert np.array_equal(off_new, o)
    src = [*x, *xp, q, w] if arrays is None else arrays
    for a, b in zip(outs, src):
        assert np.array_equal(a.view(np.uint32), b[p].view(np.uint32))
    return esc


def _grouped_by_prev(orc, n, T, x, xp, q, w):
    """The particles grouped by the tiles of their previous positions (wrapped
    into the grid), as the last step's sort left them."""
    key = [np.mod(a, np.float32(n[k])).astype(np.float32) for k, a in enumerate(xp)]
    key = [np.where(a >= n[k], np.float32(0), a) for k, a in enumerate(key)]
    _, p, off = orc.tile_sort(3, n, 1, T, key)
    p = p.astype(np.int64)
    return [a[p] for a in key], [a[p] for a in x], [a[p] for a in xp], q[p], w[p], off


@pytest.mark.parametrize("n,T,D", [
    ([32, 32, 32], 8, 0),
    ([32, 32, 32], 8, 1),
    ([32, 32, 32], 4, 0),
    ([24, 16, 32], 8, 2),
    ([32, 32, 32], 16, 1),   # fp32 window sums: deposit, then the sort's own move
])
def test_fused_matches_oracle(orc, n, T, D):
    x, xp, q, w = _inputs(n, 6, seed=770 + T + D)
    key, x, xp, q, w, off = _grouped_by_prev(orc, n, T, x, xp, q, w)
    got = _run_fused(n, T, D, x, xp, q, w, off)
    _check_fused(orc, n, T, D, key, x, xp, q, w, off, got)
    moved = orc.tile_keys(3, n, 1, T, x) != orc.tile_keys(3, n, 1, T, key)
    assert moved.sum() > 0       # particles change tile: the move's leaver path ran


def test_fused_heavy_tiles_and_queue_overflow(orc):
    """Tiles of edge 2 holding 2400 particles, most of which change tile: more
    leavers than the work-group's LDS queue (1024) takes; then one tile of
    204,800 particles (100 chunks for 8 waves)."""
    n = [8, 8, 8]
    x, xp, q, w = _inputs(n, 300, seed=781)
    key, x, xp, q, w, off = _grouped_by_prev(orc, n, 2, x, xp, q, w)
    leavers = orc.tile_keys(3, n, 1, 2, x) != orc.tile_keys(3, n, 1, 2, key)
    assert leavers.sum() > 64 * 1100   # over 1024 per tile on average
    _check_fused(orc, n, 2, 0, key, x, xp, q, w, off, _run_fused(n, 2, 0, x, xp, q, w, off))
    x, xp, q, w = _inputs([8, 8, 8], 400, seed=782)
    key, x, xp, q, w, off = _grouped_by_prev(orc, [8, 8, 8], 8, x, xp, q, w)
    assert np.diff(off.astype(np.int64)).max() > 16 * 2048
    _check_fused(orc, [8, 8, 8], 8, 1, key, x, xp, q, w, off,
                 _run_fused([8, 8, 8], 8, 1, x, xp, q, w, off))


@pytest.mark.parametrize("heavy_w", [40.0, 1e5])
def test_fused_scale_redo(orc, heavy_w):
    """The fused step's tiles take their fixed-point scale from the first
    particle of each thread; one heavy particle per tile past its first 512
    makes every tile deposit again at its true maximum (no second move).  At
    w = 1e5 the first scale would put that particle's contributions far past
    the int32 range, so it must add nothing on the first pass."""
    n, T, D = [32, 32, 32], 8, 1
    x, xp, q, w = _inputs(n, 6, seed=786)
    key, x, xp, q, w, off = _grouped_by_prev(orc, n, T, x, xp, q, w)
    w = np.full_like(w, 0.5)
    heavy = [int(off[t]) + 600 for t in range(off.size - 1) if off[t + 1] - off[t] > 600]
    assert len(heavy) == off.size - 1
    w[heavy] = heavy_w
    say("zigzag fused scale redo", n, T, D, x[0].size, heavy_w)
    _check_fused(orc, n, T, D, key, x, xp, q, w, off, _run_fused(n, T, D, x, xp, q, w, off))


def test_fused_stale_layout_falls_back_to_the_general_sort(orc):
    """A layout three tiles stale: the deposit takes the escape valve for most
    particles and the device flag hands the regrouping to the radix path."""
    n, T = [32, 32, 32], 4
    x, xp, q, w = _inputs(n, 3, seed=783)
    key = [np.mod(a + np.float32(3 * T), np.float32(n[k])).astype(np.float32)
           for k, a in enumerate(x)]
    _, p, off = orc.tile_sort(3, n, 1, T, key)
    p = p.astype(np.int64)
    key, x, xp, q, w = [a[p] for a in key], [a[p] for a in x], [a[p] for a in xp], q[p], w[p]
    esc = _check_fused(orc, n, T, 1, key, x, xp, q, w, off, _run_fused(n, T, 1, x, xp, q, w, off))
    assert esc > x[0].size // 2


def test_fused_tail_and_other_arrays(orc):
    """A tail, and arrays other than exactly (x, x_prev, q, w): the deposit and
    the sort run one after the other, with the same results."""
    n, T = [32, 32, 32], 8
    x, xp, q, w = _inputs(n, 3, seed=784)
    key, x, xp, q, w, off = _grouped_by_prev(orc, n, T, x, xp, q, w)
    cnt = x[0].size
    got = _run_fused(n, T, 0, x, xp, q, w, off, n_part=cnt - 321)
    J, esc, off_new, outs = got
    assert rel_max_err(J, orc.deposit_zigzag(n, x, xp, q, w)) <= TOL
    _, p, o = orc.tile_sort(3, n, 1, T, x)
    assert np.array_equal(off_new, o)
    ids = np.arange(cnt, dtype=np.int32).view(np.float32)
    arrays = [q, ids, *x, w]
    got = _run_fused(n, T, 0, x, xp, q, w, off, arrays=arrays)
    _check_fused(orc, n, T, 0, key, x, xp, q, w, off, got, arrays=arrays)


def test_fused_empty(orc):
    n = [8, 8, 8]
    e = np.zeros(0, np.float32)
    J, esc, off_new, outs = _run_fused(n, 4, 0, [e] * 3, [e] * 3, e, e, np.zeros(9, np.uint32))
    assert not J.any() and esc == 0 and not off_new.any()


def test_fused_full_size_step(orc):
    """The zigzag step the benchmark times, at full size (67.1M particles,
    128^3, T = 8, drift 0): J vs the oracle over the whole array; the new
    layout and all eight regrouped arrays bit for bit."""
    wl = full_workload("cic3d_128_ppc32")
    n, T = wl.n, 8
    xp = synthetic.previous_positions(wl.x, scale_v=1.0, v=wl.v)
    key, x, xp, q, w, off = _grouped_by_prev(orc, n, T, wl.x, xp, wl.q, wl.w)
    got = _run_fused(n, T, 0, x, xp, q, w, off)
    esc = _check_fused(orc, n, T, 0, key, x, xp, q, w, off, got)
    assert esc == 0
