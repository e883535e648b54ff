"""GPU deposit + regroup in one pass (deposit_currents_regroup) vs the fp64 oracle.

J: max |J_gpu - J_oracle| <= 1e-5 max |J_oracle|; escape count, new tile
offsets and every regrouped array: bit-exact against the oracle's stable tile
sort of the pushed positions ([TD] "How a tile deposit runs", "The tile-based
spatial sort").
"""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import DEV, component_errors, dev, full_workload, host, rel_max_err, say

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _J(n):
    n3 = list(n) + [1] * (3 - len(n))
    return torch.zeros(3, n3[2], n3[1], n3[0], dtype=torch.float32, device=DEV)


def _sorted_pushed(orc, wl, order, T):
    """Grouped by the tiles of x (oracle sort), then pushed to x_next."""
    _, p, o = orc.tile_sort(wl.dim, wl.n, order, T, wl.x)
    return wl.take(p.astype(np.int64)), o


def _fields(s):
    return list(s.x_next) + list(s.v) + [s.q, s.w]


def _run(s, order, T, D, off, arrays=None, n_part=None, block=0):
    dim = s.dim
    xs = [dev(a) for a in s.x_next]
    vs = [dev(a) for a in s.v]
    q, w = dev(s.q), dev(s.w)
    if arrays is None:
        arrs = xs + vs + [q, w]
    else:
        arrs = [dev(a) for a in arrays]
    J = _J(s.n)
    esc = torch.zeros(1, dtype=torch.int64, device=DEV)
    lay = pcg.Layout(T=T, order=order, tile_offsets=dev(off.view(np.int32)),
                     n_partitioned=s.count if n_part is None else n_part, drift=D, block=block)
    say("deposit_currents_regroup", dim, s.n, order, T, D, s.count, n_part, len(arrs))
    off_new, outs = pcg.deposit_currents_regroup(dim, s.n, order, xs, vs, q, w, J, lay, arrs,
                                                 n_escaped=esc)
    torch.cuda.synchronize()
    return host(J), int(esc.item()), host(off_new).view(np.uint32), [host(o) for o in outs]


def _check(orc, s, order, T, D, off, got, arrays=None, n_part=None):
    J, esc, off_new, outs = got
    ref = orc.deposit(s.dim, s.n, order, s.x_next, s.v, s.q, s.w)
    comp = component_errors(J, ref)
    say("regroup: rel err", rel_max_err(J, ref), "per component", comp)
    assert rel_max_err(J, ref) <= TOL and max(comp) <= TOL
    n_ref, _ = orc.escape(s.dim, s.n, order, T, D, s.x_next, off, n_part)
    assert esc == n_ref
    _, p, o = orc.tile_sort(s.dim, s.n, order, T, s.x_next)
    assert np.array_equal(off_new, o)
    src = _fields(s) if arrays is None else arrays
    for a, b in zip(outs, src):
        assert np.array_equal(a.view(np.uint32), b[p].view(np.uint32))
    return n_ref


@pytest.mark.parametrize("dim,n,order,T,D,far", [
    (1, [512], 1, 8, 1, 0.05),
    (2, [64, 64], 1, 8, 1, 0.02),
    (2, [64, 48], 2, 8, 2, 0.02),
    (3, [32, 32, 32], 1, 8, 1, 0.02),
    (3, [32, 32, 32], 1, 4, 0, 0.0),
    (3, [32, 32, 32], 2, 4, 1, 0.02),
    (3, [32, 32, 32], 2, 8, 1, 0.02),
    (3, [24, 16, 32], 1, 8, 2, 0.05),
])
def test_regroup_matches_oracle(orc, dim, n, order, T, D, far):
    ppc = {1: 40, 2: 6, 3: 3}[dim]
    wl = synthetic.deposit_workload(dim, n, ppc=ppc, far_fraction=far, w_uniform=True,
                                    seed=500 + dim * 10 + order + T)
    s, off = _sorted_pushed(orc, wl, order, T)
    n_esc = _check(orc, s, order, T, D, off, _run(s, order, T, D, off))
    if D == 0 or far > 0:
        assert n_esc > 0  # the escape valve ran inside the fused pass


def test_heavy_tiles_span_many_chunks(orc):
    """Tiles of ~100k particles: deposit chunks cover dozens of sort chunks."""
    wl = synthetic.deposit_workload(3, [16, 16, 16], ppc=200, far_fraction=0.01,
                                    w_uniform=True, seed=531)
    s, off = _sorted_pushed(orc, wl, 1, 8)
    assert np.diff(off).max() > 32768
    _check(orc, s, 1, 8, 1, off, _run(s, 1, 8, 1, off))


def test_far_moves_fall_back_to_the_general_sort(orc):
    """Moves of 2-4 cells cross more than one tile of edge 2: the device flag
    hands the regrouping to the radix path; the deposit still runs fused."""
    wl = synthetic.deposit_workload(3, [16, 16, 16], ppc=4, far_fraction=0.05, seed=532)
    s, off = _sorted_pushed(orc, wl, 1, 2)
    _check(orc, s, 1, 2, 1, off, _run(s, 1, 2, 1, off))


def test_queues_overflow(orc):
    """Most particles pushed 2-4 cells with tiles of edge 4: a chunk holds more
    tile-leavers than the work-group stages in LDS (1024) and more escapes than
    its queue of global deposits (512); the rest are stored and deposited
    directly."""
    wl = synthetic.deposit_workload(3, [16, 16, 16], ppc=64, far_fraction=0.9, w_uniform=True,
                                    seed=536)
    s, off = _sorted_pushed(orc, wl, 1, 4)
    n_esc = _check(orc, s, 1, 4, 1, off, _run(s, 1, 4, 1, off))
    chunks = 64 * 2  # 64 tiles of 4096 particles, chunks of 2048
    assert n_esc > chunks * 512
    leavers = int(np.sum(orc.tile_keys(3, s.n, 1, 4, s.x) != orc.tile_keys(3, s.n, 1, 4, s.x_next)))
    assert leavers > chunks * 1024


def test_other_arrays_take_the_generic_store(orc):
    """Arrays other than exactly (x, v, q, w) in order: extra fields, another order."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=3, far_fraction=0.02, seed=533)
    s, off = _sorted_pushed(orc, wl, 1, 8)
    ids = np.arange(s.count, dtype=np.int32).view(np.float32)
    arrays = [s.q, ids] + list(s.x_next) + [s.w] + list(s.v)
    got = _run(s, 1, 8, 1, off, arrays=arrays)
    _check(orc, s, 1, 8, 1, off, got, arrays=arrays)
    assert np.array_equal(np.sort(got[3][1].view(np.int32)), np.arange(s.count))


def test_tail_runs_deposit_then_sort(orc):
    """A layout that leaves a tail: the two stages run one after the other."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=3, far_fraction=0.02, seed=534)
    s, off = _sorted_pushed(orc, wl, 1, 8)
    n_part = s.count - 777
    _check(orc, s, 1, 8, 1, off, _run(s, 1, 8, 1, off, n_part=n_part), n_part=n_part)


def test_empty(orc):
    e = [np.zeros(0, np.float32)] * 3
    s = synthetic.Workload(3, [32, 32, 32], e, e, e, e[0], e[0])
    J, esc, off_new, outs = _run(s, 1, 8, 1, np.zeros(65, np.uint32))
    assert not J.any() and esc == 0 and not off_new.any()


def test_deterministic_regroup(orc):
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=4, far_fraction=0.02, seed=535)
    s, off = _sorted_pushed(orc, wl, 1, 8)
    a = _run(s, 1, 8, 1, off)
    b = _run(s, 1, 8, 1, off)
    assert np.array_equal(a[2], b[2]) and a[1] == b[1]
    assert all(np.array_equal(x, y) for x, y in zip(a[3], b[3]))


def test_full_size_cic3d_128_step(orc):
    """The benchmark's step at full size (67.1M particles, 128^3, T = 8, drift 1):
    J vs the oracle; offsets, arrays and escapes exact."""
    wl = full_workload("cic3d_128_ppc32")
    s, off = _sorted_pushed(orc, wl, 1, 8)
    got = _run(s, 1, 8, 1, off)
    n_esc = _check(orc, s, 1, 8, 1, off, got)
    say("full-size fused step: escaped", n_esc)
    assert n_esc > 0
