"""GPU tile sort vs the oracle: keys, permutation and offsets bit-exact, permuted
arrays exact ([TD] "The tile-based spatial sort")."""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import DEV, dev, full_workload, say, u32

pytestmark = pytest.mark.gpu


def _check_sort(orc, dim, n, order, T, x, arrays=()):
    say("sort", dim, n, order, T, x[0].size)
    perm, keys, off, outs = pcg.pcg_tile_sort(dim, n, order, T, [dev(a) for a in x],
                                              [dev(a) for a in arrays])
    torch.cuda.synchronize()
    k_ref, p_ref, o_ref = orc.tile_sort(dim, n, order, T, x)
    assert np.array_equal(u32(perm), p_ref)
    assert np.array_equal(u32(keys), k_ref[p_ref])
    assert np.array_equal(u32(off), o_ref)
    for a, o in zip(arrays, outs):
        assert np.array_equal(o.cpu().numpy(), a[p_ref])
    return p_ref, o_ref


@pytest.mark.parametrize("dim,n,order,T,ppc", [
    (1, [256], 1, 4, 20),
    (2, [64, 64], 1, 8, 4),
    (2, [48, 32], 2, 16, 3),
    (3, [32, 32, 32], 1, 8, 3),
    (3, [32, 32, 32], 2, 4, 2),
    (3, [32, 32, 32], 2, 16, 2),
    (3, [16, 16, 16], 1, 1, 5),       # cell layout (mass matrix)
    (3, [64, 64, 64], 1, 64, 1),      # a single tile: identity permutation
])
def test_sort_uniform(orc, dim, n, order, T, ppc):
    wl = synthetic.deposit_workload(dim, n, ppc=ppc, seed=100 + dim * 10 + T)
    _check_sort(orc, dim, n, order, T, wl.x, wl.x + wl.v + [wl.q, wl.w])


@pytest.mark.parametrize("count", [1, 2, 63, 4095, 4097, 10007, 123457])
def test_sort_ragged_counts(orc, count):
    r = np.random.default_rng(count)
    n = [24, 16, 32]
    x = [r.uniform(0, n[k], count).astype(np.float32) for k in range(3)]
    for k in range(3):
        x[k][x[k] >= n[k]] = 0
    _check_sort(orc, 3, n, 2, 8, x, [x[0], x[1]])


def test_sort_empty(orc):
    say("sort empty")
    x = [torch.empty(0, dtype=torch.float32, device=DEV) for _ in range(3)]
    perm, keys, off, _ = pcg.pcg_tile_sort(3, [16, 16, 16], 1, 8, x, [])
    torch.cuda.synchronize()
    assert perm.numel() == 0 and (off.cpu() == 0).all() and off.numel() == 9


def test_sort_skewed_all_in_one_tile(orc):
    r = np.random.default_rng(5)
    x = [r.uniform(8, 15.99, 50000).astype(np.float32) for _ in range(3)]
    _check_sort(orc, 3, [64, 64, 64], 1, 8, x, [x[2]])


def test_sort_nearly_sorted_steady_state(orc):
    """Re-sorting pushed particles that were sorted one step earlier (the every-step case)."""
    wl = synthetic.workload("cic3d_128_ppc32", dict(n=[64, 64, 64], ppc=8))
    k, p, o = orc.tile_sort(3, wl.n, 1, 8, wl.x)
    s = wl.take(p.astype(np.int64))
    _check_sort(orc, 3, wl.n, 1, 8, s.x_next, s.x_next + s.v + [s.q, s.w])


@pytest.mark.parametrize("ordered", [0.0, 0.4, 0.6, 1.0])
def test_sort_moves_arrays_by_gather_or_scatter(orc, ordered):
    """The arrays are moved by gather for an unordered input and by scatter
    through the inverse permutation where at least half of the neighbouring
    particles share a tile: inputs whose leading fraction `ordered` is in tile
    order (the rest shuffled) fall on both sides of that choice, and every
    array must come out exactly as the oracle's stable sort puts it."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=4, seed=131)
    _, p, _ = orc.tile_sort(3, wl.n, 1, 8, wl.x)
    order = p.astype(np.int64)
    cut = int(ordered * order.size)
    order[cut:] = np.random.default_rng(132).permutation(order[cut:])
    s = wl.take(order)
    _check_sort(orc, 3, wl.n, 1, 8, s.x, s.x + s.v + [s.q, s.w])


def test_sort_deterministic_repeat(orc):
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=4, seed=77)
    x = [dev(a) for a in wl.x]
    say("sort repeat")
    res = [pcg.pcg_tile_sort(3, wl.n, 2, 8, x, [])[0].cpu() for _ in range(3)]
    assert all(torch.equal(res[0], r) for r in res[1:])


def test_sort_full_size_cic3d_128(orc):
    """The headline workload's size: 67.1M particles, 4096 tiles (shuffled input)."""
    wl = full_workload("cic3d_128_ppc32")
    _check_sort(orc, 3, wl.n, 1, 8, wl.x)


def test_sort_full_size_mass_cells(orc):
    """16.8M particles into 262,144 cells (the mass-matrix layout)."""
    wl = full_workload("mass_64_ppc64")
    _check_sort(orc, 3, wl.n, 1, 1, wl.x, [wl.beta])


# ---------------------------------------------------------------- incremental path

def _check_resort(orc, wl, order, T, prev_off, x, arrays, expect_same=True, n_part=None):
    """Sort x (currently grouped by prev_off) with the previous layout given;
    the result must equal the oracle's stable sort of x exactly."""
    say("resort", wl.dim, wl.n, order, T, x[0].size)
    cnt = x[0].size
    prev = pcg.Layout(T=T, order=order, tile_offsets=dev(prev_off.view(np.int32)),
                      n_partitioned=cnt if n_part is None else n_part)
    perm, keys, off, outs = pcg.pcg_tile_sort(wl.dim, wl.n, order, T, [dev(a) for a in x],
                                              [dev(a) for a in arrays], prev=prev)
    torch.cuda.synchronize()
    k_ref, p_ref, o_ref = orc.tile_sort(wl.dim, wl.n, order, T, x)
    assert np.array_equal(u32(perm), p_ref)
    assert np.array_equal(u32(keys), k_ref[p_ref])
    assert np.array_equal(u32(off), o_ref)
    for a, o in zip(arrays, outs):
        assert np.array_equal(o.cpu().numpy(), a[p_ref])


def _sorted_state(orc, wl, order, T):
    _, p, o = orc.tile_sort(wl.dim, wl.n, order, T, wl.x)
    return wl.take(p.astype(np.int64)), o


@pytest.mark.parametrize("dim,n,order,T,ppc", [
    (3, [32, 32, 32], 1, 8, 4),
    (3, [32, 32, 32], 2, 4, 2),
    (2, [64, 64], 1, 8, 6),
    (2, [64, 32], 2, 16, 6),
    (3, [16, 8, 64], 1, 8, 4),     # 2 and 1 tiles along x and y
    (3, [24, 24, 24], 1, 1, 2),    # cell layout
])
def test_resort_steady_state(orc, dim, n, order, T, ppc):
    wl = synthetic.deposit_workload(dim, n, ppc=ppc, far_fraction=0.02, seed=600 + T + dim)
    s, off = _sorted_state(orc, wl, order, T)
    _check_resort(orc, s, order, T, off, s.x_next, s.x_next + s.v + [s.q, s.w])


@pytest.mark.parametrize("dim,n,order,T,ppc", [
    (3, [32, 32, 32], 1, 8, 4),
    (2, [64, 64], 1, 8, 6),
    (3, [24, 24, 24], 1, 1, 2),    # cell layout (the small-chunk move)
])
def test_resort_positions_among_arrays(orc, dim, n, order, T, ppc):
    """The keyed positions passed again as moved arrays (the same device
    tensors, as a step re-sorting its own state does): the move takes them
    from registers and must still give the oracle's stable order."""
    wl = synthetic.deposit_workload(dim, n, ppc=ppc, far_fraction=0.02, seed=640 + T + dim)
    s, off = _sorted_state(orc, wl, order, T)
    say("resort aliased", dim, n, order, T, s.count)
    fields = s.x_next + s.v + [s.q, s.w]
    cur = [dev(a) for a in fields]
    prev = pcg.Layout(T=T, order=order, tile_offsets=dev(off.view(np.int32)),
                      n_partitioned=s.count)
    perm, keys, noff, outs = pcg.pcg_tile_sort(dim, n, order, T, cur[:dim], cur, prev=prev)
    torch.cuda.synchronize()
    k_ref, p_ref, o_ref = orc.tile_sort(dim, n, order, T, s.x_next)
    assert np.array_equal(u32(perm), p_ref)
    assert np.array_equal(u32(noff), o_ref)
    for a, o in zip(fields, outs):
        assert np.array_equal(o.cpu().numpy(), a[p_ref])


def test_resort_far_moves_fall_back(orc):
    """Particles that moved more than one tile raise the device flag; the radix
    path then produces the same stable result."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=2, far_fraction=0.1, seed=610)
    s, off = _sorted_state(orc, wl, 1, 2)   # tiles of 2 cells: 2-4 cell pushes leave the stencil
    _check_resort(orc, s, 1, 2, off, s.x_next, [s.q])


def test_resort_invalid_prev_falls_back(orc):
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=2, seed=611)
    s, off = _sorted_state(orc, wl, 1, 8)
    bad = off.copy()
    bad[5], bad[6] = bad[6], bad[5]              # not monotone
    _check_resort(orc, s, 1, 8, bad, s.x_next, [s.w])
    bad = off.copy()
    bad[-1] -= 3                                 # does not cover every particle
    _check_resort(orc, s, 1, 8, bad, s.x_next, [s.w])


def test_resort_with_tail_uses_general_path(orc):
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=2, seed=612)
    s, off = _sorted_state(orc, wl, 1, 8)
    _check_resort(orc, s, 1, 8, off, s.x_next, [s.w], n_part=s.count - 7)


def test_resort_heavy_tiles(orc):
    wl = synthetic.deposit_workload(3, [64, 64, 64], count=600_000,
                                    blob=dict(sigma=3.0, overdensity=400.0), seed=613)
    s, off = _sorted_state(orc, wl, 2, 8)
    assert np.diff(off.astype(np.int64)).max() > 4 * 4096
    _check_resort(orc, s, 2, 8, off, s.x_next, s.x_next + [s.q])


def test_resort_full_size_cic3d_128(orc):
    """The bench step's sort: 67.1M pushed particles re-sorted from their layout."""
    wl = full_workload("cic3d_128_ppc32")
    s, off = _sorted_state(orc, wl, 1, 8)
    _check_resort(orc, s, 1, 8, off, s.x_next, [s.x_next[0], s.q])


@pytest.mark.parametrize("use_prev", [True, False])
def test_sort_without_keys_or_perm(orc, use_prev):
    """sorted_keys and perm are optional outputs: the same offsets and permuted
    arrays without them, on both the single-pass and the radix path."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=3, seed=614)
    s, off = _sorted_state(orc, wl, 1, 8)
    prev = (pcg.Layout(T=8, order=1, tile_offsets=dev(off.view(np.int32)), n_partitioned=s.count)
            if use_prev else None)
    say("sort without keys/perm", use_prev)
    perm, keys, o, outs = pcg.pcg_tile_sort(3, wl.n, 1, 8, [dev(a) for a in s.x_next],
                                            [dev(s.q), dev(s.x_next[1])], prev=prev,
                                            want_keys=False, want_perm=False)
    torch.cuda.synchronize()
    _, p_ref, o_ref = orc.tile_sort(3, wl.n, 1, 8, s.x_next)
    assert keys is None and perm is None
    assert np.array_equal(u32(o), o_ref)
    assert np.array_equal(outs[0].cpu().numpy(), s.q[p_ref])
    assert np.array_equal(outs[1].cpu().numpy(), s.x_next[1][p_ref])
