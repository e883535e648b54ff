"""GPU tile sort vs the oracle: keys, permutation and offsets bit-exact, permuted
arrays exact ([TD] "The tile-based spatial sort")."""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import DEV, dev, full_config, say, u32

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
    wl = synthetic.config(3, dict(n=[64, 64, 64], ppc=8))
    k, p, o = orc.tile_sort(3, wl.n, 1, 8, wl.x)
    s = wl.take(p.astype(np.int64))
    _check_sort(orc, 3, wl.n, 1, 8, s.x_next, s.x_next + s.v + [s.q, s.w])


def test_sort_deterministic_repeat(orc):
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=4, seed=77)
    x = [dev(a) for a in wl.x]
    say("sort repeat")
    res = [pcg.pcg_tile_sort(3, wl.n, 2, 8, x, [])[0].cpu() for _ in range(3)]
    assert all(torch.equal(res[0], r) for r in res[1:])


def test_sort_full_size_config3(orc):
    """The headline workload's size: 67.1M particles, 4096 tiles (shuffled input)."""
    wl = full_config(3)
    _check_sort(orc, 3, wl.n, 1, 8, wl.x)


def test_sort_full_size_config5_cells(orc):
    """16.8M particles into 262,144 cells (the mass-matrix layout)."""
    wl = full_config(5)
    _check_sort(orc, 3, wl.n, 1, 1, wl.x, [wl.beta])
