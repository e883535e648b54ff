"""deposit_currents_noalloc (static scratch, no workspace argument) against
deposit_currents with a workspace, on the GPU: two calls in a row, the second
smaller, each checked to the deposit tolerance (max |dJ| <= 1e-5 max |J|) with
bit-equal escape counts.  The scratch keeps the first call's map; the second
must not depend on it."""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import DEV, dev, rel_max_err, say

pytestmark = pytest.mark.gpu


def _both(orc, dim, n, order, T, D, ppc, far, seed):
    wl = synthetic.deposit_workload(dim, n, ppc=ppc, far_fraction=far, w_uniform=True, seed=seed)
    _, perm, off = orc.tile_sort(dim, wl.n, order, T, wl.x)
    s = wl.take(perm.astype(np.int64))
    xs = [dev(a) for a in s.x_next]
    vs = [dev(a) for a in s.v]
    q, w = dev(s.q), dev(s.w)
    n3 = list(n) + [1] * (3 - len(n))
    lay = pcg.Layout(T=T, order=order, tile_offsets=dev(off.view(np.int32)),
                     n_partitioned=s.count - 37, drift=D)       # with an unsorted tail
    out = []
    for fn in (pcg.deposit_currents, pcg.deposit_currents_noalloc):
        J = torch.zeros(3, n3[2], n3[1], n3[0], dtype=torch.float32, device=DEV)
        esc = torch.zeros(1, dtype=torch.int64, device=DEV)
        say(fn.__name__, dim, n, order, T, D, s.count)
        fn(dim, wl.n, order, xs, vs, q, w, J, lay, esc)
        torch.cuda.synchronize()
        out.append((J.cpu().numpy(), int(esc.item())))
    (J0, e0), (J1, e1) = out
    assert e1 == e0
    assert rel_max_err(J1, J0.astype(np.float64)) <= 1e-5
    ref = orc.deposit(dim, wl.n, order, s.x_next, s.v, s.q, s.w)
    assert rel_max_err(J1, ref) <= 1e-5
    return e0


def test_noalloc_matches_deposit_currents_twice(orc):
    e = _both(orc, 3, [32, 32, 32], 1, 8, 1, 8, 0.03, 1201)
    assert e > 0                                   # the escape valve ran
    _both(orc, 3, [16, 16, 16], 1, 4, 1, 4, 0.03, 1202)   # smaller: fewer tiles and items


def test_noalloc_tsc_2d_and_flat(orc):
    _both(orc, 2, [64, 48], 2, 8, 1, 12, 0.02, 1203)
    wl = synthetic.deposit_workload(3, [8, 8, 8], ppc=3, seed=1204)
    J = torch.zeros(3, 8, 8, 8, dtype=torch.float32, device=DEV)
    say("deposit_currents_noalloc flat")
    pcg.deposit_currents_noalloc(3, wl.n, 1, [dev(a) for a in wl.x_next], [dev(a) for a in wl.v],
                                 dev(wl.q), dev(wl.w), J, None)
    torch.cuda.synchronize()
    assert rel_max_err(J.cpu().numpy(), orc.deposit(3, wl.n, 1, wl.x_next, wl.v, wl.q,
                                                    wl.w)) <= 1e-5
