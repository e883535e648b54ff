"""GPU fused 1-D windowed sweep vs the oracle ([CS] "The problem", "Code").
Tolerance: max |H_gpu - H_oracle| <= 1e-5 max |H_oracle|; the window test and
bin index are fp64 decisions on both sides."""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import DEV, dev, rel_max_err, say

pytestmark = pytest.mark.gpu


def _run(nb, x0, v, T, dt, hw):
    H = torch.full((nb,), 7.0, dtype=torch.float32, device=DEV)   # overwritten
    say("sweep", nb, len(x0), T)
    pcg.deposit_sweep1d(nb, dev(np.asarray(x0, np.float64)), dev(np.asarray(v, np.float64)), T,
                        dt, hw, H)
    torch.cuda.synchronize()
    return H.cpu().numpy()


def test_sweep_workload(orc):
    s = synthetic.workload("sweep1d_2000")
    H = _run(s.nb, s.x0, s.v, s.T, s.dt, s.hw)
    ref = orc.sweep1d(s.nb, s.x0, s.v, s.T, s.dt, s.hw)
    assert rel_max_err(H, ref) <= 1e-5
    assert ((H != 0) == (ref != 0)).all()      # same bins selected


def test_large_count(orc):
    s = synthetic.sweep_workload(count=1_000_000, seed=61)
    H = _run(s.nb, s.x0, s.v, s.T, s.dt, s.hw)
    ref = orc.sweep1d(s.nb, s.x0, s.v, s.T, s.dt, s.hw)
    assert rel_max_err(H, ref) <= 1e-5


@pytest.mark.parametrize("nb,T,hw", [(7, 13, 0.2), (16384, 50, 0.001), (1, 5, 0.5),
                                     (64, 5000, 0.02), (16384, 4000, 0.001)])
def test_odd_shapes(orc, nb, T, hw):
    s = synthetic.sweep_workload(count=5000, nb=nb, T=T, hw=hw, seed=62)
    H = _run(nb, s.x0, s.v, T, s.dt, hw)
    ref = orc.sweep1d(nb, s.x0, s.v, T, s.dt, hw)
    assert rel_max_err(H, ref) <= 1e-5


def test_hand_cases(orc):
    H = _run(1024, [0.5, 1 / 4096], [0.0, 0.0], 50, 0.02, 0.005)
    exp = np.zeros(1024)
    exp[511] = exp[512] = 0.5
    wt = (1 - 0.048828125) ** 2
    exp[1023] += 0.25 * wt
    exp[0] += 0.75 * wt
    assert np.allclose(H, exp, rtol=1e-6, atol=0)


def test_empty_and_zero_steps(orc):
    assert not _run(64, [], [], 50, 0.02, 0.005).any()
    assert not _run(64, [0.5], [0.0], 0, 0.02, 0.005).any()
