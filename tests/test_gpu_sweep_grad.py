"""GPU reverse of the 1-D sweep (dL/dx0 for a given dL/dH) vs the oracle ([CS]
"Code": the gradient of sum (H - target)^2 with respect to x0).

Tolerance: both sides take the window and bin decisions in fp64 without fused
multiply-adds and add each particle's steps in the same order, so the selected
set is identical and max |dx0_gpu - dx0_oracle| <= 1e-13 max |dx0_oracle| covers
any difference in the fp64 library routines (division, floor, rint)."""
import numpy as np
import pytest
import torch

import particle_cell_grid_amd as pcg
import synthetic
from gpu_util import DEV, dev, say

pytestmark = pytest.mark.gpu
TOL = 1e-13


def _grad(nb, x0, v, T, dt, hw, dH):
    x0 = np.asarray(x0, np.float64)
    dx0 = torch.full((x0.size,), 7.0, dtype=torch.float64, device=DEV)   # overwritten
    say("sweep grad", nb, x0.size, T)
    pcg.deposit_sweep1d_grad(nb, dev(x0), dev(np.asarray(v, np.float64)), T, dt, hw,
                             dev(np.asarray(dH, np.float64)), dx0)
    torch.cuda.synchronize()
    return dx0.cpu().numpy()


def _check(got, ref):
    assert ((got != 0) == (ref != 0)).all()     # same particles selected
    scale = np.abs(ref).max()
    assert np.abs(got - ref).max() <= TOL * (scale if scale > 0 else 1.0)


def _seed(orc, nb, s, r):
    """dL/dH of the page's loss at the oracle's H, for a random target."""
    H = orc.sweep1d(nb, s.x0, s.v, s.T, s.dt, s.hw)
    return 2.0 * (H - r.random(nb))


def test_sweep_grad_workload(orc):
    """The page's set-up: 2000 particles, 50 steps, 1024 bins."""
    s = synthetic.workload("sweep1d_2000")
    dH = _seed(orc, s.nb, s, np.random.default_rng(90))
    ref = orc.sweep1d_grad(s.nb, s.x0, s.v, s.T, s.dt, s.hw, dH)
    _check(_grad(s.nb, s.x0, s.v, s.T, s.dt, s.hw, dH), ref)
    assert np.count_nonzero(ref) > 100


def test_sweep_grad_from_gpu_forward(orc):
    """Forward and reverse on the GPU: dL/dH from the GPU's fp32 histogram, the
    same seed given to the oracle's reverse."""
    s = synthetic.sweep_workload(count=5000, seed=91)
    H = torch.empty(s.nb, dtype=torch.float32, device=DEV)
    pcg.deposit_sweep1d(s.nb, dev(s.x0), dev(s.v), s.T, s.dt, s.hw, H)
    target = np.random.default_rng(92).random(s.nb)
    dH = 2.0 * (H.cpu().numpy().astype(np.float64) - target)
    ref = orc.sweep1d_grad(s.nb, s.x0, s.v, s.T, s.dt, s.hw, dH)
    _check(_grad(s.nb, s.x0, s.v, s.T, s.dt, s.hw, dH), ref)


def test_sweep_grad_large_count(orc):
    """10^6 particles (several work-groups per CU, grid-stride), every entry."""
    s = synthetic.sweep_workload(count=1_000_000, seed=93)
    dH = np.random.default_rng(94).normal(0.0, 1.0, s.nb)
    ref = orc.sweep1d_grad(s.nb, s.x0, s.v, s.T, s.dt, s.hw, dH)
    _check(_grad(s.nb, s.x0, s.v, s.T, s.dt, s.hw, dH), ref)


@pytest.mark.parametrize("nb,count,T,hw", [(7, 257, 13, 0.2), (16384, 3000, 50, 0.001),
                                           (1, 100, 5, 0.5), (64, 1, 200, 0.3),
                                           (64, 300, 5000, 0.02), (16384, 200, 4000, 0.001)])
def test_sweep_grad_odd_shapes(orc, nb, count, T, hw):
    """Odd bin counts (both bins wrap to 0 at nb = 1; 128 KiB of LDS at 16384),
    a ragged particle count, one particle over many steps; more steps than the
    per-step table holds, and a table that does not fit beside 16384 fp64 bins
    (both computed inline)."""
    r = np.random.default_rng(95 + nb)
    x0 = r.random(count)
    v = r.normal(0.0, 0.3, count)
    dH = r.normal(0.0, 1.0, nb)
    ref = orc.sweep1d_grad(nb, x0, v, T, 0.02, hw, dH)
    _check(_grad(nb, x0, v, T, 0.02, hw, dH), ref)


def test_sweep_grad_zero_steps_and_empty():
    """No steps: dx0 is overwritten with zeros; no particles: nothing is touched."""
    g = _grad(16, [0.1, 0.7], [0.0, 0.1], 0, 0.02, 0.1, np.ones(16))
    assert (g == 0).all()
    dx0 = torch.full((0,), 1.0, dtype=torch.float64, device=DEV)
    pcg.deposit_sweep1d_grad(16, torch.empty(0, dtype=torch.float64, device=DEV),
                             torch.empty(0, dtype=torch.float64, device=DEV), 5, 0.02, 0.1,
                             torch.zeros(16, dtype=torch.float64, device=DEV), dx0)
    torch.cuda.synchronize()


def test_sweep_loss_grad_composite(orc):
    """The one-call forward + seed + reverse: H matches the oracle's forward to the
    forward entry's tolerance (its fp32 atomics add in no fixed order), and dx0
    equals the oracle's reverse seeded from that fp32 H (and, to the fp32
    rounding of H, from the oracle's own fp64 H)."""
    s = synthetic.workload("sweep1d_2000")
    target = np.random.default_rng(96).random(s.nb)
    H = torch.full((s.nb,), 7.0, dtype=torch.float32, device=DEV)
    dx0 = torch.full((s.x0.size,), 7.0, dtype=torch.float64, device=DEV)
    say("sweep loss grad", s.nb, s.x0.size, s.T)
    pcg.deposit_sweep1d_loss_grad(s.nb, dev(s.x0), dev(s.v), s.T, s.dt, s.hw, dev(target), H, dx0)
    torch.cuda.synchronize()
    Hg, g = H.cpu().numpy(), dx0.cpu().numpy()
    Ho = orc.sweep1d(s.nb, s.x0, s.v, s.T, s.dt, s.hw)
    assert np.abs(Hg - Ho).max() <= 1e-5 * np.abs(Ho).max()
    assert ((Hg != 0) == (Ho != 0)).all()
    ref = orc.sweep1d_grad(s.nb, s.x0, s.v, s.T, s.dt, s.hw,
                           2.0 * (Hg.astype(np.float64) - target))
    _check(g, ref)
    ref64 = orc.sweep1d_grad(s.nb, s.x0, s.v, s.T, s.dt, s.hw, 2.0 * (Ho - target))
    assert np.abs(g - ref64).max() <= 1e-5 * np.abs(ref64).max()
