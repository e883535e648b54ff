"""The seeded generators: reproducible, in range, and shaped like the workloads
the pages describe (uniform ppc, |v| < 1, balanced charge, far-displaced subset,
Gaussian blob, and the 1-D window statistics)."""
import json
import os

import numpy as np

import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_reproducible():
    a = synthetic.deposit_workload(3, [16, 16, 16], ppc=4, far_fraction=0.05, seed=3)
    b = synthetic.deposit_workload(3, [16, 16, 16], ppc=4, far_fraction=0.05, seed=3)
    for k in range(3):
        assert np.array_equal(a.x[k], b.x[k]) and np.array_equal(a.x_next[k], b.x_next[k])
    assert np.array_equal(a.q, b.q)


def test_uniform_ppc_and_ranges():
    wl = synthetic.deposit_workload(3, [16, 12, 8], ppc=5, seed=4)
    n = wl.n
    for k in range(3):
        assert wl.x[k].dtype == np.float32
        assert (wl.x[k] >= 0).all() and (wl.x[k] < n[k]).all()
        assert (wl.x_next[k] >= 0).all() and (wl.x_next[k] < n[k]).all()
    cell = (np.floor(wl.x[0]).astype(int) + n[0] * (np.floor(wl.x[1]).astype(int)
                                                    + n[1] * np.floor(wl.x[2]).astype(int)))
    assert (np.bincount(cell, minlength=16 * 12 * 8) == 5).all()
    speed = np.sqrt(sum(v.astype(np.float64) ** 2 for v in wl.v))
    assert speed.max() < 1.0
    assert wl.q.sum() == 0 and set(np.unique(wl.q)) == {-1.0, 1.0}


def test_push_is_velocity_except_far_subset():
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=4, far_fraction=0.02, seed=5)
    n = np.array(wl.n)[:, None]
    d = np.stack(wl.x_next).astype(np.float64) - np.stack(wl.x)
    d = d - n * np.round(d / n)                      # minimum image
    vel = np.stack(wl.v)[:3].astype(np.float64)
    near = np.abs(d - vel).max(axis=0) < 1e-4
    far = ~near
    assert abs(far.mean() - 0.02) < 0.002
    length = np.sqrt((d[:, far] ** 2).sum(axis=0))
    assert length.min() > 2.0 - 1e-3 and length.max() < 4.0 + 1e-3
    assert np.abs(d[:, near]).max() < 1.0


def test_blob_overdensity():
    wl = synthetic.deposit_workload(3, [64, 64, 64], count=2_000_000,
                                    blob=dict(sigma=5.0, overdensity=20.0), seed=6)
    c = np.floor(np.stack(wl.x)).astype(int)
    h = np.zeros((64, 64, 64))
    np.add.at(h, (c[2], c[1], c[0]), 1)
    centre = h[30:34, 30:34, 30:34].mean()
    corner = h[:8, :8, :8].mean()
    # peak density ~ (1 + 20) x background, averaged over the 4^3 central cells
    assert 14 < centre / corner < 22


def test_mass_inputs():
    wl = synthetic.mass_workload([8, 8, 8], 16, seed=7)
    assert np.array_equal(np.abs(wl.beta), np.full(wl.count, np.float32(0.05)))
    assert np.array_equal(np.sign(wl.beta), wl.q)
    assert abs(np.std(np.stack(wl.B)) - 1.0) < 0.05


def test_sweep_statistics_match_page_scale():
    """About 1% of particles in the window per step, a per-step maximum near the
    page's capacity of 30 at N = 2000, and about half ever selected (983/2000)."""
    g = json.load(open(os.path.join(GOLDEN, "pages_structural.json")))["sweep_statistics"]
    wl = synthetic.workload("sweep1d_2000")
    t = np.arange(1, wl.T + 1)[:, None]
    x = np.mod(wl.x0[None] + wl.v[None] * (t * wl.dt), 1.0)
    d = x - t / wl.T
    d = d - np.rint(d)
    sel = np.abs(d) < wl.hw
    per_step = sel.sum(axis=1)
    assert abs(per_step.mean() / g["count"] - g["window_fraction_per_step"]) < 0.003
    assert 0.7 * g["capacity_printed"] <= per_step.max() <= 1.4 * g["capacity_printed"]
    assert 0.8 < sel.any(axis=0).sum() / g["ever_selected_printed"] < 1.2


def test_every_named_workload_builds_small():
    """Each named workload generates (shrunk) with its own seed and recipe."""
    small = {"sweep1d_2000": dict(count=64),
             "sweep1d_grad_1e7": dict(count=64),
             "cic2d_512_ppc16": dict(n=[16, 16], ppc=2),
             "cic3d_128_ppc32": dict(n=[16, 16, 16], ppc=2),
             "tsc3d_128_blob": dict(n=[16, 16, 16], count=4096,
                                    blob=dict(sigma=2.0, overdensity=20.0)),
             "mass_64_ppc64": dict(n=[8, 8, 8], ppc=2)}
    assert set(small) == set(synthetic.WORKLOADS)
    for name, scale in small.items():
        a = synthetic.workload(name, scale)
        b = synthetic.workload(name, scale)
        if name.startswith("sweep1d"):
            assert a.x0.size == 64 and np.array_equal(a.x0, b.x0)
        else:
            assert a.count > 0 and all(np.array_equal(p, r) for p, r in zip(a.x, b.x))
