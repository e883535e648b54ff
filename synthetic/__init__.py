"""Seeded synthetic workloads for particle-to-grid deposition.

This module only draws random inputs: it holds none of the deposit, sort or
mass-matrix arithmetic.  It is the one piece shared by the fp64 oracle (tests)
and the HIP library's callers (tests, bench), so both sides see bit-identical
particle arrays.

Recipe (numpy ``Generator(PCG64(seed))``, draws made in this order):
  1. positions, 2. velocities, 3. charges (deterministic), 4. weights,
  5. magnetic field, 6. the far-displaced subset.
Particles come out in a random order (as a shuffled particle array would be):
uniform loadings deal every cell exactly ppc times in a random order, and every
other per-particle quantity is drawn i.i.d. in that final order, so no array is
ever gathered.  Draws are fp32 except the 1-D workload (fp64); a coordinate that
rounds up to the grid edge n_k is mapped to 0 (positions live in [0, n_k)).

Workloads (see ``workload``):
  sweep1d_2000     1-D windowed sweep: 2000 particles, x0 ~ U[0,1),
                   v ~ N(0, 0.05) (fp64), 1024 bins, 50 steps, dt = 0.02,
                   half-width 0.005.
  cic2d_512_ppc16  2-D 512x512, exactly 16 particles per cell, uniform in-cell;
                   v ~ N(0,0.1)^3 rescaled below |v| = 1; w = 1; q = +1/-1
                   alternating; displaced by v.
  cic3d_128_ppc32  3-D 128^3, exactly 32 per cell; as the 2-D one, plus 2% of
                   the particles displaced by a random direction times U[2,4]
                   cells instead of v.
  tsc3d_128_blob   3-D 128^3, 33,554,432 particles: a Gaussian blob (sigma = 10
                   cells) at the centre with 20x peak overdensity over a uniform
                   background; v ~ N(0,0.1)^3; w ~ U[0.5,1.5].
  mass_64_ppc64    3-D 64^3, exactly 64 per cell; B ~ N(0,1)^3; q/m = +1/-1
                   alternating; beta = (q/m) dt/2 with dt = 0.1; w = 1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

SEED_BASE = 1000
F32 = np.float32


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(int(seed)))


def to_grid_f32(xd: np.ndarray, nk: int) -> np.ndarray:
    """Cast coordinates in [0, nk] to fp32, mapping a round-up to nk onto 0."""
    x = np.asarray(xd, dtype=F32).copy()
    x[(x >= F32(nk)) | (x < 0)] = F32(0.0)
    return x


def periodic_shift(x: np.ndarray, delta: np.ndarray, nk: int) -> np.ndarray:
    """Input preparation (a push, not part of the deposit): x + delta wrapped into
    [0, nk), in fp32."""
    y = np.mod(x.astype(F32) + np.asarray(delta, dtype=F32), F32(nk))
    return to_grid_f32(y, nk)


@dataclass
class Workload:
    """Particle arrays in generation-then-shuffle order (fp32 SoA)."""

    dim: int
    n: List[int]                      # nodes per axis, unused axes 1
    x: List[np.ndarray]               # positions before the push (sorted on these)
    x_next: List[np.ndarray]          # positions after the push (deposited)
    v: List[np.ndarray]               # 3 velocity components
    q: np.ndarray
    w: np.ndarray
    B: Optional[List[np.ndarray]] = None
    beta: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)

    @property
    def count(self) -> int:
        return int(self.q.size)

    def take(self, idx: np.ndarray) -> "Workload":
        """Reorder every per-particle array by idx (used to apply a permutation)."""
        f = lambda a: None if a is None else a[idx]
        return Workload(self.dim, list(self.n), [a[idx] for a in self.x],
                        [a[idx] for a in self.x_next], [a[idx] for a in self.v],
                        self.q[idx], self.w[idx],
                        None if self.B is None else [b[idx] for b in self.B],
                        f(self.beta), dict(self.meta))


def _uniform_per_cell(r, n3, dim, ppc):
    """Exactly ppc particles per cell, uniform inside the cell, in random order."""
    ncell = int(np.prod(n3[:dim]))
    cells = r.permutation(ncell * ppc) // ppc      # every cell dealt ppc times
    offs = r.random((dim, cells.size), dtype=F32)
    xs = []
    rem = cells
    for k in range(dim):
        ck = (rem % n3[k]).astype(F32)
        rem = rem // n3[k]
        x = ck + offs[k]
        # keep the particle inside its cell when fp32 rounds up to the next node
        up = x >= ck + F32(1)
        if up.any():
            x[up] = np.nextafter(ck[up] + F32(1), F32(0.0))
        x[x >= F32(n3[k])] = F32(0.0)
        xs.append(x)
    return xs


def _velocities(r, npart, sigma):
    v = r.standard_normal((3, npart), dtype=F32) * F32(sigma)
    speed = np.sqrt((v * v).sum(axis=0))
    big = speed >= 1.0
    if big.any():
        v[:, big] *= (F32(1.0 - 2.0 ** -20) / speed[big])
    return v


def _charges(npart):
    return np.where(np.arange(npart) % 2 == 0, 1.0, -1.0).astype(F32)


def deposit_workload(dim, n, ppc=None, count=None, sigma_v=0.1, w_uniform=False,
                     far_fraction=0.0, far_range=(2.0, 4.0), blob=None, seed=0):
    """Particles for a 2-D/3-D current deposit.

    Either ``ppc`` (exactly that many per cell, uniform in-cell) or ``blob``
    (dict(sigma, overdensity) with ``count`` particles: each particle belongs to
    a Gaussian blob at the centre with the probability that gives the stated
    peak overdensity over the uniform background, else to the background) sets
    the positions.  The push displaces every particle by its velocity (one cell
    per unit speed), except a ``far_fraction`` subset displaced by a random
    direction times a length drawn from ``far_range`` cells.
    """
    n3 = list(n) + [1] * (3 - len(n))
    r = rng(seed)
    # 1. positions
    if blob is None:
        xs = _uniform_per_cell(r, n3, dim, int(ppc))
    else:
        sig = float(blob["sigma"])
        amp = float(blob["overdensity"])
        vol = float(np.prod(n3[:dim]))
        blob_mass = amp * (2.0 * math.pi * sig * sig) ** (dim / 2.0)
        in_blob = r.random(count, dtype=F32) < F32(blob_mass / (blob_mass + vol))
        xs = []
        for k in range(dim):
            g = r.standard_normal(count, dtype=F32) * F32(sig) + F32(n3[k] / 2.0)
            u = r.random(count, dtype=F32) * F32(n3[k])
            xd = np.where(in_blob, np.mod(g, F32(n3[k])), u)
            xs.append(to_grid_f32(xd, n3[k]))
    npart = xs[0].size
    # 2. velocities, 3. charges, 4. weights
    v = _velocities(r, npart, sigma_v)
    q = _charges(npart)
    w = r.uniform(0.5, 1.5, npart).astype(F32) if w_uniform else np.ones(npart, F32)
    # 6. displacement: v * (1 cell per unit speed); the order is random, so the
    #    first n_far particles are a random subset, displaced far instead
    delta = v[:dim].copy()
    n_far = int(round(far_fraction * npart))
    if n_far:
        d = r.standard_normal((3, n_far), dtype=F32)
        d /= np.sqrt((d * d).sum(axis=0))
        length = r.uniform(far_range[0], far_range[1], n_far).astype(F32)
        delta[:, :n_far] = (d * length)[:dim]
    x_next = [periodic_shift(xs[k], delta[k], n3[k]) for k in range(dim)]
    return Workload(dim, n3, xs, x_next, [v[c] for c in range(3)], q, w,
                    meta=dict(ppc=ppc, count=npart, sigma_v=sigma_v, far_fraction=far_fraction,
                              n_far=n_far, seed=seed))


def previous_positions(x, max_step=0.95, scale_v=None, v=None, seed=0):
    """Unwrapped previous positions for a move deposit (fp32): x_k - d_k with
    d_k ~ U(-max_step, max_step), or, with ``v`` given, d = scale_v * v.  The
    result may lie outside [0, n_k) by less than a cell (the particle crossed
    the periodic boundary)."""
    if v is not None:
        return [(np.asarray(x[k], F32) - F32(scale_v) * np.asarray(v[k], F32)).astype(F32)
                for k in range(len(x))]
    r = rng(seed)
    return [(np.asarray(x[k], F32) - r.uniform(-max_step, max_step, x[k].size).astype(F32))
            .astype(F32) for k in range(len(x))]


def stale_keys(x, n, fraction, span, seed=0):
    """Positions to key a stale tile layout on: x, except a ``fraction`` subset
    shifted by U(-span, span) cells per axis (wrapped into [0, n_k))."""
    r = rng(seed)
    out = []
    for k in range(len(x)):
        d = r.uniform(-span, span, x[k].size).astype(F32)
        d[r.random(x[k].size) >= fraction] = 0
        out.append(periodic_shift(x[k], d, int(n[k])))
    return out


def mass_workload(n, ppc, dt=0.1, w_uniform=False, seed=0):
    """Particles for the ECSIM mass matrix: exactly ppc per cell, B ~ N(0,1)^3,
    q/m = +1/-1 alternating (m = 1), beta = (q/m) dt / 2."""
    n3 = list(n)
    r = rng(seed)
    xs = _uniform_per_cell(r, n3, 3, int(ppc))             # 1. positions
    npart = xs[0].size
    v = _velocities(r, npart, 0.1)                          # 2. velocities
    q = _charges(npart)                                     # 3. charges
    w = (r.uniform(0.5, 1.5, npart).astype(F32) if w_uniform  # 4. weights
         else np.ones(npart, F32))
    B = r.standard_normal((3, npart), dtype=F32)            # 5. magnetic field
    beta = (q.astype(np.float64) * dt / 2.0).astype(F32)
    return Workload(3, n3, xs, xs, [v[c] for c in range(3)], q, w, [B[c] for c in range(3)],
                    beta, meta=dict(ppc=ppc, count=npart, dt=dt, seed=seed))


@dataclass
class SweepWorkload:
    nb: int
    T: int
    dt: float
    hw: float
    x0: np.ndarray   # fp64
    v: np.ndarray    # fp64


def sweep_workload(count=2000, sigma_v=0.05, nb=1024, T=50, dt=0.02, hw=0.005, seed=0):
    r = rng(seed)
    x0 = r.random(count)
    v = r.normal(0.0, sigma_v, count)
    return SweepWorkload(nb, T, dt, hw, x0, v)


# ----------------------------------------------------------------------------
# the five configurations at full size, and scaled variants for tests
# ----------------------------------------------------------------------------

# The named workloads at full size; each draws from its own seed.
WORKLOADS = {
    # 1-D windowed sweep: 2000 particles, 50 steps, 1024 bins
    "sweep1d_2000": dict(kind="sweep1d", count=2000, seed=SEED_BASE + 1),
    # the same sweep at the size of the compaction page's timing table: 10^7
    # particles, 50 steps, 1024 bins (its gradient is timed there)
    "sweep1d_grad_1e7": dict(kind="sweep1d", count=10_000_000, seed=SEED_BASE + 6),
    # 2-D CIC current deposit, 512^2 periodic, 16 particles per cell
    "cic2d_512_ppc16": dict(kind="deposit", dim=2, n=[512, 512], ppc=16, order=1, T=8, D=1,
                            seed=SEED_BASE + 2),
    # 3-D CIC current deposit, 128^3 periodic, 32 per cell, 2% pushed 2-4 cells
    "cic3d_128_ppc32": dict(kind="deposit", dim=3, n=[128, 128, 128], ppc=32, order=1, T=8,
                            D=1, far_fraction=0.02, seed=SEED_BASE + 3),
    # 3-D TSC current deposit, 128^3 periodic, 16 per cell on average, Gaussian blob
    "tsc3d_128_blob": dict(kind="deposit", dim=3, n=[128, 128, 128], count=33554432, order=2,
                           Ts=[4, 8, 16], D=1, blob=dict(sigma=10.0, overdensity=20.0),
                           w_uniform=True, seed=SEED_BASE + 4),
    # ECSIM CIC mass matrix, 64^3 periodic, 64 particles per cell
    "mass_64_ppc64": dict(kind="mass", n=[64, 64, 64], ppc=64, seed=SEED_BASE + 5),
}


def workload(name: str, scale: Optional[dict] = None):
    """The named workload at full size, or with fields of WORKLOADS[name] overridden by scale."""
    info = dict(WORKLOADS[name])
    if scale:
        info.update(scale)
    seed = info["seed"]
    if info["kind"] == "sweep1d":
        return sweep_workload(count=info["count"], seed=seed)
    if info["kind"] == "mass":
        return mass_workload(info["n"], info["ppc"], w_uniform=info.get("w_uniform", False),
                             seed=seed)
    return deposit_workload(info["dim"], info["n"], ppc=info.get("ppc"), count=info.get("count"),
                            w_uniform=info.get("w_uniform", False),
                            far_fraction=info.get("far_fraction", 0.0), blob=info.get("blob"),
                            seed=seed)
