"""The oracle on every host core, for the CPU baseline of the benchmark.

TEST INFRASTRUCTURE ONLY (as the rest of this package).  Nothing here changes
the oracle's arithmetic: the particles are split into contiguous ranges, one
per thread, and each thread calls the single-threaded oracle routines of
``oracle.c`` on its range (ctypes releases the interpreter lock for the call,
so the threads run in parallel).  Sums go to per-thread private fp64 arrays
that are then added in thread order, so the result is deterministic; the
stable sort of the whole input is assembled from the threads' stable sorts of
their ranges (within a tile, range r's particles precede range r+1's, which
is the stable order).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import (deposit, deposit_zigzag, mass_matrix, mass_matrix_scalar, mass_matrix_scalar_tsc,
               mass_matrix_tsc, ntiles, stable_sort, sweep1d, sweep1d_grad, tile_keys)


def host_cores() -> int:
    """Cores this process may run on."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - not Linux
        return os.cpu_count() or 1


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def thread_count(private_bytes: int) -> int:
    """All cores, capped so that the threads' private arrays take at most a
    quarter of the host memory."""
    n = host_cores()
    try:
        mem = os.sysconf("SC_PAGE_SIZE") * os.sysconf("SC_PHYS_PAGES")
        n = min(n, max(1, int(0.25 * mem) // max(1, int(private_bytes))))
    except (ValueError, OSError):
        pass
    return max(1, n)


def _ranges(count, nthreads):
    b = np.linspace(0, count, nthreads + 1).astype(np.int64)
    return [(int(b[i]), int(b[i + 1])) for i in range(nthreads)]


def _reduce(parts):
    """Sum of the per-thread arrays in thread order (in place into the first)."""
    out = parts[0]
    for p in parts[1:]:
        out += p
    return out


def tile_sort(dim, n, order, T, x, nthreads):
    """The same (perm, tile_offsets) as oracle.tile_sort, from per-range
    oracle sorts merged in range order."""
    count = int(np.asarray(x[0]).size)
    nt = ntiles(dim, n, T)
    rngs = _ranges(count, nthreads)

    def local(r):
        lo, hi = r
        keys = tile_keys(dim, n, order, T, [a[lo:hi] for a in x[:dim]])
        perm, off = stable_sort(keys, nt)
        return perm, off

    with ThreadPoolExecutor(nthreads) as ex:
        res = list(ex.map(local, rngs))
    counts = np.stack([np.diff(off.astype(np.int64)) for _, off in res])  # [ranges, tiles]
    before = np.cumsum(counts, axis=0) - counts  # earlier ranges' share of each tile
    goff = np.zeros(nt + 1, np.int64)
    np.cumsum(counts.sum(axis=0), out=goff[1:])
    perm = np.empty(count, np.uint32)

    def place(i):
        (lo, _), (lp, loff) = rngs[i], res[i]
        tiles = np.repeat(np.arange(nt), counts[i])
        slot = goff[tiles] + before[i][tiles] + (np.arange(lp.size) - loff[tiles].astype(np.int64))
        perm[slot] = lp.astype(np.int64) + lo

    with ThreadPoolExecutor(nthreads) as ex:
        list(ex.map(place, range(nthreads)))
    return perm, goff.astype(np.uint32)


def deposit_step(dim, n, order, T, x, v, q, w, nthreads):
    """Tile sort and fp64 deposit of one step's particles (the work the
    single-threaded baseline times), on nthreads threads.  Returns J."""
    tile_sort(dim, n, order, T, x, nthreads)
    rngs = _ranges(int(q.size), nthreads)

    def part(r):
        lo, hi = r
        return deposit(dim, n, order, [a[lo:hi] for a in x[:dim]], [a[lo:hi] for a in v],
                       q[lo:hi], w[lo:hi])

    with ThreadPoolExecutor(nthreads) as ex:
        return _reduce(list(ex.map(part, rngs)))


def zigzag_step(n, T, x, xp, q, w, nthreads):
    """Tile sort on x and the fp64 zigzag deposit, on nthreads threads."""
    tile_sort(3, n, 1, T, x, nthreads)
    rngs = _ranges(int(q.size), nthreads)

    def part(r):
        lo, hi = r
        return deposit_zigzag(n, [a[lo:hi] for a in x], [a[lo:hi] for a in xp], q[lo:hi],
                              w[lo:hi])

    with ThreadPoolExecutor(nthreads) as ex:
        return _reduce(list(ex.map(part, rngs)))


def mass(n, x, q, w, nthreads, B=None, beta=None, order=1):
    """A mass matrix (tensor with B and beta, else scalar; CIC or, order 2,
    TSC) on nthreads threads, per-thread private fp64 matrices added in thread
    order."""
    rngs = _ranges(int(q.size), nthreads)

    def part(r):
        lo, hi = r
        xs = [a[lo:hi] for a in x]
        if B is None:
            f = mass_matrix_scalar if order == 1 else mass_matrix_scalar_tsc
            return f(n, xs, q[lo:hi], w[lo:hi])
        f = mass_matrix if order == 1 else mass_matrix_tsc
        return f(n, xs, [b[lo:hi] for b in B], q[lo:hi], w[lo:hi], beta[lo:hi])

    with ThreadPoolExecutor(nthreads) as ex:
        return _reduce(list(ex.map(part, rngs)))


def sweep_loss_grad(nb, x0, v, T, dt, hw, target, nthreads):
    """The 1-D sweep's forward histogram (per-thread ranges, added in thread
    order), the seed 2 (H - target), and the reverse per range: (H, dx0)."""
    rngs = _ranges(int(x0.size), nthreads)
    with ThreadPoolExecutor(nthreads) as ex:
        H = _reduce(list(ex.map(lambda r: sweep1d(nb, x0[r[0]:r[1]], v[r[0]:r[1]], T, dt, hw),
                                rngs)))
    dH = 2.0 * (H.astype(np.float64) - target)
    with ThreadPoolExecutor(nthreads) as ex:
        parts = list(ex.map(lambda r: sweep1d_grad(nb, x0[r[0]:r[1]], v[r[0]:r[1]], T, dt, hw,
                                                   dH), rngs))
    return H, np.concatenate(parts)
