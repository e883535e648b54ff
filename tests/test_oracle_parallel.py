"""The all-cores runner of the oracle (the benchmark's CPU baseline) gives the
single-threaded oracle's results: the same stable sort bit for bit, and the
same sums up to fp64 rounding order."""
import numpy as np

import synthetic
from oracle import parallel


def test_parallel_tile_sort_is_the_oracle_sort(orc):
    wl = synthetic.deposit_workload(3, [16, 16, 16], ppc=5, seed=3)
    _, perm, off = orc.tile_sort(3, wl.n, 1, 4, wl.x)
    for nth in (1, 3, 8):
        p2, off2 = parallel.tile_sort(3, wl.n, 1, 4, wl.x, nth)
        assert np.array_equal(p2, perm) and np.array_equal(off2, off)


def test_parallel_deposit_and_mass_match(orc):
    wl = synthetic.deposit_workload(3, [16, 16, 16], ppc=5, seed=4)
    J = orc.deposit(3, wl.n, 2, wl.x, wl.v, wl.q, wl.w)
    J2 = parallel.deposit_step(3, wl.n, 2, 4, wl.x, wl.v, wl.q, wl.w, 5)
    assert np.abs(J2 - J).max() <= 1e-12 * np.abs(J).max()
    m = synthetic.mass_workload([6, 5, 7], 9, w_uniform=True, seed=5)
    M = orc.mass_matrix(m.n, m.x, m.B, m.q, m.w, m.beta)
    M2 = parallel.mass(m.n, m.x, m.q, m.w, 4, B=m.B, beta=m.beta)
    assert np.abs(M2 - M).max() <= 1e-12 * np.abs(M).max()
    S = parallel.mass(m.n, m.x, m.q, m.w, 3)
    assert np.abs(S - orc.mass_matrix_scalar(m.n, m.x, m.q, m.w)).max() <= 1e-12 * np.abs(S).max()


def test_thread_count_is_bounded():
    assert 1 <= parallel.thread_count(1) <= parallel.host_cores()
    assert parallel.thread_count(1 << 62) == 1
    assert parallel.cpu_model()
