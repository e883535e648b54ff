"""The numpy row-sum helpers the full-size mass-matrix tests use, checked on the
CPU against the oracle's matrices on small grids (the mass-matrix paper,
Eq.(11): M = W diag(c) W^T, so each block row sums to sum_p c_p W_pg)."""
import numpy as np

import synthetic
from gpu_util import alpha_coefs, block_row_sums, check_row_sums, node_row_sums, seam_cells


def test_cic_tensor_row_sums_match_oracle(orc):
    wl = synthetic.mass_workload([5, 4, 6], 7, w_uniform=True, seed=31)
    M = orc.mass_matrix(wl.n, wl.x, wl.B, wl.q, wl.w, wl.beta)
    c = alpha_coefs(wl)
    want = node_row_sums(wl.n, wl.x, 1, c)
    scale = node_row_sums(wl.n, wl.x, 1, [np.abs(a) for a in c])
    assert check_row_sums(block_row_sums(M), want, scale, 1e-13) <= 1.0
    # a dropped particle is seen
    M2 = orc.mass_matrix(wl.n, [a[1:] for a in wl.x], [b[1:] for b in wl.B], wl.q[1:],
                         wl.w[1:], wl.beta[1:])
    assert np.abs(block_row_sums(M2) - want).max() > 1e-3


def test_tsc_row_sums_match_oracle(orc):
    wl = synthetic.mass_workload([5, 6, 5], 5, w_uniform=True, seed=32)
    Ms = orc.mass_matrix_scalar_tsc(wl.n, wl.x, wl.q, wl.w)
    qw = wl.q.astype(np.float64) * wl.w
    want = node_row_sums(wl.n, wl.x, 2, [qw])
    assert np.abs(block_row_sums(Ms) - want).max() <= 1e-12 * np.abs(qw).sum()
    Mt = orc.mass_matrix_tsc(wl.n, wl.x, wl.B, wl.q, wl.w, wl.beta)
    want = node_row_sums(wl.n, wl.x, 2, alpha_coefs(wl))
    assert np.abs(block_row_sums(Mt) - want).max() <= 1e-12 * np.abs(qw).sum()


def test_seam_cells_reach():
    """The node rows seam_cells names receive only from the cells it names."""
    for n, step in [(64, 8), (64, 4), (40, 8)]:
        cells, rows = seam_cells(n, step)
        for g in np.nonzero(rows)[0]:
            assert cells[(g - 1) % n] and cells[g]
        assert rows[0] and rows[n - 1] and rows[step] and rows[step - 1]
