"""Pins for the fp64 oracle: closed forms, hand-computed stencils, invariants and
library routines -- never the oracle's own formulas retyped.

Each group names the passage it pins:
  [MM] Pennati & Markidis, "Mass Matrix Assembly on Tensor Cores for Implicit PIC"
  [TD] Entity wiki, "Tiled current deposit"
  [CS] WEANJ, "03. Compaction and scatter-add"
"""
import json
import os

import numpy as np
import pytest
from scipy import integrate

import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# shape functions  ([MM] §2.3 Eq.(12))
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("x,base,w", [
    (3.25, 3, [0.75, 0.25]),
    (0.0, 0, [1.0, 0.0]),
    (7.5, 7, [0.5, 0.5]),
])
def test_cic_dyadic_values(orc, x, base, w):
    b, got = orc.shape_1d(1, x)
    assert b == base
    assert np.array_equal(got, np.array(w))


@pytest.mark.parametrize("x,base,w", [
    (5.0, 4, [1 / 8, 3 / 4, 1 / 8]),          # xi = 0: centred on node 5
    (5.25, 4, [1 / 32, 11 / 16, 9 / 32]),     # xi = 1/4 -> nodes 4,5,6
    (5.5, 5, [1 / 2, 1 / 2, 0.0]),            # xi = 1/2 -> nodes 5,6,7 (page's tie rule)
    (5.75, 5, [9 / 32, 11 / 16, 1 / 32]),     # xi = 3/4 mirrors 1/4
    (0.25, -1, [1 / 32, 11 / 16, 9 / 32]),    # base below the grid, wraps later
])
def test_tsc_dyadic_values(orc, x, base, w):
    b, got = orc.shape_1d(2, x)
    assert b == base
    assert np.array_equal(got, np.array(w))


def test_tsc_continuous_across_half(orc):
    # just below xi = 1/2 the stencil is {4,5,6}; at 1/2 it is {5,6,7}; the node
    # weights must agree (node 4 and node 7 carry ~0)
    b0, w0 = orc.shape_1d(2, np.nextafter(5.5, 0.0))
    b1, w1 = orc.shape_1d(2, 5.5)
    lo = {b0 + a: w0[a] for a in range(3)}
    hi = {b1 + a: w1[a] for a in range(3)}
    for node in range(4, 8):
        assert abs(lo.get(node, 0.0) - hi.get(node, 0.0)) < 1e-12


@pytest.mark.parametrize("order", [1, 2])
def test_partition_of_unity_and_moments(orc, order):
    """Sum W = 1, W >= 0, and B-splines reproduce linear functions:
    sum_g g W_g(x) = x; for the quadratic spline sum_g (g-x)^2 W_g = 1/4."""
    r = np.random.default_rng(7)
    for x in r.uniform(0.0, 50.0, 200):
        b, w = orc.shape_1d(order, x)
        nodes = b + np.arange(order + 1)
        assert abs(w.sum() - 1.0) < 1e-14
        assert (w >= 0).all()
        assert abs((nodes * w).sum() - x) < 1e-12
        if order == 2:
            assert abs((((nodes - x) ** 2) * w).sum() - 0.25) < 1e-12


def test_tsc_is_box_convolved_with_cic(orc):
    """Independent route: the quadratic B-spline is the unit box convolved with the
    hat, W2_g(x) = int_{-1/2}^{1/2} hat(x - g - s) ds, evaluated by quadrature."""
    r = np.random.default_rng(11)
    hat = lambda s: max(0.0, 1.0 - abs(s))
    for x in r.uniform(0.0, 20.0, 60):
        b, w = orc.shape_1d(2, x)
        for a in range(3):
            g = b + a
            val, _ = integrate.quad(lambda s: hat(x - g - s), -0.5, 0.5,
                                    points=[x - g - 1, x - g, x - g + 1], epsabs=1e-14)
            assert abs(val - w[a]) < 1e-10
        # nodes outside the support carry no weight
        for g in (b - 1, b + 3):
            val, _ = integrate.quad(lambda s: hat(x - g - s), -0.5, 0.5,
                                    points=[x - g - 1, x - g, x - g + 1], epsabs=1e-14)
            assert val < 1e-12


def test_support_sizes_match_pages(orc):
    g = json.load(open(os.path.join(GOLDEN, "pages_structural.json")))
    for order, key in ((1, "cic_3d"), (2, "tsc_3d")):
        J = orc.deposit(3, [8, 8, 8], order, [np.float32([3.3]), np.float32([4.6]),
                                               np.float32([5.2])],
                        [np.float32([1.0]), np.float32([0.0]), np.float32([0.0])],
                        np.float32([1.0]), np.float32([1.0]))
        assert np.count_nonzero(J[0]) == g["support_nodes"][key]


# ---------------------------------------------------------------------------
# current deposit  (J += q w v W; [TD] "One deposit body", [MM] Eq.(12))
# ---------------------------------------------------------------------------

def _one(vals):
    return [np.float32([v]) for v in vals]


def _expected_from_axes(n, axes, amp):
    """Outer product of hand-written per-axis (node, weight) lists, times amp[c]."""
    J = np.zeros((3, n[2], n[1], n[0]))
    for zn, zw in axes[2]:
        for yn, yw in axes[1]:
            for xn, xw in axes[0]:
                for c in range(3):
                    J[c, zn, yn, xn] += amp[c] * xw * yw * zw
    return J


def test_single_particle_cic_3d(orc):
    # x = (1.25, 2.5, 3.75): x-nodes 1,2 (3/4,1/4); y-nodes 2,3 (1/2,1/2);
    # z-nodes 3,4 (1/4,3/4).  q = -1, w = 2, v = (1, -2, 0.5)
    J = orc.deposit(3, [8, 8, 8], 1, _one([1.25, 2.5, 3.75]), _one([1.0, -2.0, 0.5]),
                    np.float32([-1.0]), np.float32([2.0]))
    exp = _expected_from_axes([8, 8, 8], [[(1, .75), (2, .25)], [(2, .5), (3, .5)],
                                          [(3, .25), (4, .75)]], [-2.0, 4.0, -1.0])
    assert np.array_equal(J, exp)
    assert J[0, 3, 2, 1] == -2.0 * 0.75 * 0.5 * 0.25


def test_single_particle_cic_periodic_wrap(orc):
    # x = 7.75 on an 8-node axis touches nodes 7 and 0
    J = orc.deposit(3, [8, 4, 4], 1, _one([7.75, 0.0, 3.5]), _one([1.0, 0.0, 0.0]),
                    np.float32([1.0]), np.float32([1.0]))
    exp = _expected_from_axes([8, 4, 4], [[(7, .25), (0, .75)], [(0, 1.0), (1, 0.0)],
                                          [(3, .5), (0, .5)]], [1.0, 0.0, 0.0])
    assert np.array_equal(J, exp)


def test_single_particle_tsc_3d_with_wrap(orc):
    # x = 0.25 -> nodes -1,0,1 = 7,0,1 (1/32, 11/16, 9/32)
    # y = 5.75 -> nodes 5,6,7 (9/32, 11/16, 1/32)
    # z = 2.0  -> nodes 1,2,3 (1/8, 3/4, 1/8)
    J = orc.deposit(3, [8, 8, 8], 2, _one([0.25, 5.75, 2.0]), _one([0.5, 1.0, -1.0]),
                    np.float32([1.0]), np.float32([4.0]))
    exp = _expected_from_axes([8, 8, 8], [[(7, 1 / 32), (0, 11 / 16), (1, 9 / 32)],
                                          [(5, 9 / 32), (6, 11 / 16), (7, 1 / 32)],
                                          [(1, 1 / 8), (2, 3 / 4), (3, 1 / 8)]], [2.0, 4.0, -4.0])
    assert np.allclose(J, exp, rtol=0, atol=1e-15)


def test_single_particle_2d(orc):
    # 2-D: (x, y) = (3.5, 0.25), CIC -> x-nodes 3,4 (1/2,1/2), y-nodes 0,1 (3/4,1/4)
    J = orc.deposit(2, [8, 8], 1, _one([3.5, 0.25]), _one([1.0, 2.0, 3.0]),
                    np.float32([1.0]), np.float32([1.0]))
    assert J.shape == (3, 1, 8, 8)
    exp = _expected_from_axes([8, 8, 1], [[(3, .5), (4, .5)], [(0, .75), (1, .25)], [(0, 1.0)]],
                              [1.0, 2.0, 3.0])
    assert np.array_equal(J, exp)


def _random_particles(r, dim, n, npart, dyadic=False):
    n3 = list(n) + [1] * (3 - len(n))
    if dyadic:
        x = [(r.integers(0, n3[k] * 64, npart) / 64.0).astype(np.float32) for k in range(dim)]
    else:
        x = [r.uniform(0, n3[k], npart).astype(np.float32) for k in range(dim)]
        for k in range(dim):
            x[k][x[k] >= n3[k]] = 0
    v = [r.normal(0, 0.3, npart).astype(np.float32) for _ in range(3)]
    q = np.where(r.random(npart) < 0.5, 1.0, -1.0).astype(np.float32)
    w = r.uniform(0.5, 1.5, npart).astype(np.float32)
    return x, v, q, w


@pytest.mark.parametrize("dim,order", [(1, 1), (2, 1), (3, 1), (1, 2), (2, 2), (3, 2)])
def test_deposit_conserves_current(orc, dim, order):
    """sum_g J_c = sum_p q w v_c (partition of unity)."""
    r = np.random.default_rng(100 + 10 * dim + order)
    n = [12, 10, 8][:dim]
    x, v, q, w = _random_particles(r, dim, n, 3000)
    J = orc.deposit(dim, n, order, x, v, q, w)
    for c in range(3):
        tot = (q.astype(np.float64) * w * v[c]).sum()
        assert abs(J[c].sum() - tot) <= 1e-12 * np.abs(q * w * v[c]).sum()


@pytest.mark.parametrize("order", [1, 2])
def test_deposit_roll_covariance(orc, order):
    """Shifting every particle by whole cells rolls J by the same amount, exactly
    (dyadic positions keep the fractional parts identical)."""
    r = np.random.default_rng(5 + order)
    n = [16, 12, 8]
    x, v, q, w = _random_particles(r, 3, n, 500, dyadic=True)
    J0 = orc.deposit(3, n, order, x, v, q, w)
    shift = (5, -3, 2)
    xs = [np.mod(x[k].astype(np.float64) + shift[k], n[k]).astype(np.float32) for k in range(3)]
    J1 = orc.deposit(3, n, order, xs, v, q, w)
    assert np.array_equal(J1, np.roll(J0, shift=(shift[2], shift[1], shift[0]), axis=(1, 2, 3)))


def test_deposit_at_nodes_is_histogram(orc):
    """CIC particles sitting exactly on nodes reduce to a nearest-node histogram."""
    r = np.random.default_rng(3)
    n = [9, 7, 5]
    idx = [r.integers(0, n[k], 400) for k in range(3)]
    x = [i.astype(np.float32) for i in idx]
    v = [r.normal(0, 1, 400).astype(np.float32) for _ in range(3)]
    q = np.ones(400, np.float32)
    w = r.uniform(0.5, 1.5, 400).astype(np.float32)
    J = orc.deposit(3, n, 1, x, v, q, w)
    lin = idx[0] + n[0] * (idx[1] + n[1] * idx[2])
    for c in range(3):
        h = np.bincount(lin, weights=(w.astype(np.float64) * v[c]), minlength=np.prod(n))
        assert np.allclose(J[c].ravel(), h, rtol=0, atol=1e-12)


def test_deposit_tsc_at_nodes_is_fixed_stencil(orc):
    """TSC particles on nodes spread (1/8, 3/4, 1/8) per axis: a convolution of the
    node histogram, computed here with np.roll."""
    r = np.random.default_rng(4)
    n = [8, 8, 8]
    idx = [r.integers(0, 8, 300) for _ in range(3)]
    x = [i.astype(np.float32) for i in idx]
    v = [np.ones(300, np.float32), np.zeros(300, np.float32), np.zeros(300, np.float32)]
    J = orc.deposit(3, n, 2, x, v, np.ones(300, np.float32), np.ones(300, np.float32))
    H = np.zeros((8, 8, 8))
    np.add.at(H, (idx[2], idx[1], idx[0]), 1.0)
    for ax in (0, 1, 2):
        H = 0.75 * H + 0.125 * (np.roll(H, 1, axis=ax) + np.roll(H, -1, axis=ax))
    assert np.allclose(J[0], H, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# tile keys, stable sort, offsets  ([TD] "The tile-based spatial sort")
# ---------------------------------------------------------------------------

def test_tile_keys_hand_values(orc):
    n = [16, 16, 16]
    x = [np.float32([5.5, 0.3, 15.9]), np.float32([0.2, 7.9, 8.0]), np.float32([13.9, 4.0, 0.1])]
    # CIC base nodes: (5,0,13) -> tiles (1,0,3) -> 1 + 4*(0 + 4*3) = 49
    #                 (0,7,4)  -> (0,1,1) -> 0 + 4*(1 + 4*1) = 20
    #                 (15,8,0) -> (3,2,0) -> 3 + 4*2 = 11
    assert list(orc.tile_keys(3, n, 1, 4, x)) == [49, 20, 11]
    # TSC bases: x=5.5 -> 5, 0.3 -> -1 = 15, 15.9 -> 15; y=0.2 -> 15, 7.9 -> 7, 8.0 -> 7;
    # z=13.9 -> 13, 4.0 -> 3, 0.1 -> 15
    # tiles: (1,3,3)=1+4*(3+12)=61; (3,1,0)=3+4*1=7; (3,1,3)=3+4*(1+12)=55
    assert list(orc.tile_keys(3, n, 2, 4, x)) == [61, 7, 55]
    # T = 1 gives the cell (base node) index
    assert list(orc.tile_keys(3, n, 1, 1, x)) == [5 + 16 * (0 + 16 * 13), 0 + 16 * (7 + 16 * 4),
                                                 15 + 16 * 8]


@pytest.mark.parametrize("dim,order,T", [(2, 1, 8), (3, 1, 4), (3, 2, 4), (3, 1, 1)])
def test_stable_sort_matches_numpy(orc, dim, order, T):
    r = np.random.default_rng(dim * 100 + order * 10 + T)
    n = [16, 16, 8][:dim]
    x, _, _, _ = _random_particles(r, dim, n, 5000)
    keys, perm, off = orc.tile_sort(dim, n, order, T, x)
    nt = orc.ntiles(dim, n, T)
    assert np.array_equal(perm, np.argsort(keys, kind="stable").astype(np.uint32))
    cnt = np.bincount(keys, minlength=nt)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]).astype(np.uint32))
    # every slot of tile t holds a particle keyed t, i.e. whose base node is in tile t
    sk = keys[perm]
    for t in range(nt):
        assert (sk[off[t]:off[t + 1]] == t).all()


def test_stable_sort_ties_keep_index_order(orc):
    key = np.array([3, 1, 3, 0, 1, 3], np.uint32)
    perm, off = orc.stable_sort(key, 4)
    assert list(perm) == [3, 1, 4, 0, 2, 5]
    assert list(off) == [0, 1, 3, 3, 6]


# ---------------------------------------------------------------------------
# escape valve  ([TD] "Halo sizing", "Correctness is independent of the halo")
# ---------------------------------------------------------------------------

def _escape_by_sets(n, order, T, D, x, off):
    """Brute force: a particle escapes iff some stencil node lies outside its
    tile's scratch window, the TE = T + order + 2D nodes starting D below the
    tile origin (sets of wrapped node indices; valid for n >= 2 TE)."""
    dim = len(x)
    TE = T + order + 2 * D
    nt = [n[k] // T for k in range(dim)] + [1] * (3 - dim)
    out = np.zeros(x[0].size, bool)
    for t in range(len(off) - 1):
        tc = [t % nt[0], (t // nt[0]) % nt[1], t // (nt[0] * nt[1])]
        for j in range(off[t], off[t + 1]):
            for k in range(dim):
                window = {(tc[k] * T - D + s) % n[k] for s in range(TE)}
                xf = float(x[k][j])
                i = int(np.floor(xf))
                if order == 2 and xf - i < 0.5:
                    i -= 1
                nodes = {(i + a) % n[k] for a in range(order + 1)}
                if not nodes <= window:
                    out[j] = True
    return out


def _sorted_then_pushed(orc, wl, order, T):
    keys, perm, off = orc.tile_sort(wl.dim, wl.n, order, T, wl.x)
    return wl.take(perm.astype(np.int64)), off


@pytest.mark.parametrize("order", [1, 2])
def test_no_escape_when_push_below_one_cell(orc, order):
    """With |displacement| < 1 cell per axis and D = 1 nothing escapes."""
    wl = synthetic.deposit_workload(3, [32, 32, 32], ppc=2, seed=21)
    s, off = _sorted_then_pushed(orc, wl, order, 8)
    cnt, esc = orc.escape(3, wl.n, order, 8, 1, s.x_next, off)
    assert cnt == 0 and not esc.any()


@pytest.mark.parametrize("order,D", [(1, 0), (1, 1), (2, 0), (2, 1)])
def test_escape_matches_set_brute_force(orc, order, D):
    wl = synthetic.deposit_workload(3, [24, 24, 24], ppc=1, far_fraction=0.05, seed=22)
    s, off = _sorted_then_pushed(orc, wl, order, 4)
    cnt, esc = orc.escape(3, wl.n, order, 4, D, s.x_next, off)
    ref = _escape_by_sets(wl.n, order, 4, D, s.x_next, off)
    assert np.array_equal(esc, ref)
    assert cnt == ref.sum() and cnt > 0


def test_escape_stale_layout_and_tail(orc):
    """A layout that puts every particle in tile 0 escapes all but those near tile 0;
    slots past n_part are the flat tail and never counted."""
    r = np.random.default_rng(9)
    n = [32, 32]
    x, _, _, _ = _random_particles(r, 2, n, 2000)
    nt = orc.ntiles(2, n, 8)
    off = np.zeros(nt + 1, np.uint32)
    off[1:] = 2000
    cnt, esc = orc.escape(2, n, 1, 8, 1, x, off)
    ref = _escape_by_sets(n, 1, 8, 1, x, off)
    assert np.array_equal(esc, ref) and cnt == ref.sum()
    cnt2, esc2 = orc.escape(2, n, 1, 8, 1, x, off, n_part=1000)
    assert not esc2[1000:].any() and cnt2 == ref[:1000].sum()


# ---------------------------------------------------------------------------
# rotation-response tensor  ([MM] §2.1 Eq.(5))
# ---------------------------------------------------------------------------

def _cross_matrix(om):
    """C with C u = om x u, built with numpy's cross product."""
    return np.stack([np.cross(om, e) for e in np.eye(3)], axis=1)


def test_alpha_hand_value(orc):
    # omega = z: I + C = [[1,-1,0],[1,1,0],[0,0,1]] -> alpha = [[.5,.5,0],[-.5,.5,0],[0,0,1]]
    a = orc.alpha([0.0, 0.0, 1.0])
    assert np.array_equal(a, np.array([[0.5, 0.5, 0.0], [-0.5, 0.5, 0.0], [0.0, 0.0, 1.0]]))
    assert np.array_equal(orc.alpha([0.0, 0.0, 0.0]), np.eye(3))


def test_alpha_inverts_implicit_rotation(orc):
    """alpha is the inverse of (I + C(omega)) -- checked against numpy's inverse."""
    r = np.random.default_rng(12)
    for om in r.normal(0, 1.5, (50, 3)):
        a = orc.alpha(om)
        Cm = _cross_matrix(om)
        assert np.abs(a @ (np.eye(3) + Cm) - np.eye(3)).max() < 1e-13
        assert np.abs(a - np.linalg.inv(np.eye(3) + Cm)).max() < 1e-13
        assert np.abs(a.T - orc.alpha(-om)).max() < 1e-15


# ---------------------------------------------------------------------------
# mass matrix  ([MM] §2.1 Eq.(4)/(6), §2.2 Eq.(9)-(11), §3.4)
# ---------------------------------------------------------------------------

OFFS = [(dx, dy, dz) for dz in (-1, 0, 1) for dy in (-1, 0, 1) for dx in (-1, 0, 1)]


def _weights_matrix(orc, n, x):
    """Dense W (Ng x Np): column p is the deposit of particle p alone with unit
    charge, weight and v = (1,0,0)."""
    npart = x[0].size
    ng = int(np.prod(n))
    W = np.zeros((ng, npart))
    for p in range(npart):
        J = orc.deposit(3, n, 1, [a[p:p + 1] for a in x],
                        [np.float32([1]), np.float32([0]), np.float32([0])],
                        np.float32([1]), np.float32([1]))
        W[:, p] = J[0].ravel()
    return W


def _mm_inputs(r, n, npart, zero_B=False):
    x = [r.uniform(0, n[k], npart).astype(np.float32) for k in range(3)]
    B = [np.zeros(npart, np.float32) if zero_B else r.normal(0, 1, npart).astype(np.float32)
         for _ in range(3)]
    q = np.where(r.random(npart) < 0.5, 1.0, -1.0).astype(np.float32)
    w = r.uniform(0.5, 1.5, npart).astype(np.float32)
    beta = (q * 0.05 * r.uniform(0.5, 4, npart)).astype(np.float32)
    return x, B, q, w, beta


def _coeffs(orc, B, q, w, beta):
    """Per-particle s^ij = q w alpha^ij ([MM] Eq.(6)), alpha from the (pinned) oracle."""
    out = []
    for p in range(q.size):
        om = float(beta[p]) * np.array([B[0][p], B[1][p], B[2][p]], np.float64)
        out.append(float(q[p]) * float(w[p]) * orc.alpha(om).ravel())
    return np.stack(out)


def test_mass_matrix_equals_dense_contraction(orc):
    """[MM] Eq.(10): M^ij = W diag(s^ij) W^T with s = q w alpha, on a 4^3 grid,
    against the 27-offset store."""
    r = np.random.default_rng(31)
    n = [4, 4, 4]
    x, B, q, w, beta = _mm_inputs(r, n, 120)
    M = orc.mass_matrix(n, x, B, q, w, beta)
    W = _weights_matrix(orc, n, x)
    s = _coeffs(orc, B, q, w, beta)  # [Np, 9]
    ng = 64
    for ij in range(9):
        dense = W @ np.diag(s[:, ij]) @ W.T
        store = np.zeros((ng, ng))
        for gz in range(4):
            for gy in range(4):
                for gx in range(4):
                    g = gx + 4 * (gy + 4 * gz)
                    for o, (dx, dy, dz) in enumerate(OFFS):
                        g2 = (gx + dx) % 4 + 4 * (((gy + dy) % 4) + 4 * ((gz + dz) % 4))
                        store[g, g2] += M[gz, gy, gx, o].ravel()[ij]
        assert np.abs(store - dense).max() < 1e-12 * max(1.0, np.abs(dense).max())


def test_mass_matrix_symmetry_and_row_sums(orc):
    r = np.random.default_rng(32)
    n = [6, 5, 4]
    x, B, q, w, beta = _mm_inputs(r, n, 400)
    M = orc.mass_matrix(n, x, B, q, w, beta)
    # [MM] Eq.(11): for each component, M_{g,g+o} = M_{g+o,g}  (no transpose of ij)
    for o, (dx, dy, dz) in enumerate(OFFS):
        mo = OFFS.index((-dx, -dy, -dz))
        rolled = np.roll(M[:, :, :, mo], shift=(-dz, -dy, -dx), axis=(0, 1, 2))
        assert np.abs(M[:, :, :, o] - rolled).max() < 1e-13
    # block row sums: sum_o M[g][o] = sum_p s_p W_pg ; grand total = sum_p s_p
    s = _coeffs(orc, B, q, w, beta)
    rows = M.sum(axis=3).reshape(-1, 9)
    W = _weights_matrix(orc, n, x)
    for ij in range(9):
        assert np.abs(rows[:, ij] - W @ s[:, ij]).max() < 1e-12
        assert abs(M[..., ij // 3, ij % 3].sum() - s[:, ij].sum()) < 1e-10


def test_mass_matrix_zero_field_is_scalar(orc):
    """B = 0: alpha = I, so M^ij = delta_ij times the scalar (MPM-type) mass matrix
    ([MM] Eq.(6) with s = q delta_ij)."""
    r = np.random.default_rng(33)
    n = [5, 5, 5]
    x, B, q, w, beta = _mm_inputs(r, n, 300, zero_B=True)
    M = orc.mass_matrix(n, x, B, q, w, beta)
    assert np.abs(M[..., 0, 1]).max() == 0 and np.abs(M[..., 2, 0]).max() == 0
    assert np.array_equal(M[..., 0, 0], M[..., 1, 1]) and np.array_equal(M[..., 0, 0], M[..., 2, 2])


def test_mass_matrix_single_particle_rank_one(orc):
    # x = (1.25, 2.5, 3.75) on 8^3, B = (0,0,1), beta = 1 -> alpha from the hand value
    x = _one([1.25, 2.5, 3.75])
    M = orc.mass_matrix([8, 8, 8], x, _one([0.0, 0.0, 1.0]), np.float32([1.0]),
                        np.float32([2.0]), np.float32([1.0]))
    alpha = np.array([[0.5, 0.5, 0.0], [-0.5, 0.5, 0.0], [0.0, 0.0, 1.0]])
    wx = {1: .75, 2: .25}
    wy = {2: .5, 3: .5}
    wz = {3: .25, 4: .75}
    nz = 0
    for gz in wz:
        for gy in wy:
            for gx in wx:
                for o, (dx, dy, dz) in enumerate(OFFS):
                    hx, hy, hz = gx + dx, gy + dy, gz + dz
                    if hx in wx and hy in wy and hz in wz:
                        val = 2.0 * alpha * (wx[gx] * wy[gy] * wz[gz]) * (wx[hx] * wy[hy] * wz[hz])
                        assert np.array_equal(M[gz, gy, gx, o], val)
                        nz += 1
    assert nz == 64
    assert np.count_nonzero(np.abs(M).sum(axis=(4, 5))) == 64


def test_mass_matrix_row_nonzeros_bounded(orc):
    g = json.load(open(os.path.join(GOLDEN, "pages_structural.json")))
    r = np.random.default_rng(34)
    n = [6, 6, 6]
    x, B, q, w, beta = _mm_inputs(r, n, 2000)
    M = orc.mass_matrix(n, x, B, q, w, beta)
    per_row = np.count_nonzero(np.abs(M).sum(axis=(4, 5)), axis=3)
    assert per_row.max() == g["row_nonzeros_max"]["cic_3d"] == 27


def test_scalar_mass_matrix_equals_dense_contraction(orc):
    """[MM] Eq.(10) in the scalar case of Eq.(6): M = W diag(q w) W^T on a 4^3
    grid, against the 27-offset store."""
    r = np.random.default_rng(41)
    n = [4, 4, 4]
    x, _, q, w, _ = _mm_inputs(r, n, 150)
    M = orc.mass_matrix_scalar(n, x, q, w)
    W = _weights_matrix(orc, n, x)
    dense = W @ np.diag(q.astype(np.float64) * w.astype(np.float64)) @ W.T
    store = np.zeros((64, 64))
    for gz in range(4):
        for gy in range(4):
            for gx in range(4):
                g = gx + 4 * (gy + 4 * gz)
                for o, (dx, dy, dz) in enumerate(OFFS):
                    g2 = (gx + dx) % 4 + 4 * (((gy + dy) % 4) + 4 * ((gz + dz) % 4))
                    store[g, g2] += M[gz, gy, gx, o]
    assert np.abs(store - dense).max() < 1e-12 * max(1.0, np.abs(dense).max())


def test_scalar_mass_matrix_symmetry_row_sums_and_charge(orc):
    """[MM] Eq.(11) symmetry; row sums equal the CIC deposit of q w (partition of
    unity of the second factor), and the grand total is sum q w."""
    r = np.random.default_rng(42)
    n = [6, 5, 4]
    x, _, q, w, _ = _mm_inputs(r, n, 500)
    M = orc.mass_matrix_scalar(n, x, q, w)
    for o, (dx, dy, dz) in enumerate(OFFS):
        mo = OFFS.index((-dx, -dy, -dz))
        rolled = np.roll(M[:, :, :, mo], shift=(-dz, -dy, -dx), axis=(0, 1, 2))
        assert np.abs(M[:, :, :, o] - rolled).max() < 1e-13
    ones = np.ones_like(q)
    zeros = np.zeros_like(q)
    J = orc.deposit(3, n, 1, x, [ones, zeros, zeros], q, w)  # J_x = sum_p q w W_pg
    assert np.abs(M.sum(axis=3) - J[0]).max() < 1e-12
    assert abs(M.sum() - float(np.sum(q.astype(np.float64) * w.astype(np.float64)))) < 1e-10


def test_scalar_mass_matrix_single_particle(orc):
    # x = (1.25, 2.5, 3.75) on 8^3, q w = -3: M_{g,g+o} = -3 W_g W_{g+o}, by hand
    x = _one([1.25, 2.5, 3.75])
    M = orc.mass_matrix_scalar([8, 8, 8], x, np.float32([-1.0]), np.float32([3.0]))
    wx = {1: .75, 2: .25}
    wy = {2: .5, 3: .5}
    wz = {3: .25, 4: .75}
    nz = 0
    for gz in wz:
        for gy in wy:
            for gx in wx:
                for o, (dx, dy, dz) in enumerate(OFFS):
                    hx, hy, hz = gx + dx, gy + dy, gz + dz
                    if hx in wx and hy in wy and hz in wz:
                        val = -3.0 * (wx[gx] * wy[gy] * wz[gz]) * (wx[hx] * wy[hy] * wz[hz])
                        assert M[gz, gy, gx, o] == val
                        nz += 1
    assert nz == 64 and np.count_nonzero(M) == 64


def test_scalar_mass_matrix_is_the_zero_field_tensor_diagonal(orc):
    """B = 0 gives alpha = I, so each diagonal component of the ECSIM matrix is
    the scalar matrix ([MM] Eq.(6) with s = q delta_ij)."""
    r = np.random.default_rng(43)
    n = [5, 4, 6]
    x, B, q, w, beta = _mm_inputs(r, n, 300, zero_B=True)
    Ms = orc.mass_matrix_scalar(n, x, q, w)
    Mt = orc.mass_matrix(n, x, B, q, w, beta)
    for i in range(3):
        assert np.abs(Mt[..., i, i] - Ms).max() < 1e-13


# ---------------------------------------------------------------------------
# 1-D windowed sweep  ([CS] "The problem", "Code")
# ---------------------------------------------------------------------------

SW = dict(nb=1024, T=50, dt=0.02, hw=0.005)


def test_sweep_centred_particle(orc):
    # x0 = 1/2, v = 0: only step t = 25 (centre 1/2) selects it, d = 0, weight 1;
    # g = 512 - 1/2 -> bins 511, 512 get 1/2 each
    H = orc.sweep1d(SW["nb"], [0.5], [0.0], SW["T"], SW["dt"], SW["hw"])
    exp = np.zeros(1024)
    exp[511] = exp[512] = 0.5
    assert np.array_equal(H, exp)


def test_sweep_offset_particle(orc):
    # x0 = 1/2 + 1/512: d = 1/512, weight (1 - 0.390625)^2 = 0.371337890625;
    # g = 513.5 -> bins 513 and 514 get half each
    H = orc.sweep1d(SW["nb"], [0.5 + 1 / 512], [0.0], SW["T"], SW["dt"], SW["hw"])
    exp = np.zeros(1024)
    exp[513] = exp[514] = 0.371337890625 / 2
    assert np.allclose(H, exp, rtol=1e-15, atol=0)


def test_sweep_bin_and_window_wrap(orc):
    # x0 = 1/4096, v = 0: selected only at t = 50 (centre 1 == 0 by minimum image),
    # d = 1/4096 -> weight (1 - 0.048828125)^2; g = -1/4 -> j = -1, f = 3/4:
    # bin 1023 gets 1/4, bin 0 (whose centre 1/2048 is nearer) gets 3/4
    H = orc.sweep1d(SW["nb"], [1 / 4096], [0.0], SW["T"], SW["dt"], SW["hw"])
    wt = (1 - 0.048828125) ** 2
    exp = np.zeros(1024)
    exp[1023] = 0.25 * wt
    exp[0] = 0.75 * wt
    assert np.allclose(H, exp, rtol=1e-15, atol=0)


def test_sweep_moving_particle_position_wrap(orc):
    # x0 = 0.9, v = -1: x(t) = 0.9 - 0.02 t wraps below 0; the window centre moves
    # +0.02 per step, so the particle meets it when 0.9 - 0.02t = 0.02t (mod 1),
    # i.e. t = 22.5 (no) or 0.9 + 1 = 0.04t -> t = 47.5 (no): never within 0.005
    H = orc.sweep1d(SW["nb"], [0.9], [-1.0], SW["T"], SW["dt"], SW["hw"])
    assert not H.any()
    # x0 = 0.92, v = -1: meets the centre when 0.92 - 0.04 t is an integer: t = 23
    # (x = 0.46) and, after wrapping below 0, t = 48 (x = 0.96); d = 0 both times
    H = orc.sweep1d(SW["nb"], [0.92], [-1.0], SW["T"], SW["dt"], SW["hw"])
    nzb = np.nonzero(H)[0]
    # 0.46*1024 - 1/2 = 470.54 -> bins 470, 471; 0.96*1024 - 1/2 = 982.54 -> 982, 983
    assert set(nzb) == {470, 471, 982, 983} and abs(H.sum() - 2.0) < 1e-12
    assert abs(H[470] - 0.46) < 1e-9 and abs(H[983] - 0.54) < 1e-9


def test_sweep_is_linear_in_particles(orc):
    wl = synthetic.sweep_workload(count=300, seed=5)
    Hall = orc.sweep1d(wl.nb, wl.x0, wl.v, wl.T, wl.dt, wl.hw)
    Hsum = sum(orc.sweep1d(wl.nb, wl.x0[i:i + 1], wl.v[i:i + 1], wl.T, wl.dt, wl.hw)
               for i in range(300))
    assert np.allclose(Hall, Hsum, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# 1-D sweep, reverse  ([CS] "Code": the gradient of sum (H - target)^2 in x0)

def test_sweep_grad_hand_values(orc):
    """One step (T = 1: the window centre is c = 1 = 0 mod 1), v = 0, nb = 8,
    hw = 1/4, dyadic positions, by hand from the forward formulas."""
    def g(x0, dH):
        return orc.sweep1d_grad(8, [x0], [0.0], 1, 0.5, 0.25, dH)[0]
    # x0 = 1/16: d = 1/16, u = 3/4, w = 9/16, dw/dx = -6; g = 0 -> j = 0, f = 0:
    # -6 (1 dH0 + 0 dH1) + (9/16) 8 (dH1 - dH0) = -10.5 dH0 + 4.5 dH1
    assert g(1 / 16, [1, 2, 0, 0, 0, 0, 0, 0]) == -1.5
    # x0 = 29/32: d = -3/32, u = 5/8, w = 25/64, dw/dx = +5; g = 6.75 -> j = 6,
    # f = 3/4: 5 (dH6/4 + 3 dH7/4) + (25/8)(dH7 - dH6)
    assert g(29 / 32, [0, 0, 0, 0, 0, 0, 3, -1]) == -12.5
    # x0 = 1/64: d = 1/64, u = 15/16, w = 225/256, dw/dx = -7.5; g = -3/8 -> j = -1
    # (bin 7), f = 5/8: -7.5 (3/8 dH7 + 5/8 dH0) + (225/32)(dH0 - dH7)
    assert g(1 / 64, [2, 0, 0, 0, 0, 0, 0, 1]) == -5.15625
    # outside the window (|d| = 1/4 is not < hw): no contribution
    assert g(0.25, [1, 1, 1, 1, 1, 1, 1, 1]) == 0.0


def test_sweep_grad_matches_finite_differences(orc):
    """Central differences of L(x0) = sum (H(x0) - target)^2 over the oracle's own
    forward sweep, particle by particle: L is piecewise smooth, and a random
    particle is not within eps of a kink (|d| = 0, a bin centre)."""
    r = np.random.default_rng(81)
    nb, T, dt, hw, n = 64, 20, 0.02, 0.06, 40
    x0 = r.random(n)
    v = r.normal(0.0, 0.3, n)
    target = r.random(nb)
    H = orc.sweep1d(nb, x0, v, T, dt, hw)
    grad = orc.sweep1d_grad(nb, x0, v, T, dt, hw, 2.0 * (H - target))
    assert np.count_nonzero(grad) > n // 2
    eps = 1e-6
    for i in range(n):
        xp = x0.copy()
        xp[i] += eps
        xm = x0.copy()
        xm[i] -= eps
        lp = np.sum((orc.sweep1d(nb, xp, v, T, dt, hw) - target) ** 2)
        lm = np.sum((orc.sweep1d(nb, xm, v, T, dt, hw) - target) ** 2)
        fd = (lp - lm) / (2 * eps)
        assert abs(fd - grad[i]) <= 1e-5 * max(1.0, abs(grad[i])), (i, fd, grad[i])


def test_sweep_grad_zero_when_never_selected(orc):
    # T = 10 window centres at 0.1, ..., 1.0 with hw = 0.01: a particle resting
    # at 0.05 is never inside, so neither H nor dL/dx0 sees it
    dH = np.linspace(-1, 1, 32)
    g = orc.sweep1d_grad(32, [0.05, 0.3], [0.0, 0.0], 10, 0.02, 0.01, dH)
    assert g[0] == 0.0 and g[1] != 0.0


# ---------------------------------------------------------------------------
# Scalar mass matrix with TSC weights  ([MM] Eq.(6) scalar case, §2.3 order 2)

OFFS5 = [(dx, dy, dz) for dz in (-2, -1, 0, 1, 2) for dy in (-2, -1, 0, 1, 2)
         for dx in (-2, -1, 0, 1, 2)]


def _weights_matrix_tsc(orc, n, x):
    """Dense TSC W (Ng x Np) from the oracle's own order-2 deposit."""
    npart = x[0].size
    W = np.zeros((int(np.prod(n)), npart))
    for p in range(npart):
        J = orc.deposit(3, n, 2, [a[p:p + 1] for a in x],
                        [np.float32([1]), np.float32([0]), np.float32([0])],
                        np.float32([1]), np.float32([1]))
        W[:, p] = J[0].ravel()
    return W


def test_tsc_scalar_mass_matrix_equals_dense_contraction(orc):
    """[MM] Eq.(10): W diag(q w) W^T on a 5^3 grid (the 125 offsets are then every
    node once), against the 125-offset store."""
    r = np.random.default_rng(45)
    n = [5, 5, 5]
    x, _, q, w, _ = _mm_inputs(r, n, 120)
    M = orc.mass_matrix_scalar_tsc(n, x, q, w)
    W = _weights_matrix_tsc(orc, n, x)
    dense = W @ np.diag(q.astype(np.float64) * w.astype(np.float64)) @ W.T
    store = np.zeros((125, 125))
    for gz in range(5):
        for gy in range(5):
            for gx in range(5):
                g = gx + 5 * (gy + 5 * gz)
                for o, (dx, dy, dz) in enumerate(OFFS5):
                    g2 = (gx + dx) % 5 + 5 * (((gy + dy) % 5) + 5 * ((gz + dz) % 5))
                    store[g, g2] += M[gz, gy, gx, o]
    assert np.abs(store - dense).max() < 1e-12 * max(1.0, np.abs(dense).max())


def test_tsc_scalar_mass_matrix_symmetry_and_charge(orc):
    """Eq.(11) symmetry; row sums equal the TSC deposit of q w; total sum q w."""
    r = np.random.default_rng(46)
    n = [7, 6, 8]
    x, _, q, w, _ = _mm_inputs(r, n, 400)
    M = orc.mass_matrix_scalar_tsc(n, x, q, w)
    for o, (dx, dy, dz) in enumerate(OFFS5):
        mo = OFFS5.index((-dx, -dy, -dz))
        rolled = np.roll(M[..., mo], shift=(-dz, -dy, -dx), axis=(0, 1, 2))
        assert np.abs(M[..., o] - rolled).max() < 1e-13
    ones, zeros = np.ones_like(q), np.zeros_like(q)
    J = orc.deposit(3, n, 2, x, [ones, zeros, zeros], q, w)
    assert np.abs(M.sum(axis=3) - J[0]).max() < 1e-12
    assert abs(M.sum() - float(np.sum(q.astype(np.float64) * w.astype(np.float64)))) < 1e-10


def test_tsc_scalar_mass_matrix_single_particle(orc):
    # x = (3.0, 2.25, 3.75) on 8^3, q w = 2.  TSC weights by hand ([MM] §2.3):
    # x: frac 0 -> base 2, (1/8, 3/4, 1/8); y: frac 1/4 < 1/2 -> base 1,
    # (1/32, 11/16, 9/32); z: frac 3/4 -> base 3, (9/32, 11/16, 1/32)
    x = _one([3.0, 2.25, 3.75])
    M = orc.mass_matrix_scalar_tsc([8, 8, 8], x, np.float32([2.0]), np.float32([1.0]))
    wx = {2: 0.125, 3: 0.75, 4: 0.125}
    wy = {1: 0.03125, 2: 0.6875, 3: 0.28125}
    wz = {3: 0.28125, 4: 0.6875, 5: 0.03125}
    nz = 0
    for gz in wz:
        for gy in wy:
            for gx in wx:
                for o, (dx, dy, dz) in enumerate(OFFS5):
                    hx, hy, hz = gx + dx, gy + dy, gz + dz
                    if hx in wx and hy in wy and hz in wz:
                        assert M[gz, gy, gx, o] == 2.0 * (wx[gx] * wy[gy] * wz[gz]) * (
                            wx[hx] * wy[hy] * wz[hz])
                        nz += 1
    assert nz == 729 and np.count_nonzero(M) == 729


# ---------------------------------------------------------------------------
# ECSIM mass matrix with TSC weights  ([MM] Eq.(4)-(6), §2.3 order 2)

def test_tsc_mass_matrix_equals_dense_contraction(orc):
    """[MM] Eq.(10) per component: M^ij = W diag(q w alpha^ij) W^T on 5^3 with the
    order-2 W, against the 125-offset store."""
    r = np.random.default_rng(47)
    n = [5, 5, 5]
    x, B, q, w, beta = _mm_inputs(r, n, 80)
    M = orc.mass_matrix_tsc(n, x, B, q, w, beta)
    W = _weights_matrix_tsc(orc, n, x)
    s = _coeffs(orc, B, q, w, beta)
    for ij in range(9):
        dense = W @ np.diag(s[:, ij]) @ W.T
        store = np.zeros((125, 125))
        for gz in range(5):
            for gy in range(5):
                for gx in range(5):
                    g = gx + 5 * (gy + 5 * gz)
                    for o, (dx, dy, dz) in enumerate(OFFS5):
                        g2 = (gx + dx) % 5 + 5 * (((gy + dy) % 5) + 5 * ((gz + dz) % 5))
                        store[g, g2] += M[gz, gy, gx, o].ravel()[ij]
        assert np.abs(store - dense).max() < 1e-12 * max(1.0, np.abs(dense).max())


def test_tsc_mass_matrix_symmetry_row_sums_and_zero_field(orc):
    """Eq.(11) component-wise symmetry; block row sums W s; with B = 0 each diagonal
    component is the scalar TSC matrix and the off-diagonal ones vanish."""
    r = np.random.default_rng(48)
    n = [6, 5, 7]
    x, B, q, w, beta = _mm_inputs(r, n, 300)
    M = orc.mass_matrix_tsc(n, x, B, q, w, beta)
    for o, (dx, dy, dz) in enumerate(OFFS5):
        mo = OFFS5.index((-dx, -dy, -dz))
        rolled = np.roll(M[:, :, :, mo], shift=(-dz, -dy, -dx), axis=(0, 1, 2))
        assert np.abs(M[:, :, :, o] - rolled).max() < 1e-13
    s = _coeffs(orc, B, q, w, beta)
    rows = M.sum(axis=3).reshape(-1, 9)
    W = _weights_matrix_tsc(orc, n, x)
    for ij in range(9):
        assert np.abs(rows[:, ij] - W @ s[:, ij]).max() < 1e-12
    x, B, q, w, beta = _mm_inputs(r, n, 200, zero_B=True)
    M0 = orc.mass_matrix_tsc(n, x, B, q, w, beta)
    Ms = orc.mass_matrix_scalar_tsc(n, x, q, w)
    for i in range(3):
        assert np.abs(M0[..., i, i] - Ms).max() < 1e-13
    assert np.abs(M0[..., 0, 1]).max() == 0 and np.abs(M0[..., 2, 1]).max() == 0


# ---------------------------------------------------------------------------
# Charge-conserving zigzag deposit  ([TD] "Halo sizing", reading in the header)

def _zz_inputs(r, n, npart):
    x = [r.uniform(0, n[k], npart).astype(np.float32) for k in range(3)]
    xp = [(x[k] - r.uniform(-0.95, 0.95, npart)).astype(np.float32) for k in range(3)]
    q = np.where(r.random(npart) < 0.5, 1.0, -1.0).astype(np.float32)
    w = r.uniform(0.5, 1.5, npart).astype(np.float32)
    return x, xp, q, w


def test_zigzag_conserves_charge(orc):
    """rho(x) - rho(xp) + div J = 0 at every node, with rho the oracle's own CIC
    charge deposit and J_c staggered by half a cell along c (moves that cross
    cells and the periodic boundary included)."""
    r = np.random.default_rng(51)
    n = [6, 5, 7]
    x, xp, q, w = _zz_inputs(r, n, 400)
    J = orc.deposit_zigzag(n, x, xp, q, w)
    ones, zeros = np.ones_like(q), np.zeros_like(q)
    rho1 = orc.deposit(3, n, 1, x, [ones, zeros, zeros], q, w)[0]
    rho0 = orc.deposit(3, n, 1, xp, [ones, zeros, zeros], q, w)[0]
    div = sum(J[c] - np.roll(J[c], 1, axis=2 - c) for c in range(3))
    assert np.abs(rho1 - rho0 + div).max() < 1e-12


def test_zigzag_total_current(orc):
    """sum_g J_c = sum_p q w (x_c - xp_c) per component."""
    r = np.random.default_rng(52)
    n = [5, 6, 5]
    x, xp, q, w = _zz_inputs(r, n, 300)
    J = orc.deposit_zigzag(n, x, xp, q, w)
    qw = q.astype(np.float64) * w
    for c in range(3):
        tot = np.sum(qw * (x[c].astype(np.float64) - xp[c].astype(np.float64)))
        assert abs(J[c].sum() - tot) < 1e-11


def test_zigzag_single_particle(orc):
    # xp = (2.25, 3.5, 1.5) -> x = (2.75, 3.5, 1.5), q w = 1, inside cell (2, 3, 1):
    # relay at x = 2.5; each half carries F_x = 1/4 at transverse weights 1/2,
    # so J_x = 2 * 1/4 * 1/4 = 1/8 at the four nodes (2, 3..4, 1..2); no J_y, J_z
    J = orc.deposit_zigzag([8, 8, 8], _one([2.75, 3.5, 1.5]), _one([2.25, 3.5, 1.5]),
                           np.float32([1.0]), np.float32([1.0]))
    exp = np.zeros_like(J)
    for gz in (1, 2):
        for gy in (3, 4):
            exp[0, gz, gy, 2] = 0.125
    assert np.array_equal(J, exp)


def test_zigzag_single_particle_bound(orc):
    """A move of less than a cell puts at most 2 * 13/12 |q w| on any one J value
    (two segments, each |F'| <= 1 with weights in [0, 1] and the cross term at
    most 1/12): the bound the tiled kernel's fixed-point scale rests on.  Moves
    that reach the edge of the bound's assumptions (near a whole cell, across
    the periodic boundary) are included."""
    r = np.random.default_rng(53)
    n = [6, 6, 6]
    worst = 0.0
    for _ in range(300):
        x = [np.float32([r.uniform(0, n[k])]) for k in range(3)]
        d = r.choice([-0.999, 0.999], 3) * r.uniform(0.5, 1.0, 3)
        xp = [(x[k] - np.float32(d[k])).astype(np.float32) for k in range(3)]
        qw = r.uniform(0.5, 1.5)
        J = orc.deposit_zigzag(n, x, xp, np.float32([1.0]), np.float32([qw]))
        worst = max(worst, float(np.abs(J).max()) / float(np.float32(qw)))
    assert worst <= 2.0 * 13.0 / 12.0
    assert worst > 0.5  # long moves do come near it
