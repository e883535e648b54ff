"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def say(*a):
    """Name the case before a GPU step, flushed, so a crash log identifies it."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.detach().cpu().numpy()


def u32(t):
    return host(t).view(np.uint32)


def rel_max_err(got, ref):
    """max |got - ref| / max |ref| over the whole array (the deposit tolerance)."""
    scale = np.abs(ref).max()
    return float(np.abs(got.astype(np.float64) - ref).max() / (scale if scale > 0 else 1.0))


def rel_frob_err(got, ref):
    scale = np.linalg.norm(ref)
    return float(np.linalg.norm(got.astype(np.float64) - ref) / (scale if scale > 0 else 1.0))


def particle_arrays(wl, use_next=True):
    """Device copies in the order the library's permute takes them:
    x (dim arrays), v (3), q, w."""
    xs = wl.x_next if use_next else wl.x
    return [dev(a) for a in xs] + [dev(a) for a in wl.v] + [dev(wl.q), dev(wl.w)]


_FULL = {}


def full_workload(name):
    """The named full-size workload, generated once per test session."""
    import synthetic

    if name not in _FULL:
        _FULL.clear()   # keep at most one full-size workload in host memory
        _FULL[name] = synthetic.workload(name)
    return _FULL[name]


# ---------------------------------------------------------------------------
# Independent checks of the mass matrices at full size (numpy, fp64)
# ---------------------------------------------------------------------------

def axis_weights(x, n, order):
    """B-spline weights on one axis (the mass-matrix paper, §2.3 Eq.(12)):
    the first support node (wrapped) and the order + 1 weights, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    i = np.floor(x)
    f = x - i
    if order == 1:
        base, ws = i, [1.0 - f, f]
    else:
        lo = f < 0.5
        base = np.where(lo, i - 1.0, i)
        d = np.where(lo, f, f - 1.0)
        ws = [0.5 * (0.5 - d) ** 2, 0.75 - d * d, 0.5 * (0.5 + d) ** 2]
    return base.astype(np.int64) % n, ws


def node_row_sums(n, x, order, coefs):
    """sum_p c_p W_pg at every node g, for each coefficient array c in `coefs`:
    the block row sums sum_o M_{g,g+o} of a mass matrix whose per-particle
    coefficient is c (the mass-matrix paper, Eq.(11): M is W diag(c) W^T and the
    weights of a particle sum to one).  Returns [len(coefs), nz, ny, nx] fp64."""
    nx, ny, nz = n
    ng = nx * ny * nz
    (bx, wx), (by, wy), (bz, wz) = [axis_weights(x[k], n[k], order) for k in range(3)]
    cf = [np.asarray(c, dtype=np.float64) for c in coefs]
    out = np.zeros((len(cf), ng))
    for az in range(order + 1):
        gz = (bz + az) % nz
        for ay in range(order + 1):
            gzy = gz * ny + (by + ay) % ny
            wzy = wz[az] * wy[ay]
            for ax in range(order + 1):
                g = gzy * nx + (bx + ax) % nx
                W = wzy * wx[ax]
                for k, c in enumerate(cf):
                    out[k] += np.bincount(g, weights=c * W, minlength=ng)
    return out.reshape(len(cf), nz, ny, nx)


def alpha_coefs(wl):
    """q w alpha^{ij} per particle, i, j = 0..2 (row-major, 9 fp64 arrays), with
    alpha = (I - C(omega) + omega omega^T) / (1 + |omega|^2), C(omega)u = omega x u,
    omega = beta B (the mass-matrix paper, Eq.(5) with c = 1)."""
    om = np.stack([wl.beta.astype(np.float64) * b for b in wl.B])
    den = 1.0 + (om * om).sum(axis=0)
    qw = wl.q.astype(np.float64) * wl.w
    eps = np.zeros((3, 3, 3))
    eps[0, 1, 2] = eps[1, 2, 0] = eps[2, 0, 1] = 1
    eps[0, 2, 1] = eps[2, 1, 0] = eps[1, 0, 2] = -1
    out = []
    for i in range(3):
        for j in range(3):
            out.append(qw * ((i == j) + np.einsum("k,kp->p", eps[i, j], om) + om[i] * om[j]) / den)
    return out


def block_row_sums(M):
    """sum_o M_{g,g+o} per node and component, in fp64: [k, nz, ny, nx] for M
    of shape [nz, ny, nx, offsets] + component shape (k components)."""
    s = M.sum(axis=3, dtype=np.float64)
    return np.moveaxis(s.reshape(M.shape[:3] + (-1,)), -1, 0)


def check_row_sums(got, ref, abs_ref, tol):
    """|got - ref| <= tol * A_g at every node and component, with
    A_g = sum_p |c_p| W_pg (what the accumulated rounding of an entry scales
    with).  Returns the worst ratio to the bound."""
    worst = float((np.abs(got - ref) / (tol * abs_ref + 1e-300)).max())
    assert worst <= 1.0, f"row sums off by {worst:.3g} x the bound"
    return worst


def seam_cells(n, step):
    """Cell planes z with z mod step in {step-2, step-1, 0} and the node planes
    z mod step in {step-1, 0} that only they reach (node z touches cells z-1, z):
    both sides of every plane z = k step, the wrap 0 | n-1 included."""
    z = np.arange(n)
    return (z % step >= step - 2) | (z % step == 0), (z % step == step - 1) | (z % step == 0)


def full_size_checks(orc, wl, M, tol):
    """The full-size checks of a CIC tensor mass matrix M (fp32 or fp64, 64^3
    or any grid whose n_z is a multiple of 8), tolerance `tol`.
    (1) Element-wise: the oracle runs on the particles of the cell planes on
    both sides of every z plane 8k (the wrap 63 | 0 included); the node rows
    they alone reach are compared entry by entry.  The slab spans the whole
    x-y extent, so every x and y column boundary is crossed as well.
    (2) Every row: the block row sums sum_o M_{g,g+o} equal sum_p q w alpha_p
    W_pg (Eq.(11) with the weights' partition of unity), computed in numpy."""
    cells, rows = seam_cells(wl.n[2], 8)
    cz = np.floor(wl.x[2]).astype(np.int64)
    sub = wl.take(np.nonzero(cells[cz])[0])
    ref = orc.mass_matrix(wl.n, sub.x, sub.B, sub.q, sub.w, sub.beta)
    _check_tol(M[rows], ref[rows], tol)
    del ref
    coefs = alpha_coefs(wl)
    want = node_row_sums(wl.n, wl.x, 1, coefs)
    scale = node_row_sums(wl.n, wl.x, 1, [np.abs(c) for c in coefs])
    worst = check_row_sums(block_row_sums(M), want, scale, tol)
    say("row sums: worst error / bound", worst)


def _check_tol(M, ref, tol):
    assert rel_frob_err(M, ref) <= tol
    assert np.abs(M - ref).max() <= tol * np.abs(ref).max()


def component_errors(J, ref):
    """Per component c of a current: max |J_c - ref_c| / max |ref_c| (the
    deposit tolerance applied to each component on its own)."""
    return [rel_max_err(J[c], ref[c]) for c in range(J.shape[0])]
