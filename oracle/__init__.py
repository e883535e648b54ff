"""fp64 CPU oracle for particle-to-grid scatter deposition (ctypes wrapper).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in the graft entry
module and the ``cpu_baseline`` leg of ``bench.py`` may import this package.
The product library (``particle_cell_grid_amd``) never imports it, and this
package never imports the product: the two share nothing but the seeded input
arrays produced by ``synthetic``.

The arithmetic lives in ``oracle.c`` (plain C, fp64, single-threaded loops in
particle order); this module only marshals numpy arrays.  Each wrapper names
the passage of the pages it follows; the C source states the definitions.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-adds, so every fp64 operation rounds
# exactly as written (the GPU sweep kernel makes the same choice).
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc and return its path."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """The loaded oracle library.  PCG_ORACLE_LIB names another build of
    oracle.c to load instead (the mutant tests load copies with a planted
    mistake, to show that the pins catch it)."""
    global _lib
    if _lib is None:
        path = os.environ.get("PCG_ORACLE_LIB") or _LIB
        if path == _LIB and not os.path.exists(_LIB):
            build(force=True)
        L = C.CDLL(path)
        i32p = C.POINTER(C.c_int32)
        fpp = C.POINTER(C.c_void_p)
        L.oracle_shape_1d.argtypes = [C.c_int, C.c_double, C.POINTER(C.c_int64), C.c_void_p]
        L.oracle_shape_1d.restype = C.c_int
        L.oracle_deposit.argtypes = [C.c_int, i32p, C.c_int, C.c_int64, fpp, fpp,
                                     C.c_void_p, C.c_void_p, C.c_void_p]
        L.oracle_deposit.restype = C.c_int
        L.oracle_tile_keys.argtypes = [C.c_int, i32p, C.c_int, C.c_int, C.c_int64, fpp, C.c_void_p]
        L.oracle_tile_keys.restype = C.c_int
        L.oracle_stable_sort.argtypes = [C.c_int64, C.c_void_p, C.c_uint32, C.c_void_p, C.c_void_p]
        L.oracle_stable_sort.restype = C.c_int
        L.oracle_escape.argtypes = [C.c_int, i32p, C.c_int, C.c_int, C.c_int, C.c_int64, fpp,
                                    C.c_void_p, C.c_int64, C.c_void_p]
        L.oracle_escape.restype = C.c_int64
        L.oracle_alpha.argtypes = [C.c_void_p, C.c_void_p]
        L.oracle_alpha.restype = None
        L.oracle_mass_matrix.argtypes = [i32p, C.c_int64, fpp, fpp, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_void_p]
        L.oracle_mass_matrix.restype = C.c_int
        L.oracle_mass_matrix_tsc.argtypes = [i32p, C.c_int64, fpp, fpp, C.c_void_p, C.c_void_p,
                                         C.c_void_p, C.c_void_p]
        L.oracle_mass_matrix_tsc.restype = C.c_int
        L.oracle_deposit_zigzag.argtypes = [i32p, C.c_int64, fpp, fpp, C.c_void_p, C.c_void_p,
                                            C.c_void_p]
        L.oracle_deposit_zigzag.restype = C.c_int
        L.oracle_mass_matrix_scalar.argtypes = [i32p, C.c_int64, fpp, C.c_void_p, C.c_void_p,
                                                C.c_void_p]
        L.oracle_mass_matrix_scalar.restype = C.c_int
        L.oracle_mass_matrix_scalar_tsc.argtypes = [i32p, C.c_int64, fpp, C.c_void_p, C.c_void_p,
                                                C.c_void_p]
        L.oracle_mass_matrix_scalar_tsc.restype = C.c_int
        L.oracle_sweep1d.argtypes = [C.c_int, C.c_int64, C.c_void_p, C.c_void_p, C.c_int,
                                     C.c_double, C.c_double, C.c_void_p]
        L.oracle_sweep1d.restype = C.c_int
        L.oracle_sweep1d_grad.argtypes = [C.c_int, C.c_int64, C.c_void_p, C.c_void_p, C.c_int,
                                          C.c_double, C.c_double, C.c_void_p, C.c_void_p]
        L.oracle_sweep1d_grad.restype = C.c_int
        _lib = L
    return _lib


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return a.ctypes.data_as(C.c_void_p)


def _grid(n):
    n = list(n) + [1] * (3 - len(n))
    return (C.c_int32 * 3)(*[int(v) for v in n])


def _ptrs(arrs, keep):
    out = (C.c_void_p * 3)()
    for k, a in enumerate(arrs):
        if a is None:
            out[k] = None
        else:
            a = _f32(a)
            keep.append(a)
            out[k] = a.ctypes.data
    return out


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (status {rc})")


# ----------------------------------------------------------------------------
# public wrappers
# ----------------------------------------------------------------------------

def shape_1d(order: int, x: float):
    """Mass-matrix paper §2.3 Eq.(12): (first support node, weights) on one axis."""
    base = C.c_int64()
    w = np.zeros(3, dtype=np.float64)
    m = lib().oracle_shape_1d(int(order), float(x), C.byref(base), _ptr(w))
    _check(0 if m > 0 else -1, "shape_1d")
    return int(base.value), w[:m].copy()


def deposit(dim, n, order, x, v, q, w, J=None):
    """Current deposit J_c += q w v_c W (fp64, accumulated); J is [3, nz, ny, nx]."""
    n3 = list(n) + [1] * (3 - len(n))
    keep = []
    xs = _ptrs(list(x)[:dim] + [None] * (3 - dim), keep)
    vs = _ptrs(list(v), keep)
    q = _f32(q)
    w = _f32(w)
    if J is None:
        J = np.zeros((3, n3[2], n3[1], n3[0]), dtype=np.float64)
    assert J.dtype == np.float64 and J.flags.c_contiguous and J.size == 3 * n3[0] * n3[1] * n3[2]
    rc = lib().oracle_deposit(int(dim), _grid(n3), int(order), int(q.size), xs, vs,
                              _ptr(q), _ptr(w), _ptr(J))
    _check(rc, "deposit")
    return J


def tile_keys(dim, n, order, T, x):
    """Entity tiled-deposit page, "The tile-based spatial sort": tile key per particle."""
    keep = []
    xs = _ptrs(list(x)[:dim] + [None] * (3 - dim), keep)
    npart = int(np.asarray(x[0]).size)
    key = np.zeros(npart, dtype=np.uint32)
    rc = lib().oracle_tile_keys(int(dim), _grid(n), int(order), int(T), npart, xs, _ptr(key))
    _check(rc, "tile_keys")
    return key


def stable_sort(key, nkeys):
    """Stable counting sort: (perm, offsets[nkeys+1])."""
    key = np.ascontiguousarray(key, dtype=np.uint32)
    perm = np.zeros(key.size, dtype=np.uint32)
    offsets = np.zeros(int(nkeys) + 1, dtype=np.uint32)
    rc = lib().oracle_stable_sort(int(key.size), _ptr(key), int(nkeys), _ptr(perm), _ptr(offsets))
    _check(rc, "stable_sort")
    return perm, offsets


def ntiles(dim, n, T):
    n3 = list(n) + [1] * (3 - len(n))
    t = 1
    for k in range(dim):
        t *= n3[k] // T
    return t


def tile_sort(dim, n, order, T, x):
    """Keys, then the stable sort: (keys, perm, tile_offsets)."""
    keys = tile_keys(dim, n, order, T, x)
    perm, off = stable_sort(keys, ntiles(dim, n, T))
    return keys, perm, off


def escape(dim, n, order, T, D, x, tile_offsets, n_part=None):
    """Escape-valve classification of a tiled layout: (count, escaped[n] as bool)."""
    keep = []
    xs = _ptrs(list(x)[:dim] + [None] * (3 - dim), keep)
    npart = int(np.asarray(x[0]).size)
    if n_part is None:
        n_part = npart
    off = np.ascontiguousarray(tile_offsets, dtype=np.uint32)
    assert off.size == ntiles(dim, n, T) + 1
    esc = np.zeros(npart, dtype=np.uint8)
    cnt = lib().oracle_escape(int(dim), _grid(n), int(order), int(T), int(D), npart, xs,
                              _ptr(off), int(n_part), _ptr(esc))
    if cnt < 0:
        raise ValueError("oracle escape: invalid arguments")
    return int(cnt), esc.astype(bool)


def alpha(omega):
    """Mass-matrix paper §2.1 Eq.(5): rotation-response tensor, 3x3 row-major."""
    om = np.ascontiguousarray(omega, dtype=np.float64)
    out = np.zeros(9, dtype=np.float64)
    lib().oracle_alpha(_ptr(om), _ptr(out))
    return out.reshape(3, 3)


def mass_matrix(n, x, B, q, w, beta, M=None):
    """ECSIM mass matrix, 27-offset store [nz, ny, nx, 27, 3, 3] fp64 (accumulated)."""
    n3 = list(n)
    keep = []
    xs = _ptrs(list(x), keep)
    bs = _ptrs(list(B), keep)
    q, w, beta = _f32(q), _f32(w), _f32(beta)
    if M is None:
        M = np.zeros((n3[2], n3[1], n3[0], 27, 3, 3), dtype=np.float64)
    assert M.dtype == np.float64 and M.flags.c_contiguous
    rc = lib().oracle_mass_matrix(_grid(n3), int(q.size), xs, bs, _ptr(q), _ptr(w), _ptr(beta),
                                  _ptr(M))
    _check(rc, "mass_matrix")
    return M


def mass_matrix_tsc(n, x, B, q, w, beta, M=None):
    """ECSIM mass matrix with TSC weights, 125-offset store [nz, ny, nx, 125, 3, 3]
    fp64 (accumulated)."""
    n3 = list(n)
    keep = []
    xs = _ptrs(list(x), keep)
    bs = _ptrs(list(B), keep)
    q, w, beta = _f32(q), _f32(w), _f32(beta)
    if M is None:
        M = np.zeros((n3[2], n3[1], n3[0], 125, 3, 3), dtype=np.float64)
    assert M.dtype == np.float64 and M.flags.c_contiguous
    rc = lib().oracle_mass_matrix_tsc(_grid(n3), int(q.size), xs, bs, _ptr(q), _ptr(w),
                                      _ptr(beta), _ptr(M))
    _check(rc, "mass_matrix_tsc")
    return M


def deposit_zigzag(n, x, xp, q, w, J=None):
    """Charge-conserving zigzag current deposit, J fp64 [3, nz, ny, nx] (accumulated;
    J_c staggered by half a cell along c).  x: new positions, xp: previous ones
    (unwrapped, less than one cell away per axis)."""
    n3 = list(n)
    keep = []
    xs = _ptrs(list(x), keep)
    ps = _ptrs(list(xp), keep)
    q, w = _f32(q), _f32(w)
    if J is None:
        J = np.zeros((3, n3[2], n3[1], n3[0]), dtype=np.float64)
    assert J.dtype == np.float64 and J.flags.c_contiguous
    rc = lib().oracle_deposit_zigzag(_grid(n3), int(q.size), xs, ps, _ptr(q), _ptr(w), _ptr(J))
    _check(rc, "deposit_zigzag")
    return J


def mass_matrix_scalar(n, x, q, w, M=None):
    """Scalar mass matrix (one component per node pair), 27-offset store
    [nz, ny, nx, 27] fp64 (accumulated)."""
    n3 = list(n)
    keep = []
    xs = _ptrs(list(x), keep)
    q, w = _f32(q), _f32(w)
    if M is None:
        M = np.zeros((n3[2], n3[1], n3[0], 27), dtype=np.float64)
    assert M.dtype == np.float64 and M.flags.c_contiguous
    rc = lib().oracle_mass_matrix_scalar(_grid(n3), int(q.size), xs, _ptr(q), _ptr(w), _ptr(M))
    _check(rc, "mass_matrix_scalar")
    return M


def mass_matrix_scalar_tsc(n, x, q, w, M=None):
    """Scalar mass matrix with TSC weights (27 support nodes), 125-offset store
    [nz, ny, nx, 125] fp64 (accumulated)."""
    n3 = list(n)
    keep = []
    xs = _ptrs(list(x), keep)
    q, w = _f32(q), _f32(w)
    if M is None:
        M = np.zeros((n3[2], n3[1], n3[0], 125), dtype=np.float64)
    assert M.dtype == np.float64 and M.flags.c_contiguous
    rc = lib().oracle_mass_matrix_scalar_tsc(_grid(n3), int(q.size), xs, _ptr(q), _ptr(w),
                                             _ptr(M))
    _check(rc, "mass_matrix_scalar_tsc")
    return M


def sweep1d(nb, x0, v, T, dt, hw):
    """Compaction/scatter-add page: windowed 1-D CIC sweep, H fp64 [nb] (overwritten)."""
    x0 = np.ascontiguousarray(x0, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    H = np.zeros(int(nb), dtype=np.float64)
    rc = lib().oracle_sweep1d(int(nb), int(x0.size), _ptr(x0), _ptr(v), int(T), float(dt),
                              float(hw), _ptr(H))
    _check(rc, "sweep1d")
    return H


def sweep1d_grad(nb, x0, v, T, dt, hw, dH):
    """The reverse of sweep1d: dL/dx0 fp64 [count] for a given dL/dH (fp64 [nb])."""
    x0 = np.ascontiguousarray(x0, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    dH = np.ascontiguousarray(dH, dtype=np.float64)
    assert dH.size == int(nb)
    dx0 = np.zeros(x0.size, dtype=np.float64)
    rc = lib().oracle_sweep1d_grad(int(nb), int(x0.size), _ptr(x0), _ptr(v), int(T), float(dt),
                                   float(hw), _ptr(dH), _ptr(dx0))
    _check(rc, "sweep1d_grad")
    return dx0
