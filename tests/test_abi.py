"""The C-ABI library: it loads, exports every function include/pcg.h declares,
and rejects invalid arguments on the host with the documented status codes
before anything is enqueued (so these run without a GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# PCG_LIB names another build of the library to check (the sanitizer build)
LIB = os.environ.get("PCG_LIB") or os.path.join(ROOT, "particle_cell_grid_amd", "libpcg.so")
HEADER = os.path.join(ROOT, "include", "pcg.h")

EINVAL, EUNSUPPORTED, ELDS, EWORKSPACE = -1, -2, -3, -4


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import subprocess
        import sys

        subprocess.check_call([sys.executable, os.path.join(ROOT, "particle_cell_grid_amd",
                                                            "csrc", "build.py")])
    return C.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["pcg_tile_sort", "pcg_sort_workspace_bytes", "deposit_currents",
              "pcg_deposit_workspace_bytes", "deposit_currents_regroup",
              "pcg_deposit_regroup_workspace_bytes", "pcg_mass_workspace_bytes", "assemble_mass_matrix",
              "assemble_mass_matrix_scalar", "assemble_mass_matrix_scalar_tsc",
              "assemble_mass_matrix_tsc",
              "assemble_mass_matrix_f64",
              "assemble_mass_matrix_scalar_f64", "deposit_sweep1d", "deposit_sweep1d_grad",
              "deposit_sweep1d_loss_grad", "deposit_currents_zigzag",
              "deposit_currents_zigzag_regroup", "deposit_currents_noalloc",
              "pcg_status_string", "pcg_last_error", "pcg_version", "pcg_timing_enable",
              "pcg_timing_reset", "pcg_timing_read", "pcg_timing_names"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"libpcg.so does not export {n}"


class Grid(C.Structure):
    _fields_ = [("dim", C.c_int32), ("n", C.c_int32 * 3)]


class Particles(C.Structure):
    _fields_ = [("count", C.c_int64), ("x", C.c_void_p * 3), ("v", C.c_void_p * 3),
                ("q", C.c_void_p), ("w", C.c_void_p)]


class Tile(C.Structure):
    _fields_ = [("T", C.c_int32), ("order", C.c_int32), ("drift", C.c_int32),
                ("block", C.c_int32), ("n_partitioned", C.c_int64), ("tile_offsets", C.c_void_p)]


FAKE = 0x10000  # never dereferenced: validation fails before any launch


def grid(dim, n):
    return Grid(dim, (C.c_int32 * 3)(*(list(n) + [1] * (3 - len(n)))))


def particles(count):
    P = Particles()
    P.count = count
    for k in range(3):
        P.x[k] = FAKE
        P.v[k] = FAKE
    P.q = FAKE
    P.w = FAKE
    return P


def test_status_strings(lib):
    lib.pcg_status_string.restype = C.c_char_p
    lib.pcg_version.restype = C.c_char_p
    assert b"EINVAL" in lib.pcg_status_string(EINVAL)
    assert b"LDS" in lib.pcg_status_string(ELDS)
    assert b"gfx950" in lib.pcg_version()


def test_sort_workspace_size(lib):
    lib.pcg_sort_workspace_bytes.restype = C.c_size_t
    g = grid(3, [128, 128, 128])
    ws = lib.pcg_sort_workspace_bytes(C.byref(g), C.c_int64(1 << 20), 8)
    assert ws >= 5 * 4 * (1 << 20)
    assert lib.pcg_sort_workspace_bytes(C.byref(g), C.c_int64(100), 7) == 0   # 128 % 7
    bad = grid(4, [8, 8, 8])
    assert lib.pcg_sort_workspace_bytes(C.byref(bad), C.c_int64(100), 1) == 0


def test_deposit_validation(lib):
    lib.pcg_last_error.restype = C.c_char_p
    dc = lib.deposit_currents
    P = particles(1000)
    J = C.c_void_p(FAKE)

    def call(g, order=1, tile=None, J=J, ws=C.c_void_p(FAKE), wsb=1 << 30, P=P):
        return dc(C.byref(g), C.byref(P), order, C.byref(tile) if tile else None, J, None, ws,
                  C.c_size_t(wsb), None)

    assert call(grid(0, [1, 1, 1])) == EINVAL
    assert call(grid(2, [8, 8, 8])) == EINVAL                     # unused axis not 1
    assert call(grid(3, [8, 8, 8]), order=3) == EUNSUPPORTED
    assert call(grid(3, [8, 8, 8]), J=None) == EINVAL
    P2 = particles(1000)
    P2.q = None
    assert call(grid(3, [8, 8, 8]), P=P2) == EINVAL
    assert call(grid(3, [8, 8, 8]), P=particles(-1)) == EINVAL
    assert call(grid(3, [8, 8, 8]), P=particles(1 << 30)) == EINVAL   # 32-bit byte offsets
    g = grid(3, [64, 64, 64])
    t = Tile(8, 2, 1, 0, 1000, FAKE)
    assert call(g, order=1, tile=t) == EINVAL                     # layout keyed with TSC
    assert b"order" in lib.pcg_last_error()
    t = Tile(6, 1, 1, 0, 1000, FAKE)
    assert call(g, tile=t) == EINVAL                              # 64 % 6
    t = Tile(8, 1, -1, 0, 1000, FAKE)
    assert call(g, tile=t) == EINVAL                              # negative drift
    t = Tile(8, 1, 1, 0, 1001, FAKE)
    assert call(g, tile=t) == EINVAL                              # n_partitioned > count
    t = Tile(8, 1, 1, 0, 1000, None)
    assert call(g, tile=t) == EINVAL                              # no offsets
    t = Tile(16, 2, 8, 0, 1000, FAKE)                             # TE = 34: 34^3*12 B > 160 KiB
    assert call(g, order=2, tile=t) == ELDS
    t = Tile(8, 1, 1, 0, 1000, FAKE)
    assert call(g, tile=t, ws=None) == EWORKSPACE
    assert call(g, tile=t, wsb=16) == EWORKSPACE
    small = grid(3, [4, 4, 4])
    t = Tile(4, 1, 3, 0, 1000, FAKE)                              # drift + order >= n
    assert call(small, tile=t) == EINVAL


def test_zigzag_validation(lib):
    lib.pcg_last_error.restype = C.c_char_p
    zz = lib.deposit_currents_zigzag
    P = particles(1000)
    xp = (C.c_void_p * 3)(FAKE, FAKE, FAKE)

    def call(g, tile=None, J=C.c_void_p(FAKE), P=P, xp=xp):
        return zz(C.byref(g), C.byref(P), xp, C.byref(tile) if tile else None, J, None, None)

    assert call(grid(0, [1, 1, 1])) == EINVAL
    assert call(grid(2, [8, 8])) == EUNSUPPORTED                  # 3-D only
    assert call(grid(3, [8, 8, 8]), J=None) == EINVAL
    assert call(grid(3, [8, 8, 8]), xp=None) == EINVAL
    bad = (C.c_void_p * 3)(FAKE, None, FAKE)
    assert call(grid(3, [8, 8, 8]), xp=bad) == EINVAL
    P2 = particles(1000)
    P2.w = None
    assert call(grid(3, [8, 8, 8]), P=P2) == EINVAL
    assert call(grid(3, [8, 8, 8]), P=particles(-1)) == EINVAL
    assert call(grid(3, [8, 8, 8]), P=particles(1 << 31)) == EINVAL
    g = grid(3, [64, 64, 64])
    assert call(g, tile=Tile(8, 2, 1, 0, 1000, FAKE)) == EINVAL  # layout keyed with TSC
    assert b"order" in lib.pcg_last_error()
    assert call(g, tile=Tile(6, 1, 1, 0, 1000, FAKE)) == EINVAL  # 64 % 6
    assert call(g, tile=Tile(8, 1, -1, 0, 1000, FAKE)) == EINVAL  # negative drift
    assert call(g, tile=Tile(8, 1, 1, 0, 1001, FAKE)) == EINVAL  # n_partitioned > count
    assert call(g, tile=Tile(8, 1, 1, 0, 1000, None)) == EINVAL  # no offsets
    assert call(g, tile=Tile(16, 1, 8, 0, 1000, FAKE)) == ELDS   # TE = 35: 35^3*12 B > 160 KiB
    assert call(g, tile=Tile(8, 1, 1 << 30, 0, 1000, FAKE)) == ELDS  # T + 2D + 3 overflows int
    big = grid(3, [2048, 2048, 2048])
    assert call(big, tile=Tile(1, 1, 1, 0, 1000, FAKE)) == EINVAL  # 2^33 tiles: one launch
    # no particles: nothing to check beyond the grid, nothing launched
    assert call(g, P=particles(0), xp=None) == 0


def test_zigzag_regroup_validation(lib):
    lib.pcg_last_error.restype = C.c_char_p
    zr = lib.deposit_currents_zigzag_regroup
    lib.pcg_sort_workspace_bytes.restype = C.c_size_t
    P = particles(1000)
    xp = (C.c_void_p * 3)(FAKE, FAKE, FAKE)
    arrs = (C.c_void_p * 8)(*([FAKE] * 8))
    outs = (C.c_void_p * 8)(*([FAKE + 64] * 8))
    g = grid(3, [64, 64, 64])
    need = lib.pcg_sort_workspace_bytes(C.byref(g), C.c_int64(1000), 8)

    def call(g=g, tile=Tile(8, 1, 0, 0, 1000, FAKE), ws=C.c_void_p(FAKE * 256), wsb=need,
             off=C.c_void_p(FAKE * 2), na=8):
        return zr(C.byref(g), C.byref(P), xp, C.byref(tile) if tile else None, C.c_void_p(FAKE),
                  None, na, arrs, outs, off, ws, C.c_size_t(wsb), None)

    assert call(tile=None) == EINVAL                                # the layout is required
    assert call(g=grid(2, [8, 8])) == EUNSUPPORTED
    assert call(tile=Tile(8, 2, 0, 0, 1000, FAKE)) == EINVAL       # keyed with TSC
    assert call(wsb=need - 1) == EWORKSPACE
    assert call(ws=None) == EWORKSPACE
    assert call(off=None) == EINVAL
    assert call(off=C.c_void_p(FAKE)) == EINVAL                     # same as the layout's
    assert call(na=17) == EINVAL


def test_deposit_workspace_size(lib):
    lib.pcg_deposit_workspace_bytes.restype = C.c_size_t
    g = grid(3, [128, 128, 128])
    t = Tile(8, 1, 1, 0, 0, FAKE)
    assert lib.pcg_deposit_workspace_bytes(C.byref(g), C.byref(t)) >= 4097 * 4
    assert lib.pcg_deposit_workspace_bytes(C.byref(g), None) == 0


def test_regroup_validation(lib):
    lib.pcg_deposit_regroup_workspace_bytes.restype = C.c_size_t
    fr = lib.deposit_currents_regroup
    g = grid(3, [32, 32, 32])
    P = particles(1000)
    arr = (C.c_void_p * 1)(FAKE)
    outs = (C.c_void_p * 1)(FAKE + 4096)
    t = Tile(8, 1, 1, 0, 1000, FAKE)
    need = lib.pcg_deposit_regroup_workspace_bytes(C.byref(g), C.byref(t), C.c_int64(1000))
    assert need >= lib.pcg_sort_workspace_bytes(C.byref(g), C.c_int64(1000), 8)
    assert lib.pcg_deposit_regroup_workspace_bytes(C.byref(g), None, C.c_int64(1000)) == 0

    def call(tile=t, P=P, ws=FAKE, wsb=need, off=FAKE + 8192, J=FAKE, order=1):
        return fr(C.byref(g), C.byref(P), order, C.byref(tile) if tile else None, C.c_void_p(J),
                  None, 1, arr, outs, C.c_void_p(off), C.c_void_p(ws), C.c_size_t(wsb), None)

    assert call(tile=None) == EINVAL                              # needs the current layout
    assert call(wsb=need - 1) == EWORKSPACE
    assert call(ws=FAKE + 8) == EWORKSPACE                        # misaligned
    assert call(J=0) == EINVAL
    assert call(order=3) == EUNSUPPORTED
    assert call(tile=Tile(8, 2, 1, 0, 1000, FAKE)) == EINVAL      # keyed with TSC
    assert call(off=0) == EINVAL                                  # no output offsets
    assert call(off=FAKE) == EINVAL                               # output offsets alias the layout


def test_tile_sort_validation(lib):
    ts = lib.pcg_tile_sort
    g = grid(3, [32, 32, 32])
    kx = (C.c_void_p * 3)(FAKE, FAKE, FAKE)
    arr = (C.c_void_p * 1)(FAKE)
    arr2 = (C.c_void_p * 1)(FAKE + 4096)

    def call(g=g, order=1, T=8, count=100, n_arrays=1, outs=arr2, perm=FAKE, off=FAKE, ws=FAKE,
             wsb=1 << 30, prev=None):
        return ts(C.byref(g), order, T, C.c_int64(count), kx, n_arrays, arr, outs,
                  C.c_void_p(perm), None, C.c_void_p(off), C.byref(prev) if prev else None,
                  C.c_void_p(ws), C.c_size_t(wsb), None)

    assert call(T=0) == EINVAL
    assert call(T=5) == EINVAL
    assert call(order=0) == EUNSUPPORTED
    assert call(count=-5) == EINVAL
    assert call(n_arrays=17) == EINVAL
    assert call(outs=arr) == EINVAL                               # in place
    assert call(off=0) == EINVAL
    assert call(ws=0) == EWORKSPACE
    assert call(wsb=10) == EWORKSPACE
    assert call(ws=FAKE + 8) == EWORKSPACE                        # misaligned
    assert call(prev=Tile(4, 1, 1, 0, 100, FAKE)) == EINVAL       # prev keyed with another T
    assert call(prev=Tile(8, 2, 1, 0, 100, FAKE)) == EINVAL       # or another order
    assert call(prev=Tile(8, 1, 1, 0, 100, None)) == EINVAL       # no offsets
    assert call(prev=Tile(8, 1, 1, 0, 100, FAKE)) == EINVAL       # offsets aliasing the output


def test_mass_and_sweep_validation(lib):
    am = lib.assemble_mass_matrix
    am.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                   C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
    P = particles(100)
    B = (C.c_void_p * 3)(FAKE, FAKE, FAKE)
    g8 = C.byref(grid(3, [8, 8, 8]))

    def call(g=g8, variant=0, cells=None, ws=FAKE, wsb=256):
        return am(g, C.byref(P), B, FAKE, cells, variant, FAKE, ws, wsb, None)

    assert call(g=C.byref(grid(2, [8, 8]))) == EUNSUPPORTED
    assert call(g=C.byref(grid(3, [2, 8, 8]))) == EINVAL
    assert call(variant=9) == EINVAL
    big = particles(1 << 30)
    assert am(g8, C.byref(big), B, FAKE, None, 0, FAKE, FAKE, 256, None) == EINVAL
    assert call(variant=1) == EINVAL                              # MFMA needs cells
    t = Tile(2, 1, 0, 0, 100, FAKE)
    assert call(variant=1, cells=C.byref(t)) == EINVAL            # not a cell layout
    c1 = Tile(1, 1, 0, 0, 100, FAKE)
    assert call(variant=1, cells=C.byref(c1), ws=None) == EWORKSPACE
    assert call(variant=1, cells=C.byref(c1), wsb=8) == EWORKSPACE
    assert call(variant=1, cells=C.byref(c1), ws=FAKE + 8) == EWORKSPACE   # misaligned
    lib.pcg_mass_workspace_bytes.restype = C.c_size_t
    assert lib.pcg_mass_workspace_bytes(g8) >= 4
    # the scalar matrix: the same checks, without B and beta
    sm = lib.assemble_mass_matrix_scalar
    sm.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                   C.c_size_t, C.c_void_p]

    def scall(g=g8, variant=0, cells=None, ws=FAKE, wsb=256, p=P, M=FAKE):
        return sm(g, C.byref(p) if p is not None else None, cells, variant, M, ws, wsb, None)

    assert scall(g=C.byref(grid(2, [8, 8]))) == EUNSUPPORTED
    assert scall(g=C.byref(grid(3, [8, 2, 8]))) == EINVAL
    assert scall(variant=-1) == EINVAL
    assert scall(p=None) == EINVAL
    assert scall(M=None) == EINVAL
    assert scall(p=big) == EINVAL
    nox = particles(100)
    nox.q = None
    assert scall(p=nox) == EINVAL
    assert scall(variant=2) == EINVAL                             # VALU needs cells
    assert scall(variant=1, cells=C.byref(t)) == EINVAL
    assert scall(variant=1, cells=C.byref(c1), ws=None) == EWORKSPACE
    assert scall(variant=1, cells=C.byref(c1), ws=FAKE + 8) == EWORKSPACE
    assert scall(variant=1, cells=C.byref(Tile(1, 1, 0, 0, 101, FAKE))) == EINVAL  # > count
    # the scalar TSC matrix: n_k >= 5, an order-2 cell layout
    tm = lib.assemble_mass_matrix_scalar_tsc
    tm.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]
    assert tm(C.byref(grid(3, [8, 4, 8])), C.byref(P), None, 0, FAKE, None) == EINVAL
    assert tm(C.byref(grid(2, [8, 8])), C.byref(P), None, 0, FAKE, None) == EUNSUPPORTED
    assert tm(g8, C.byref(P), None, 1, FAKE, None) == EINVAL               # MFMA needs groups
    assert tm(g8, C.byref(P), None, 2, FAKE, None) == EINVAL               # VALU too
    assert tm(g8, C.byref(P), C.byref(c1), 1, FAKE, None) == EINVAL        # order 1 layout
    o2 = Tile(1, 2, 0, 0, 100, FAKE)
    assert tm(g8, C.byref(P), C.byref(Tile(1, 2, 0, 0, 101, FAKE)), 1, FAKE, None) == EINVAL
    assert tm(g8, C.byref(P), C.byref(Tile(1, 2, 0, 0, 100, None)), 1, FAKE, None) == EINVAL
    assert tm(g8, C.byref(P), C.byref(o2), 9, FAKE, None) == EINVAL
    assert tm(g8, C.byref(P), C.byref(o2), 1, None, None) == EINVAL       # no M
    assert tm(g8, C.byref(big), C.byref(o2), 1, FAKE, None) == EINVAL
    tt = lib.assemble_mass_matrix_tsc
    tt.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32,
                   C.c_void_p, C.c_void_p]
    assert tt(g8, C.byref(P), None, FAKE, C.byref(o2), 1, FAKE, None) == EINVAL    # no B
    assert tt(g8, C.byref(P), B, None, C.byref(o2), 1, FAKE, None) == EINVAL       # no beta
    assert tt(C.byref(grid(3, [4, 8, 8])), C.byref(P), B, FAKE, None, 0, FAKE, None) == EINVAL
    assert tt(g8, C.byref(P), B, FAKE, C.byref(c1), 1, FAKE, None) == EINVAL       # order 1
    assert tt(g8, C.byref(P), B, FAKE, None, 1, FAKE, None) == EINVAL              # no groups
    # the fp64 entry points validate alike
    af = lib.assemble_mass_matrix_f64
    af.argtypes = am.argtypes
    assert af(g8, C.byref(P), B, FAKE, None, 9, FAKE, FAKE, 256, None) == EINVAL
    assert af(g8, C.byref(P), None, FAKE, None, 0, FAKE, FAKE, 256, None) == EINVAL  # no B
    assert af(g8, C.byref(P), B, FAKE, C.byref(c1), 1, FAKE, None, 0, None) == EWORKSPACE
    sf = lib.assemble_mass_matrix_scalar_f64
    sf.argtypes = sm.argtypes
    assert sf(C.byref(grid(2, [8, 8])), C.byref(P), None, 0, FAKE, FAKE, 256, None) == EUNSUPPORTED
    assert sf(g8, C.byref(P), C.byref(t), 1, FAKE, FAKE, 256, None) == EINVAL
    assert sf(g8, C.byref(P), None, 0, None, FAKE, 256, None) == EINVAL            # no M
    sw = lib.deposit_sweep1d
    sw.argtypes = [C.c_int32, C.c_int64, C.c_void_p, C.c_void_p, C.c_int32, C.c_double,
                   C.c_double, C.c_void_p, C.c_void_p]
    assert sw(0, 10, FAKE, FAKE, 50, 0.02, 0.005, FAKE, None) == EINVAL
    assert sw(1 << 15, 10, FAKE, FAKE, 50, 0.02, 0.005, FAKE, None) == EINVAL
    assert sw(1024, 10, FAKE, FAKE, 50, 0.02, 0.0, FAKE, None) == EINVAL
    assert sw(1024, 10, None, FAKE, 50, 0.02, 0.005, FAKE, None) == EINVAL
    gr = lib.deposit_sweep1d_grad
    gr.argtypes = [C.c_int32, C.c_int64, C.c_void_p, C.c_void_p, C.c_int32, C.c_double,
                   C.c_double, C.c_void_p, C.c_void_p, C.c_void_p]
    assert gr(0, 10, FAKE, FAKE, 50, 0.02, 0.005, FAKE, FAKE, None) == EINVAL
    assert gr(16385, 10, FAKE, FAKE, 50, 0.02, 0.005, FAKE, FAKE, None) == EINVAL
    assert gr(1024, -1, FAKE, FAKE, 50, 0.02, 0.005, FAKE, FAKE, None) == EINVAL
    assert gr(1024, 10, FAKE, FAKE, -1, 0.02, 0.005, FAKE, FAKE, None) == EINVAL
    assert gr(1024, 10, FAKE, FAKE, 50, 0.02, 0.0, FAKE, FAKE, None) == EINVAL
    assert gr(1024, 10, FAKE, FAKE, 50, 0.02, 0.005, None, FAKE, None) == EINVAL   # no dH
    assert gr(1024, 10, FAKE, FAKE, 50, 0.02, 0.005, FAKE, None, None) == EINVAL   # no dx0
    assert gr(1024, 0, None, None, 50, 0.02, 0.005, None, None, None) == 0        # empty
    lg = lib.deposit_sweep1d_loss_grad
    lg.argtypes = [C.c_int32, C.c_int64, C.c_void_p, C.c_void_p, C.c_int32, C.c_double,
                   C.c_double, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
    assert lg(0, 10, FAKE, FAKE, 50, 0.02, 0.005, FAKE, FAKE, FAKE, None) == EINVAL
    assert lg(1024, 10, FAKE, FAKE, 50, 0.02, 0.005, None, FAKE, FAKE, None) == EINVAL  # target
    assert lg(1024, 10, FAKE, FAKE, 50, 0.02, 0.005, FAKE, None, FAKE, None) == EINVAL  # H
    assert lg(1024, 10, FAKE, FAKE, 50, 0.02, 0.005, FAKE, FAKE, None, None) == EINVAL  # dx0


def test_deposit_noalloc_validation(lib):
    """The entry point with a static scratch: a layout whose map exceeds it is
    refused with PCG_EWORKSPACE, and bad arguments with the deposit's codes,
    before any HIP call."""
    lib.pcg_last_error.restype = C.c_char_p
    dn = lib.deposit_currents_noalloc
    P = particles(1000)

    def call(g, order=1, tile=None, J=C.c_void_p(FAKE), P=P):
        return dn(C.byref(g), C.byref(P), order, C.byref(tile) if tile else None, J, None, None)

    big = grid(3, [256, 256, 256])                    # 16.8M cell tiles: a 335 MB map
    assert call(big, tile=Tile(1, 1, 0, 0, 1000, FAKE)) == EWORKSPACE
    assert b"static" in lib.pcg_last_error()
    g = grid(3, [64, 64, 64])
    assert call(g, tile=Tile(8, 1, 1, 0, 1000, FAKE), J=None) == EINVAL
    assert call(g, order=3, tile=Tile(8, 1, 1, 0, 1000, FAKE)) == EUNSUPPORTED
    assert call(g, tile=Tile(8, 1, 1, 0, 1001, FAKE)) == EINVAL     # n_partitioned > count
    assert call(grid(0, [1, 1, 1])) == EINVAL


def test_mass_constants_match_the_header(lib):
    """The binding's PCG_MASS_* values are the header's (the overwrite flag too)."""
    import sys

    sys.path.insert(0, ROOT)
    import particle_cell_grid_amd as pcg

    defs = {m.group(1): int(m.group(2))
            for m in re.finditer(r"#define (PCG_MASS_\w+) (\d+)", open(HEADER).read())}
    assert "PCG_MASS_OVERWRITE" in defs and len(defs) == 5
    for name, value in defs.items():
        assert getattr(pcg, name) == value


def test_mass_overwrite_flag_validation(lib):
    """With the overwrite flag the checks are those without it, all before
    anything is enqueued (M is never touched on an error)."""
    sm = lib.assemble_mass_matrix_scalar
    sm.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                   C.c_size_t, C.c_void_p]
    g8 = C.byref(grid(3, [8, 8, 8]))
    P = particles(100)
    c1 = Tile(1, 1, 0, 0, 100, FAKE)
    OVER = 16
    assert sm(g8, C.byref(P), None, 7 | OVER, FAKE, FAKE, 256, None) == EINVAL
    assert sm(g8, C.byref(P), None, 2 | OVER, FAKE, FAKE, 256, None) == EINVAL   # VALU needs cells
    assert sm(g8, C.byref(P), C.byref(c1), 1 | OVER, FAKE, None, 0, None) == EWORKSPACE
    tm = lib.assemble_mass_matrix_scalar_tsc
    tm.argtypes = [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p]
    assert tm(g8, C.byref(P), None, 1 | OVER, FAKE, None) == EINVAL           # MFMA needs groups
    assert tm(g8, C.byref(P), None, 7 | OVER, FAKE, None) == EINVAL
