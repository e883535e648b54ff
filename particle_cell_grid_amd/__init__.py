"""particle_cell_grid_amd -- particle-to-grid scatter deposition on AMD MI355X.

A thin ctypes binding over the HIP library ``libpcg.so`` (C ABI in
``include/pcg.h``).  Functions carry the C names; they take torch tensors that
live on the GPU, pass their device pointers and the current torch stream, and
raise ``PcgError`` on a non-zero status.  Nothing here computes: every step runs
in the library's kernels.  Importing the package fails loudly if the library
has not been built (run ``particle_cell_grid_amd/csrc/build.py``).
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpcg.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"particle_cell_grid_amd: HIP library {LIB_PATH} is missing; build it with "
        "`python particle_cell_grid_amd/csrc/build.py` (hipcc, gfx950)")

_lib = C.CDLL(LIB_PATH)

PCG_MASS_AUTO, PCG_MASS_MFMA, PCG_MASS_VALU, PCG_MASS_FLAT = 0, 1, 2, 3
PCG_MASS_OVERWRITE = 16  # OR'ed into a variant: M = the matrix, not M += the matrix


class Grid(C.Structure):
    _fields_ = [("dim", C.c_int32), ("n", C.c_int32 * 3)]


class Particles(C.Structure):
    _fields_ = [("count", C.c_int64), ("x", C.c_void_p * 3), ("v", C.c_void_p * 3),
                ("q", C.c_void_p), ("w", C.c_void_p)]


class Tile(C.Structure):
    _fields_ = [("T", C.c_int32), ("order", C.c_int32), ("drift", C.c_int32),
                ("block", C.c_int32), ("n_partitioned", C.c_int64),
                ("tile_offsets", C.c_void_p)]


_P = C.POINTER
_lib.pcg_sort_workspace_bytes.argtypes = [_P(Grid), C.c_int64, C.c_int32]
_lib.pcg_sort_workspace_bytes.restype = C.c_size_t
_lib.pcg_tile_sort.argtypes = [_P(Grid), C.c_int32, C.c_int32, C.c_int64, C.c_void_p, C.c_int32,
                               C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                               C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
_lib.pcg_tile_sort.restype = C.c_int32
_lib.pcg_deposit_workspace_bytes.argtypes = [_P(Grid), _P(Tile)]
_lib.pcg_deposit_workspace_bytes.restype = C.c_size_t
_lib.deposit_currents.argtypes = [_P(Grid), _P(Particles), C.c_int32, _P(Tile), C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
_lib.deposit_currents.restype = C.c_int32
_lib.deposit_currents_noalloc.argtypes = [_P(Grid), _P(Particles), C.c_int32, _P(Tile),
                                          C.c_void_p, C.c_void_p, C.c_void_p]
_lib.deposit_currents_noalloc.restype = C.c_int32
_lib.pcg_deposit_regroup_workspace_bytes.argtypes = [_P(Grid), _P(Tile), C.c_int64]
_lib.pcg_deposit_regroup_workspace_bytes.restype = C.c_size_t
_lib.deposit_currents_regroup.argtypes = [_P(Grid), _P(Particles), C.c_int32, _P(Tile),
                                          C.c_void_p, C.c_void_p, C.c_int32, C.c_void_p,
                                          C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t,
                                          C.c_void_p]
_lib.deposit_currents_regroup.restype = C.c_int32
_lib.deposit_currents_zigzag.argtypes = [_P(Grid), _P(Particles), C.c_void_p, _P(Tile),
                                         C.c_void_p, C.c_void_p, C.c_void_p]
_lib.deposit_currents_zigzag.restype = C.c_int32
_lib.deposit_currents_zigzag_regroup.argtypes = [_P(Grid), _P(Particles), C.c_void_p,
                                                 _P(Tile), C.c_void_p, C.c_void_p, C.c_int32,
                                                 C.c_void_p, C.c_void_p, C.c_void_p,
                                                 C.c_void_p, C.c_size_t, C.c_void_p]
_lib.deposit_currents_zigzag_regroup.restype = C.c_int32
_lib.pcg_mass_workspace_bytes.argtypes = [_P(Grid)]
_lib.pcg_mass_workspace_bytes.restype = C.c_size_t
_lib.assemble_mass_matrix.argtypes = [_P(Grid), _P(Particles), C.c_void_p, C.c_void_p, _P(Tile),
                                      C.c_int32, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
_lib.assemble_mass_matrix.restype = C.c_int32
_lib.assemble_mass_matrix_scalar.argtypes = [_P(Grid), _P(Particles), _P(Tile), C.c_int32,
                                             C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
_lib.assemble_mass_matrix_scalar.restype = C.c_int32
_lib.assemble_mass_matrix_scalar_tsc.argtypes = [_P(Grid), _P(Particles), _P(Tile), C.c_int32,
                                                 C.c_void_p, C.c_void_p]
_lib.assemble_mass_matrix_scalar_tsc.restype = C.c_int32
_lib.assemble_mass_matrix_tsc.argtypes = [_P(Grid), _P(Particles), C.c_void_p, C.c_void_p,
                                          _P(Tile), C.c_int32, C.c_void_p, C.c_void_p]
_lib.assemble_mass_matrix_tsc.restype = C.c_int32
_lib.assemble_mass_matrix_f64.argtypes = _lib.assemble_mass_matrix.argtypes
_lib.assemble_mass_matrix_f64.restype = C.c_int32
_lib.assemble_mass_matrix_scalar_f64.argtypes = _lib.assemble_mass_matrix_scalar.argtypes
_lib.assemble_mass_matrix_scalar_f64.restype = C.c_int32
_lib.deposit_sweep1d.argtypes = [C.c_int32, C.c_int64, C.c_void_p, C.c_void_p, C.c_int32,
                                 C.c_double, C.c_double, C.c_void_p, C.c_void_p]
_lib.deposit_sweep1d.restype = C.c_int32
_lib.deposit_sweep1d_grad.argtypes = [C.c_int32, C.c_int64, C.c_void_p, C.c_void_p, C.c_int32,
                                      C.c_double, C.c_double, C.c_void_p, C.c_void_p,
                                      C.c_void_p]
_lib.deposit_sweep1d_grad.restype = C.c_int32
_lib.deposit_sweep1d_loss_grad.argtypes = [C.c_int32, C.c_int64, C.c_void_p, C.c_void_p,
                                           C.c_int32, C.c_double, C.c_double, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_void_p]
_lib.deposit_sweep1d_loss_grad.restype = C.c_int32
_lib.pcg_status_string.argtypes = [C.c_int32]
_lib.pcg_status_string.restype = C.c_char_p
_lib.pcg_last_error.argtypes = []
_lib.pcg_last_error.restype = C.c_char_p
_lib.pcg_version.argtypes = []
_lib.pcg_version.restype = C.c_char_p
_lib.pcg_timing_enable.argtypes = [C.c_int32]
_lib.pcg_timing_enable.restype = C.c_int32
_lib.pcg_timing_reset.argtypes = []
_lib.pcg_timing_reset.restype = C.c_int32
_lib.pcg_timing_read.argtypes = [C.c_char_p, _P(C.c_double), _P(C.c_int64)]
_lib.pcg_timing_read.restype = C.c_int32
_lib.pcg_timing_names.argtypes = [C.c_char_p, C.c_size_t]
_lib.pcg_timing_names.restype = C.c_int32


class PcgError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.pcg_last_error().decode() or _lib.pcg_status_string(status).decode()
        super().__init__(f"{where}: {_lib.pcg_status_string(status).decode()} ({msg})")


def _check(status: int, where: str):
    if status != 0:
        raise PcgError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_grid(dim: int, n: Sequence[int]) -> Grid:
    n3 = list(n) + [1] * (3 - len(n))
    return Grid(int(dim), (C.c_int32 * 3)(*[int(v) for v in n3]))


def _particles(count, x, v=None, q=None, w=None) -> Particles:
    P = Particles()
    P.count = int(count)
    for k in range(3):
        P.x[k] = x[k].data_ptr() if k < len(x) and x[k] is not None else None
        P.v[k] = v[k].data_ptr() if v is not None else None
    P.q = q.data_ptr() if q is not None else None
    P.w = w.data_ptr() if w is not None else None
    return P


@dataclass
class Layout:
    """A tile layout (pcg_tile): T, the shape order it was keyed with, the halo
    budget `drift`, the work-group size knob `block` (0 = auto), the count of
    tile-sorted particles and the device tile offsets."""

    T: int
    order: int
    tile_offsets: torch.Tensor
    n_partitioned: int
    drift: int = 1
    block: int = 0

    def to_c(self) -> Tile:
        return Tile(int(self.T), int(self.order), int(self.drift), int(self.block),
                    int(self.n_partitioned), self.tile_offsets.data_ptr())


def ntiles(dim: int, n: Sequence[int], T: int) -> int:
    t = 1
    for k in range(dim):
        t *= int(n[k]) // int(T)
    return t


def pcg_sort_workspace_bytes(dim: int, n: Sequence[int], count: int, T: int) -> int:
    g = make_grid(dim, n)
    return int(_lib.pcg_sort_workspace_bytes(C.byref(g), int(count), int(T)))


def pcg_tile_sort(dim: int, n: Sequence[int], order: int, T: int, key_x: List[torch.Tensor],
                  arrays: Sequence[torch.Tensor] = (), outs: Optional[List[torch.Tensor]] = None,
                  perm: Optional[torch.Tensor] = None, sorted_keys: Optional[torch.Tensor] = None,
                  tile_offsets: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, prev: Optional["Layout"] = None,
                  want_keys: bool = True, want_perm: bool = True):
    """Stable tile sort.  Returns (perm, sorted_keys, tile_offsets, outs);
    output tensors are allocated when not given.  `prev` is the layout the
    input is currently grouped by (enables the single-pass path); with
    want_keys=False / want_perm=False (and no tensor given) the sorted keys /
    the permutation are not written."""
    g = make_grid(dim, n)
    count = int(key_x[0].numel())
    dev = key_x[0].device
    if perm is None and want_perm:
        perm = torch.empty(count, dtype=torch.int32, device=dev)
    if sorted_keys is None and want_keys:
        sorted_keys = torch.empty(count, dtype=torch.int32, device=dev)
    if tile_offsets is None:
        tile_offsets = torch.empty(ntiles(dim, n, T) + 1, dtype=torch.int32, device=dev)
    if outs is None:
        outs = [torch.empty_like(a) for a in arrays]
    need = pcg_sort_workspace_bytes(dim, n, count, T)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    kx = (C.c_void_p * 3)(*[key_x[k].data_ptr() if k < len(key_x) else None for k in range(3)])
    na = len(arrays)
    ins = (C.c_void_p * max(na, 1))(*[a.data_ptr() for a in arrays])
    ous = (C.c_void_p * max(na, 1))(*[o.data_ptr() for o in outs])
    pt = prev.to_c() if prev is not None else None
    st = _lib.pcg_tile_sort(C.byref(g), int(order), int(T), count, kx, na, ins, ous,
                            _ptr(perm), _ptr(sorted_keys), _ptr(tile_offsets),
                            C.byref(pt) if pt is not None else None, _ptr(workspace),
                            int(workspace.numel()), _stream())
    _check(st, "pcg_tile_sort")
    return perm, sorted_keys, tile_offsets, outs


def pcg_deposit_workspace_bytes(dim: int, n: Sequence[int], layout: Optional[Layout]) -> int:
    if layout is None:
        return 0
    g = make_grid(dim, n)
    t = layout.to_c()
    return int(_lib.pcg_deposit_workspace_bytes(C.byref(g), C.byref(t)))


def deposit_currents(dim: int, n: Sequence[int], order: int, x: List[torch.Tensor],
                     v: List[torch.Tensor], q: torch.Tensor, w: torch.Tensor, J: torch.Tensor,
                     layout: Optional[Layout] = None, n_escaped: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None):
    """J[3, nz, ny, nx] (fp32) += the order-`order` deposit of q w v."""
    g = make_grid(dim, n)
    P = _particles(q.numel(), x, v, q, w)
    tile = layout.to_c() if layout is not None else None
    need = pcg_deposit_workspace_bytes(dim, n, layout)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = _lib.deposit_currents(C.byref(g), C.byref(P), int(order),
                               C.byref(tile) if tile is not None else None, _ptr(J),
                               _ptr(n_escaped), _ptr(workspace) if need else None,
                               int(workspace.numel()) if need else 0, _stream())
    _check(st, "deposit_currents")
    return J


def deposit_currents_noalloc(dim: int, n: Sequence[int], order: int, x: List[torch.Tensor],
                             v: List[torch.Tensor], q: torch.Tensor, w: torch.Tensor,
                             J: torch.Tensor, layout: Optional[Layout] = None,
                             n_escaped: Optional[torch.Tensor] = None):
    """deposit_currents without a workspace: the library's static scratch."""
    g = make_grid(dim, n)
    P = _particles(q.numel(), x, v, q, w)
    tile = layout.to_c() if layout is not None else None
    st = _lib.deposit_currents_noalloc(C.byref(g), C.byref(P), int(order),
                                       C.byref(tile) if tile is not None else None, _ptr(J),
                                       _ptr(n_escaped), _stream())
    _check(st, "deposit_currents_noalloc")
    return J


def pcg_deposit_regroup_workspace_bytes(dim: int, n: Sequence[int], layout: Layout,
                                        count: int) -> int:
    g = make_grid(dim, n)
    t = layout.to_c()
    return int(_lib.pcg_deposit_regroup_workspace_bytes(C.byref(g), C.byref(t), int(count)))


def deposit_currents_regroup(dim: int, n: Sequence[int], order: int, x: List[torch.Tensor],
                             v: List[torch.Tensor], q: torch.Tensor, w: torch.Tensor,
                             J: torch.Tensor, layout: Layout, arrays: Sequence[torch.Tensor],
                             outs: Optional[List[torch.Tensor]] = None,
                             tile_offsets: Optional[torch.Tensor] = None,
                             n_escaped: Optional[torch.Tensor] = None,
                             workspace: Optional[torch.Tensor] = None):
    """J += the deposit of q w v with `layout`, and `arrays` regrouped by the
    tiles of x into `outs` / `tile_offsets` (the next layout), in one pass.
    Returns (tile_offsets, outs)."""
    g = make_grid(dim, n)
    count = int(q.numel())
    P = _particles(count, x, v, q, w)
    tile = layout.to_c()
    dev = q.device
    if tile_offsets is None:
        tile_offsets = torch.empty(ntiles(dim, n, layout.T) + 1, dtype=torch.int32, device=dev)
    if outs is None:
        outs = [torch.empty_like(a) for a in arrays]
    need = pcg_deposit_regroup_workspace_bytes(dim, n, layout, count)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    na = len(arrays)
    ins = (C.c_void_p * max(na, 1))(*[a.data_ptr() for a in arrays])
    ous = (C.c_void_p * max(na, 1))(*[o.data_ptr() for o in outs])
    st = _lib.deposit_currents_regroup(C.byref(g), C.byref(P), int(order), C.byref(tile), _ptr(J),
                                       _ptr(n_escaped), na, ins, ous, _ptr(tile_offsets),
                                       _ptr(workspace), int(workspace.numel()), _stream())
    _check(st, "deposit_currents_regroup")
    return tile_offsets, outs


def deposit_currents_zigzag(n: Sequence[int], x: List[torch.Tensor], x_prev: List[torch.Tensor],
                            q: torch.Tensor, w: torch.Tensor, J: torch.Tensor,
                            layout: Optional[Layout] = None,
                            n_escaped: Optional[torch.Tensor] = None):
    """J[3, nz, ny, nx] (fp32) += the charge-conserving zigzag current of each
    particle's move from x_prev to x (3-D).  `layout`: an order-1 tile layout
    keyed on x, or None for the flat kernel."""
    g = make_grid(3, n)
    P = _particles(q.numel(), x, None, q, w)
    xp = (C.c_void_p * 3)(*[x_prev[k].data_ptr() for k in range(3)])
    tile = layout.to_c() if layout is not None else None
    st = _lib.deposit_currents_zigzag(C.byref(g), C.byref(P), xp,
                                      C.byref(tile) if tile is not None else None, _ptr(J),
                                      _ptr(n_escaped), _stream())
    _check(st, "deposit_currents_zigzag")
    return J


def deposit_currents_zigzag_regroup(n: Sequence[int], x: List[torch.Tensor],
                                    x_prev: List[torch.Tensor], q: torch.Tensor,
                                    w: torch.Tensor, J: torch.Tensor, layout: Layout,
                                    arrays: Sequence[torch.Tensor],
                                    outs: Optional[List[torch.Tensor]] = None,
                                    tile_offsets: Optional[torch.Tensor] = None,
                                    n_escaped: Optional[torch.Tensor] = None,
                                    workspace: Optional[torch.Tensor] = None):
    """J += the zigzag current of each move from x_prev to x with `layout`, and
    `arrays` regrouped by the tiles of x into `outs` / `tile_offsets` (the next
    layout), in one pass.  Returns (tile_offsets, outs)."""
    g = make_grid(3, n)
    count = int(q.numel())
    P = _particles(count, x, None, q, w)
    xp = (C.c_void_p * 3)(*[x_prev[k].data_ptr() for k in range(3)])
    tile = layout.to_c()
    dev = q.device
    if tile_offsets is None:
        tile_offsets = torch.empty(ntiles(3, n, layout.T) + 1, dtype=torch.int32, device=dev)
    if outs is None:
        outs = [torch.empty_like(a) for a in arrays]
    need = pcg_sort_workspace_bytes(3, n, count, layout.T)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    na = len(arrays)
    ins = (C.c_void_p * max(na, 1))(*[a.data_ptr() for a in arrays])
    ous = (C.c_void_p * max(na, 1))(*[o.data_ptr() for o in outs])
    st = _lib.deposit_currents_zigzag_regroup(C.byref(g), C.byref(P), xp, C.byref(tile), _ptr(J),
                                              _ptr(n_escaped), na, ins, ous, _ptr(tile_offsets),
                                              _ptr(workspace), int(workspace.numel()), _stream())
    _check(st, "deposit_currents_zigzag_regroup")
    return tile_offsets, outs


def pcg_mass_workspace_bytes(n: Sequence[int]) -> int:
    g = make_grid(3, n)
    return int(_lib.pcg_mass_workspace_bytes(C.byref(g)))


def _mass_suffix(M: torch.Tensor) -> str:
    """The entry point for M's dtype: fp32 -> "", fp64 -> "_f64"."""
    if M.dtype == torch.float32:
        return ""
    if M.dtype == torch.float64:
        return "_f64"
    raise TypeError(f"mass matrix: M must be float32 or float64, not {M.dtype}")


def assemble_mass_matrix(n: Sequence[int], x: List[torch.Tensor], B: List[torch.Tensor],
                         beta: torch.Tensor, q: torch.Tensor, w: torch.Tensor, M: torch.Tensor,
                         cells: Optional[Layout] = None, variant: int = PCG_MASS_AUTO,
                         workspace: Optional[torch.Tensor] = None):
    """M[nz, ny, nx, 27, 3, 3] += the ECSIM CIC mass matrix (M = it with
    PCG_MASS_OVERWRITE OR'ed into variant), in M's dtype (fp32, or fp64: the fp64
    entry point).  With a cell layout a workspace of pcg_mass_workspace_bytes()
    is needed; one is taken from torch's allocator when none is given."""
    g = make_grid(3, n)
    P = _particles(q.numel(), x, None, q, w)
    bp = (C.c_void_p * 3)(*[b.data_ptr() for b in B])
    tile = cells.to_c() if cells is not None else None
    if cells is not None and workspace is None:
        workspace = torch.empty(pcg_mass_workspace_bytes(n), dtype=torch.uint8, device=M.device)
    wsb = int(workspace.numel()) if workspace is not None else 0
    fn = "assemble_mass_matrix" + _mass_suffix(M)
    st = getattr(_lib, fn)(C.byref(g), C.byref(P), bp, _ptr(beta),
                           C.byref(tile) if tile is not None else None, int(variant),
                           _ptr(M), _ptr(workspace), wsb, _stream())
    _check(st, fn)
    return M


def assemble_mass_matrix_scalar(n: Sequence[int], x: List[torch.Tensor], q: torch.Tensor,
                                w: torch.Tensor, M: torch.Tensor, cells: Optional[Layout] = None,
                                variant: int = PCG_MASS_AUTO,
                                workspace: Optional[torch.Tensor] = None):
    """M[nz, ny, nx, 27] += the scalar CIC mass matrix (coefficient q w), in M's
    dtype (fp32 or fp64).  Layout, variants and workspace as for
    assemble_mass_matrix."""
    g = make_grid(3, n)
    P = _particles(q.numel(), x, None, q, w)
    tile = cells.to_c() if cells is not None else None
    if cells is not None and workspace is None:
        workspace = torch.empty(pcg_mass_workspace_bytes(n), dtype=torch.uint8, device=M.device)
    wsb = int(workspace.numel()) if workspace is not None else 0
    fn = "assemble_mass_matrix_scalar" + _mass_suffix(M)
    st = getattr(_lib, fn)(C.byref(g), C.byref(P), C.byref(tile) if tile is not None else None,
                           int(variant), _ptr(M), _ptr(workspace), wsb, _stream())
    _check(st, fn)
    return M


def assemble_mass_matrix_scalar_tsc(n: Sequence[int], x: List[torch.Tensor], q: torch.Tensor,
                                    w: torch.Tensor, M: torch.Tensor,
                                    groups: Optional[Layout] = None,
                                    variant: int = PCG_MASS_AUTO):
    """M[nz, ny, nx, 125] (fp32) += the scalar mass matrix with TSC weights.  groups:
    a T = 1, order = 2 layout (particles grouped by support base), or None (flat)."""
    g = make_grid(3, n)
    P = _particles(q.numel(), x, None, q, w)
    tile = groups.to_c() if groups is not None else None
    st = _lib.assemble_mass_matrix_scalar_tsc(C.byref(g), C.byref(P),
                                              C.byref(tile) if tile is not None else None,
                                              int(variant), _ptr(M), _stream())
    _check(st, "assemble_mass_matrix_scalar_tsc")
    return M


def assemble_mass_matrix_tsc(n: Sequence[int], x: List[torch.Tensor], B: List[torch.Tensor],
                             beta: torch.Tensor, q: torch.Tensor, w: torch.Tensor,
                             M: torch.Tensor, groups: Optional[Layout] = None,
                             variant: int = PCG_MASS_AUTO):
    """M[nz, ny, nx, 125, 3, 3] (fp32) += the ECSIM mass matrix with TSC weights.
    groups: a T = 1, order = 2 layout, or None (flat)."""
    g = make_grid(3, n)
    P = _particles(q.numel(), x, None, q, w)
    bp = (C.c_void_p * 3)(*[b.data_ptr() for b in B])
    tile = groups.to_c() if groups is not None else None
    st = _lib.assemble_mass_matrix_tsc(C.byref(g), C.byref(P), bp, _ptr(beta),
                                       C.byref(tile) if tile is not None else None,
                                       int(variant), _ptr(M), _stream())
    _check(st, "assemble_mass_matrix_tsc")
    return M


def deposit_sweep1d(nb: int, x0: torch.Tensor, v: torch.Tensor, steps: int, dt: float,
                    half_width: float, H: torch.Tensor):
    """H[nb] (fp32) = the fused windowed 1-D sweep deposit (overwritten)."""
    st = _lib.deposit_sweep1d(int(nb), int(x0.numel()), _ptr(x0), _ptr(v), int(steps), float(dt),
                              float(half_width), _ptr(H), _stream())
    _check(st, "deposit_sweep1d")
    return H


def deposit_sweep1d_grad(nb: int, x0: torch.Tensor, v: torch.Tensor, steps: int, dt: float,
                         half_width: float, dH: torch.Tensor,
                         dx0: Optional[torch.Tensor] = None):
    """dx0[count] (fp64) = dL/dx0 of the sweep for dL/dH = dH (fp64 [nb]), overwritten."""
    if dx0 is None:
        dx0 = torch.empty_like(x0)
    st = _lib.deposit_sweep1d_grad(int(nb), int(x0.numel()), _ptr(x0), _ptr(v), int(steps),
                                   float(dt), float(half_width), _ptr(dH), _ptr(dx0), _stream())
    _check(st, "deposit_sweep1d_grad")
    return dx0


def deposit_sweep1d_loss_grad(nb: int, x0: torch.Tensor, v: torch.Tensor, steps: int, dt: float,
                              half_width: float, target: torch.Tensor, H: torch.Tensor,
                              dx0: torch.Tensor):
    """Forward sweep into H (fp32 [nb]), then dx0 = dL/dx0 of L = sum (H - target)^2
    (target fp64 [nb], dx0 fp64 [count]); both outputs overwritten."""
    st = _lib.deposit_sweep1d_loss_grad(int(nb), int(x0.numel()), _ptr(x0), _ptr(v), int(steps),
                                        float(dt), float(half_width), _ptr(target), _ptr(H),
                                        _ptr(dx0), _stream())
    _check(st, "deposit_sweep1d_loss_grad")
    return H, dx0


def pcg_timing_enable(enable: bool = True):
    _check(_lib.pcg_timing_enable(1 if enable else 0), "pcg_timing_enable")


def pcg_timing_reset():
    _check(_lib.pcg_timing_reset(), "pcg_timing_reset")


def pcg_timing_read(kernel: str):
    ms = C.c_double()
    n = C.c_int64()
    _check(_lib.pcg_timing_read(kernel.encode(), C.byref(ms), C.byref(n)), "pcg_timing_read")
    return float(ms.value), int(n.value)


def pcg_timing_names() -> List[str]:
    buf = C.create_string_buffer(4096)
    _check(_lib.pcg_timing_names(buf, 4096), "pcg_timing_names")
    s = buf.value.decode()
    return [t for t in s.split(",") if t]


def pcg_version() -> str:
    return _lib.pcg_version().decode()


def pcg_last_error() -> str:
    return _lib.pcg_last_error().decode()


def pcg_status_string(status: int) -> str:
    return _lib.pcg_status_string(int(status)).decode()
