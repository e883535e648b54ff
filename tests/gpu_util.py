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
