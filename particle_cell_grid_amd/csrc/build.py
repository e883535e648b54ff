"""Build the HIP library libpcg.so for gfx950 (in-tree, next to the package).

Run as a script (``python particle_cell_grid_amd/csrc/build.py``) or call
``build()``; it does not import the package, so it works before anything is
built.  Every .hip source in this directory is compiled to an object (in parallel,
under _build/) and the objects are linked into the shared library.

Flags: -O3, C++17, gfx950 only, and packed-FP32 instruction selection turned
off (``-target-feature -packed-fp32-ops``) so hipcc never emits v_pk_*_f32.

``build_asan()`` (``build.py --asan``) makes a debug copy,
``_build/asan/libpcg_asan.so``, whose HOST code is built with AddressSanitizer
and UndefinedBehaviorSanitizer; the device code is compiled as usual (no GPU
sanitizer).  It is for CPU runs of the argument checks: load it into a process
started with ``asan_runtime()`` in ``LD_PRELOAD``.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpcg.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(HERE, "*.hip")))


# host-only sanitizer flags (each -fsanitize= behind -Xarch_host, so the
# device compile never sees them)
ASAN_HOST = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
    "-Xarch_host", "-g",
]
ASAN_DIR = os.path.join(HERE, "_build", "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libpcg_asan.so")


def _build(out: str, obj_dir: str, extra: list, verbose: bool) -> str:
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", HERE]
    compile_flags = [f for f in FLAGS if f != "-shared"] + extra

    def compile_one(src):
        obj = os.path.join(obj_dir, os.path.basename(src)[:-4] + ".o")
        cmd = [HIPCC, *compile_flags, *inc, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd)
        return obj

    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = out + ".tmp"
    link_extra = ["-shared-libasan"] if extra else []
    cmd = [HIPCC, *FLAGS, *extra, *link_extra, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every .hip source to an object (in parallel), then link libpcg.so."""
    return _build(LIB, os.path.join(HERE, "_build"), [], verbose)


def source_digest() -> str:
    """sha256 over the sources and the public header (names and bytes)."""
    import hashlib

    h = hashlib.sha256()
    for p in sources() + sorted(glob.glob(os.path.join(HERE, "*.hpp"))) + [
            os.path.join(ROOT, "include", "pcg.h"), os.path.abspath(__file__)]:
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def build_asan(verbose: bool = False) -> str:
    """Build (or reuse, when the sources are unchanged) the sanitizer copy."""
    stamp = os.path.join(ASAN_DIR, "digest")
    digest = source_digest()
    if os.path.exists(ASAN_LIB) and os.path.exists(stamp) and open(stamp).read() == digest:
        return ASAN_LIB
    _build(ASAN_LIB, ASAN_DIR, ASAN_HOST, verbose)
    with open(stamp, "w") as f:
        f.write(digest)
    return ASAN_LIB


def host_clang() -> str:
    """The clang that hipcc drives for host code."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "lib", "llvm", "bin",
                         "clang")
    return clang if os.path.exists(clang) else "/opt/rocm/llvm/bin/clang"


def asan_runtime() -> str:
    """The ASan runtime of hipcc's host compiler, for LD_PRELOAD."""
    return subprocess.check_output(
        [host_clang(), "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()


if __name__ == "__main__":
    if "--asan" in sys.argv:
        print(build_asan(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
