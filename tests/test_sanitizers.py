"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds are checked:

* the oracle, ``oracle.c`` built with gcc's sanitizers, running its pins
  (``test_oracle.py``, ``test_row_sums.py``);
* the library's host code, the sanitizer copy of ``libpcg.so`` from
  ``build.py --asan`` (device code built as usual), running the argument
  checks of ``test_abi.py``, which return before anything reaches a GPU.

Each run is a child process with the sanitizer runtime in ``LD_PRELOAD`` and
halts on the first report.  A planted heap overflow in a tiny C library, built
and loaded the same way, shows that each runtime really reports.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "particle_cell_grid_amd", "csrc"))
import build as libbuild  # noqa: E402

SAN_ENV = {
    "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
    "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
}

OVERFLOW_C = r"""
#include <stdlib.h>
int planted_overflow(int n)
{
    volatile int *a = (int *)malloc(sizeof(int) * (size_t)n);
    int s = 0;
    for (int i = 0; i <= n; ++i)   /* one past the end */
        s += a[i] = i;
    free((void *)a);
    return s;
}
"""


def _env(preload, **extra):
    env = dict(os.environ)
    env.update(SAN_ENV)
    env["LD_PRELOAD"] = preload
    env.update(extra)
    return env


def _run(args, env, timeout=600):
    return subprocess.run(args, cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=timeout)


def _planted(tmp_path, cc, flags, preload):
    src = tmp_path / "planted.c"
    src.write_text(OVERFLOW_C)
    so = tmp_path / f"planted_{os.path.basename(cc)}.so"
    subprocess.check_call([cc, "-O1", "-g", "-fPIC", "-shared", *flags, str(src), "-o", str(so)])
    code = f"import ctypes; ctypes.CDLL({str(so)!r}).planted_overflow(8)"
    return _run([sys.executable, "-c", code], _env(preload), timeout=120)


def test_oracle_under_asan(tmp_path):
    import oracle

    gcc_asan = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    r = _planted(tmp_path, "gcc", san, gcc_asan)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]

    lib = tmp_path / "liboracle_asan.so"
    flags = [f for f in oracle.CFLAGS if f != "-O2"] + ["-O1", "-g", *san]
    subprocess.check_call(["gcc", *flags, os.path.join(ROOT, "oracle", "oracle.c"), "-o",
                           str(lib), "-lm"])
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
              "tests/test_oracle.py", "tests/test_row_sums.py"],
             _env(gcc_asan, PCG_ORACLE_LIB=str(lib)))
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr


def test_host_argument_checks_under_asan(tmp_path):
    rt = libbuild.asan_runtime()
    if not os.path.exists(rt):
        pytest.fail(f"hipcc's ASan runtime is missing: {rt}")
    r = _planted(tmp_path, libbuild.host_clang(), ["-fsanitize=address", "-shared-libasan"], rt)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]

    lib = libbuild.build_asan()
    syms = subprocess.check_output(["nm", "-D", lib], text=True)
    assert "__asan_report" in syms  # the host code really is instrumented
    r = _run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
              "tests/test_abi.py"], _env(rt, PCG_LIB=lib))
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr
