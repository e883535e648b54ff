"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/oracle.c (on the CPU, in a
temporary directory), builds it, and runs the pin suite tests/test_oracle.py
against that build through PCG_ORACLE_LIB.  The suite must fail for every
mutant: a dropped term, a wrong sign, a swapped index or an off-by-one in the
oracle would otherwise go unnoticed and the GPU parity tests would check the
kernels against a wrong reference.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (what the mistake is, text in oracle.c, replacement)
MUTANTS = [
    ("TSC tie at 1/2 sent to the lower base",
     "(x - j) < 0.5", "(x - j) <= 0.5"),
    ("TSC outer weight not squared",
     "return 0.5 * (1.5 - a) * (1.5 - a);", "return 0.5 * (1.5 - a);"),
    ("TSC centre weight off by a constant",
     "return 0.75 - a * a;", "return 0.7 - a * a;"),
    ("deposit drops the charge",
     "J[c * ng + g] += qw * (double)v[c][p] * wt;",
     "J[c * ng + g] += (double)w[p] * (double)v[c][p] * wt;"),
    ("deposit swaps y and z node weights",
     "double wt = W[0][ax] * W[1][ay] * W[2][az];",
     "double wt = W[0][ax] * W[1][az] * W[2][ay];"),
    ("tile key without the periodic wrap",
     "t[k] = wrap(support_base(order, (double)x[k][p]), n[k]) / T;",
     "t[k] = support_base(order, (double)x[k][p]) / T;"),
    ("sort is not stable (ties in reverse)",
     "perm[count[key[p]]++] = (uint32_t)p;", "perm[--count[key[p] + 1]] = (uint32_t)p;"),
    ("escape window without the low drift",
     "if (wrap(origin - D + s0 - b, n[k]) == 0)", "if (wrap(origin + s0 - b, n[k]) == 0)"),
    ("escape window one node wider",
     "const int64_t TE = T + order + 2 * D;", "const int64_t TE = T + order + 2 * D + 1;"),
    ("alpha with the wrong sign of the rotation",
     "- C[i][j] + omega[i] * omega[j]", "+ C[i][j] + omega[i] * omega[j]"),
    ("alpha without the omega omega^T term",
     "- C[i][j] + omega[i] * omega[j]", "- C[i][j]"),
    ("mass-matrix offset with x and y swapped",
     "int o = (bx - ax + 1) + 3 * (by - ay + 1)", "int o = (by - ay + 1) + 3 * (bx - ax + 1)"),
    ("mass matrix scaled by W_a only",
     "double wab = wa * wb;", "double wab = wa;"),
    ("sweep taper not squared",
     "double weight = u * u;", "double weight = u;"),
    ("sweep upper bin gets the lower share",
     "H[wrap(j + 1, nb)] += weight * f;", "H[wrap(j + 1, nb)] += weight * (1.0 - f);"),
    ("sweep distance without the minimum image",
     "double d = r - rint(r);", "double d = r;"),
    ("sweep taper over the full width",
     "double u = 1.0 - fabs(d) / hw;", "double u = 1.0 - fabs(d) / (2.0 * hw);"),
    ("sweep bins without the half-bin shift",
     "double g = x * (double)nb - 0.5;", "double g = x * (double)nb;"),
    ("sweep gradient drops the bin-position term",
     " + weight * (double)nb * (h1 - h0);", ";"),
    ("sweep gradient with the taper slope's sign flipped",
     "double dw = -2.0 * u * sgn / hw;", "double dw = 2.0 * u * sgn / hw;"),
    ("sweep gradient reads the two bins swapped",
     "double h0 = dH[wrap(j, nb)], h1 = dH[wrap(j + 1, nb)];",
     "double h0 = dH[wrap(j + 1, nb)], h1 = dH[wrap(j, nb)];"),
    ("scalar mass matrix without the weight",
     "const double s = (double)q[p] * (double)w[p];", "const double s = (double)q[p];"),
    ("scalar mass matrix weighted by the first node twice",
     "M[g * 27 + o] += s * wg * wh;", "M[g * 27 + o] += s * wg * wg;"),
    ("TSC scalar mass matrix with the z offset reversed",
     "25 * (bz - az + 2)", "25 * (az - bz + 2)"),
    ("TSC scalar mass matrix without the second node's weight",
     "M[g * 125 + o] += s * wg * wh;", "M[g * 125 + o] += s * wg;"),
    ("TSC tensor mass matrix with the first node's z taken from its y digit",
     "int ax = a % 3, ay = (a / 3) % 3, az = a / 9;",
     "int ax = a % 3, ay = (a / 3) % 3, az = (a / 3) % 3;"),
    ("zigzag deposit without the straight-segment cross term",
     "const double wt = w1 * w2 + (d1 == d2 ? cross : -cross);", "const double wt = w1 * w2;"),
    ("zigzag relay point from the lower bound twice",
     "xr[k] = fmin(lo, fmax(hi, 0.5 * (a[k] + b[k])));",
     "xr[k] = fmin(lo, fmax(lo - 1.0, 0.5 * (a[k] + b[k])));"),
    ("TSC tensor mass matrix without the node weights' product",
     "row[ij] += s[ij] * (wa * wb);", "row[ij] += s[ij] * wa;"),
]


def _run_mutant(case, tmpdir):
    name, old, new = case
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    tag = str(abs(hash(name)))
    csrc = os.path.join(tmpdir, f"mutant_{tag}.c")
    so = os.path.join(tmpdir, f"mutant_{tag}.so")
    open(csrc, "w").write(src.replace(old, new, 1))
    sys.path.insert(0, ROOT)
    import oracle

    subprocess.check_call(["gcc", *oracle.CFLAGS, csrc, "-o", so, "-lm"])
    env = dict(os.environ, PCG_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                        "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return name, r.returncode, r.stdout[-400:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda c: _run_mutant(c, str(tmp_path)), MUTANTS))
    survived = [(name, out) for name, rc, out in results if rc == 0]
    assert not survived, "mutants the pins did not catch: " + "; ".join(n for n, _ in survived)
    # a failing collection would also give rc != 0: each mutant must fail a test
    for name, rc, out in results:
        assert rc == 1, f"{name}: pytest exit {rc} (expected test failures): {out}"


def test_unmutated_copy_passes(tmp_path):
    """The harness itself: the same build of an unchanged copy passes the pins."""
    name, rc, out = _run_mutant(("unchanged", "#include <math.h>", "#include <math.h>"),
                                str(tmp_path))
    assert rc == 0, out
