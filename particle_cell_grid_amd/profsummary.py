"""Short text summaries of rocprofv3 output, for the committed profile records.

    python -m particle_cell_grid_amd.profsummary trace   <dir> <out.md> <title> <command>
    python -m particle_cell_grid_amd.profsummary traffic <fetch dir> <write dir> <out.md>
        <workload> <fetch command> <write command> <traffic.json>
    python -m particle_cell_grid_amd.profsummary counters <dir> <out.md> <title> <command>

`trace` tabulates a `--kernel-trace --stats` run.  `traffic` turns one
FETCH_SIZE and one WRITE_SIZE pass into HBM bytes per dispatch, scaled by what
the same counters read for the 1 GiB device copy the benchmark times (a kernel
whose bytes are known), and records them with a digest of the kernel's sources
so that a later change of the kernel voids them.  `counters` tabulates any other
`--pmc` pass (median per dispatch).
"""
import collections
import csv
import glob
import hashlib
import json
import os
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
KERNEL_SOURCES = {"deposit": "deposit.hip", "sort": "sort.hip", "mass": "mass.hip",
                  "mass_tsc": "mass_tsc.hip", "sweep": "sweep.hip", "zigzag": "zigzag.hip"}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30          # the benchmark's context copy: 2^28 fp32 read and written


def source_digest(kernel):
    """sha1 over the file that holds `kernel` (named <file>_<what>) and the
    headers every kernel file includes."""
    h = hashlib.sha1()
    # the longest source key the name starts with (mass_tsc_* before mass_*)
    key = max((k for k in KERNEL_SOURCES if kernel.startswith(k)), key=len)
    for f in (KERNEL_SOURCES[key], "common.hpp", "layout.hpp", "regroup.hpp"):
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def short(name):
    """Kernel symbol -> readable name, e.g. pcg::(anonymous namespace)::k_inc_move<3>."""
    name = name.replace("pcg::(anonymous namespace)::", "").replace("void ", "")
    depth, out = 0, []
    for ch in name:                 # drop the parameter list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


def tap_name(kernel):
    """The library's launch names for its kernels (as the benchmark reports them).
    Template arguments tell apart launches of one kernel template: the tiled
    deposit with its regroup flag set is `deposit_regroup`, the column mass
    kernel on matrix cores is `mass_mfma` (`mass_scalar_mfma` for the scalar
    matrix)."""
    base = kernel.split("<")[0]
    targs = kernel[len(base) + 1:-1].split(",") if "<" in kernel else []
    last = targs[-1].strip() if targs else ""
    if base == "k_deposit_tiled":
        return "deposit_regroup" if last == "true" else "deposit_tiled"
    if base == "k_mass_tsc_brick":
        return "mass_tsc_tensor_mfma" if last == "true" else "mass_tsc_mfma"
    if base == "k_zigzag_tiled":
        # <fixed point, window edge>
        return "zigzag_tiled" if targs and targs[0].strip() == "true" else "zigzag_tiled_f32"
    if base in ("k_mass_tsc_flat", "k_mass_tsc_tensor_flat"):
        return base[2:]
    if base.startswith("k_mass_") and targs:
        # <MFMA, scalar, real> for the column kernel, <scalar, real> otherwise
        scalar = "mass_scalar_" if targs[-2].strip() == "true" else "mass_"
        f64 = "_f64" if last == "double" else ""
        if base == "k_mass_column":
            return scalar + ("mfma" if targs[0].strip() == "true" else "valu") + f64
        if base in ("k_mass_flat", "k_mass_strays"):
            return scalar + base[len("k_mass_"):] + f64
    table = {"k_deposit_flat": "deposit_flat",
             "k_inc_move": "sort_inc_move", "k_inc_count": "sort_inc_count",
             "k_inc_tiles": "sort_inc_tiles",
             "k_permute": "sort_permute", "k_tile_keys": "sort_keys",
             "k_sweep1d": "sweep1d", "k_sweep1d_grad": "sweep1d_grad",
             "k_zigzag_tiled": "zigzag_tiled", "k_zigzag_flat": "zigzag_flat",
             "k_zigzag_regroup": "zigzag_regroup", "k_mass_tsc_valu": "mass_tsc_valu",
             "k_mass_tsc_tensor_valu": "mass_tsc_tensor_valu"}
    return table.get(base)


def one(pattern):
    f = glob.glob(pattern, recursive=True)
    if not f:
        sys.exit(f"profsummary: nothing matches {pattern}")
    return f[0]


def trace(d, out, title, command):
    rows = list(csv.DictReader(open(one(os.path.join(d, "**", "*kernel_stats.csv")))))
    lines = [f"# {title}", "", "Command (from the repository root, one MI355X):", "", "```",
             command, "```", "",
             "rocprofv3 `--stats` over every dispatch of the run (set-up sort, warm-up, timed "
             "steps and the extra timings the benchmark makes).", "",
             "| kernel | calls | average us | min us | max us | % of GPU time |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.1f} |")
    open(out, "w").write("\n".join(lines) + "\n")


def per_dispatch(d, counter):
    out = collections.defaultdict(list)
    for r in csv.DictReader(open(one(os.path.join(d, "**", "*counter_collection.csv")))):
        if r["Counter_Name"] == counter:
            out[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return out


def median(v):
    v = sorted(v)
    return v[len(v) // 2]


def calibration_reading(values):
    """The counter's reading for the 1 GiB copy: the median over the copy
    dispatches of at least half the largest one (a workload may also run small
    copies of its own through the same copy kernel)."""
    top = max(values)
    return median([v for v in values if v >= 0.5 * top])


def traffic(fetch_dir, write_dir, out, workload, cmd_fetch, cmd_write, json_path):
    fe = per_dispatch(fetch_dir, "FETCH_SIZE")
    wr = per_dispatch(write_dir, "WRITE_SIZE")
    if COPY_KERNEL not in fe or COPY_KERNEL not in wr:
        sys.exit("profsummary: the copy kernel is missing from a pass; no calibration")
    kib = COPY_BYTES / 1024
    ffac = kib / calibration_reading(fe[COPY_KERNEL])
    wfac = kib / calibration_reading(wr[COPY_KERNEL])
    lines = [f"# HBM traffic per dispatch: {workload}", "", "Commands (from the repository root, "
             "one MI355X; one counter per pass):", "", "```", cmd_fetch, cmd_write, "```", "",
             f"Calibration: the 1 GiB device copy (`{COPY_KERNEL}`, {kib:,.0f} KiB read and "
             f"{kib:,.0f} KiB written) reads FETCH_SIZE = {calibration_reading(fe[COPY_KERNEL]):,.0f} "
             f"KiB and WRITE_SIZE = {calibration_reading(wr[COPY_KERNEL]):,.0f} KiB per dispatch, "
             f"so the counters "
             f"are scaled by {ffac:.3f} (fetch) and {wfac:.3f} (write).", "",
             "Median over the dispatches of each kernel:", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | "
             "write MB (scaled) |", "|---|---:|---:|---:|---:|---:|"]
    try:
        rec = json.load(open(json_path))
    except (OSError, ValueError):
        rec = {}
    rec.setdefault("note", "HBM bytes per dispatch from rocprofv3 FETCH_SIZE/WRITE_SIZE, "
                           "scaled by the 1 GiB copy calibration; source_sha1 digests the "
                           "kernel's sources at the time the counters were taken")
    kern = rec.setdefault("kernels", {})[workload] = {}  # this pass replaces the workload's record
    for n in sorted(fe):
        if n == COPY_KERNEL:
            continue
        f, w = median(fe[n]), median(wr.get(n, [0.0]))
        lines.append(f"| `{n}` | {len(fe[n])} | {f:,.0f} | {w:,.0f} | {f * ffac * 1024 / 1e6:,.1f} | "
                     f"{w * wfac * 1024 / 1e6:,.1f} |")
        tn = tap_name(n)
        if tn:
            kern[tn] = dict(read_bytes=round(f * ffac * 1024), write_bytes=round(w * wfac * 1024),
                            fetch_kib=f, write_kib=w, source_sha1=source_digest(tn))
    rec["calibration"] = dict(fetch_factor=round(ffac, 4), write_factor=round(wfac, 4))
    open(out, "w").write("\n".join(lines) + "\n")
    json.dump(rec, open(json_path, "w"), indent=1, sort_keys=True)
    open(json_path, "a").write("\n")


def counters(d, out, title, command):
    by = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(one(os.path.join(d, "**", "*counter_collection.csv")))):
        by[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    cols = sorted({c for k in by.values() for c in k})
    lines = [f"# {title}", "", "Command (from the repository root, one MI355X):", "", "```",
             command, "```", "", "Median per dispatch, summed over the chip.", "",
             "| kernel | dispatches | " + " | ".join(cols) + " |", "|---|---:|" + "---:|" * len(cols)]
    for n in sorted(by):
        if n == COPY_KERNEL or "elementwise" in n or "reduce_kernel" in n:
            continue
        ncall = max(len(v) for v in by[n].values())
        lines.append(f"| `{n}` | {ncall} | " +
                     " | ".join(f"{median(by[n][c]):,.0f}" if c in by[n] else "" for c in cols) + " |")
    open(out, "w").write("\n".join(lines) + "\n")


def main(argv):
    if not argv:
        sys.exit(__doc__)
    cmd, rest = argv[0], argv[1:]
    {"trace": trace, "traffic": traffic, "counters": counters}[cmd](*rest)


if __name__ == "__main__":
    main(sys.argv[1:])
