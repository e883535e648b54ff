"""Benchmark of the particle-to-grid deposition hot path on one MI355X.

Default (the headline): 3-D CIC current deposit on a 128^3 periodic grid with
32 particles per cell (67,108,864 particles), tile edge 8, drift 1, 2% of the
particles pushed 2-4 cells so the escape valve runs.  One "step" is one pass of
the whole path over that batch, as a PIC step runs it:
    zero J; deposit_currents(pushed particles, previous layout) -> J;
    pcg_tile_sort(pushed particles) -> new layout + permuted SoA arrays.
Inputs are resident in HBM before timing starts; W warm-up steps, then K timed
steps between a device synchronisation on each side (HIP events on the
library's stream).  Per-kernel durations come from the library's event tap
(events recorded around every launch, on the launch stream) during the same
timed steps.

Other workloads (--workload): cic2d_512_ppc16 (2-D CIC 512^2), tsc3d_128_blob
(3-D TSC clustered, T from --tile), mass_64_ppc64 (ECSIM mass matrix 64^3: cell
sort + MFMA assembly), mass_f64_64_ppc64 (the same in fp64), mass_scalar_64_ppc64
(the scalar mass matrix, coefficient q w, on the same particles), sweep1d_2000
(1-D windowed sweep), mass_tsc_scalar_64_ppc64 (the scalar matrix with TSC
weights, support-group sort + MFMA assembly), mass_tsc_64_ppc64 (the ECSIM
matrix with TSC weights), sweep1d_grad_1e7 (the sweep's loss gradient, 10^7 particles:
forward sweep, seed and reverse gather in one library call), zigzag3d_128_ppc32
(the charge-conserving zigzag deposit of the cic3d particles moved by their
velocities, with the incremental tile sort).

Prints ONE JSON line (rank 0).  Only one GPU is used: --gpus above 1 exits.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix
MFMA_FP64_PEAK_TFLOPS = 78.6   # MI355X dense fp64 matrix

# HBM bytes per dispatch measured by rocprofv3 FETCH_SIZE / WRITE_SIZE passes
# (scaled by the copy calibration), with the digest of the kernel's sources at
# the time the counters were taken.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")

METRIC = "deposited particles/s (3D CIC 128^3, 32 ppc) + % of HBM roofline"
HEADLINE = "cic3d_128_ppc32"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=HEADLINE,
                    choices=["sweep1d_2000", "cic2d_512_ppc16", "cic3d_128_ppc32",
                             "tsc3d_128_blob", "mass_64_ppc64", "mass_f64_64_ppc64",
                             "mass_scalar_64_ppc64", "mass_tsc_scalar_64_ppc64",
                             "mass_tsc_64_ppc64",
                             "sweep1d_grad_1e7", "zigzag3d_128_ppc32"])
    ap.add_argument("--tile", type=int, default=0, help="tile edge T (0 = the workload's)")
    ap.add_argument("--block", type=int, default=0)
    ap.add_argument("--drift", type=int, default=-1,
                    help="zigzag workload: the layout's drift D (-1 = the workload's)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-flat", action="store_true", help="skip the flat-path comparison")
    ap.add_argument("--no-copy-bandwidth", action="store_true",
                    help="skip the 1 GiB device copy timed for context (its dispatches "
                         "also calibrate the HBM traffic counters)")
    return ap.parse_args()


# ----------------------------------------------------------------- helpers

def progress(msg):
    """One progress line on stderr (the JSON result line is the only stdout)."""
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def kernel_times(pcg, names):
    out = {}
    for nm in names:
        ms, n = pcg.pcg_timing_read(nm)
        if n:
            out[nm] = dict(total_ms=ms, launches=n, avg_us=1000.0 * ms / n)
    return out


EVICT_BYTES = 1 << 30  # written before each rep of the cold-cache protocol


def time_steps(torch, pcg, step, steps, warmup):
    """K timed steps, back to back, twice.  The first, uninstrumented, gives ms
    per step and the wall time; the second repeats the same K steps with the
    library's per-launch HIP events (recorded on the launch stream) for each
    kernel's duration.  The events add gaps between launches, so they stay out
    of the step time."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    pcg.pcg_timing_reset()
    pcg.pcg_timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    pcg.pcg_timing_enable(False)
    kt = kernel_times(pcg, pcg.pcg_timing_names())
    return ms, wall, kt


def time_cold(torch, fn, reps, evict):
    """The cold-cache protocol: before every rep, outside its timed region, a
    write of `evict` (1 GiB) flushes the L2s and the Infinity Cache of
    everything the previous rep left; each rep is timed alone with events on
    the current stream.  Returns dict(median, min, p90, reps) in ms."""
    import numpy as np

    times = []
    for i in range(reps):
        evict.fill_(i & 255)
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record()
        fn()
        ev1.record()
        torch.cuda.synchronize()
        times.append(ev0.elapsed_time(ev1))
    t = np.asarray(times)
    return dict(median=round(float(np.median(t)), 4), min=round(float(t.min()), 4),
                p90=round(float(np.percentile(t, 90)), 4), reps=reps,
                evict_bytes=int(evict.numel()))


def time_plain(torch, fn, reps):
    """Average ms of fn over reps (events on the current stream, after one warm-up)."""
    fn()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        fn()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / reps


def measured_traffic(kernel, workload):
    """Scaled HBM bytes (read + write) per dispatch from the committed counter
    summary, or None when there is none for this kernel and workload or the
    kernel's sources changed since the counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))["kernels"][workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    from particle_cell_grid_amd.profsummary import source_digest

    if rec.get("source_sha1") != source_digest(kernel):
        return None
    return int(rec["read_bytes"] + rec["write_bytes"])


def roofline_entry(kt, name, bytes_per_launch=None, flops_per_launch=None,
                   mfma_peak=MFMA_FP32_PEAK_TFLOPS):
    k = kt.get(name)
    if not k:
        return None
    sec = k["avg_us"] * 1e-6
    if flops_per_launch is not None:
        achieved = flops_per_launch / sec / 1e12
        return dict(bound="mfma", achieved=round(achieved, 3), peak=mfma_peak,
                    unit="TFLOP/s", frac=round(achieved / mfma_peak, 4),
                    traffic=None, kernel=name, avg_us=round(k["avg_us"], 2))
    achieved = bytes_per_launch / sec / 1e9
    return dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                frac=round(achieved / HBM_PEAK_GBS, 4), traffic=None, kernel=name,
                avg_us=round(k["avg_us"], 2))


# Launches of the general sort path.  When a step re-sorts from the previous
# layout, the library enqueues them behind the incremental path and they
# return at once unless a device flag hands them the work (a particle moved
# further than a tile, or the layout was not a partition).
GENERAL_SORT = ("sort_keys", "sort_hist", "sort_scatter", "sort_scan_reduce",
                "sort_scan_partials", "sort_scan_down", "sort_offsets", "sort_permute",
                "radix_hist", "radix_scatter", "radix_scan", "radix_offsets", "radix_permute")


def kernel_table(kt, steps, alg, gated=False):
    """Per-kernel entries of the timed steps: average duration and launches per
    step, and for a kernel that does the step's work its algorithmic bytes and
    their rate.  With gated=True the general sort's launches are marked as
    such and carry no bytes (they moved none)."""
    out = {}
    for nm, kk in kt.items():
        e = dict(avg_us=round(kk["avg_us"], 2), launches_per_step=kk["launches"] / steps)
        if gated and nm in GENERAL_SORT:
            e["gated"] = ("general-sort fallback enqueued behind the incremental sort; returns "
                          "at once unless the device flag is raised")
        elif nm in alg:
            e["alg_bytes"] = alg[nm]
            e["GBps"] = round(alg[nm] / (kk["avg_us"] * 1e-6) / 1e9, 1)
        out[nm] = e
    return out


def cpu_baseline(single, parallel_fn, nthreads, unit):
    """The cpu_baseline object: the oracle on every host core it may use (the
    reported figure), with the single-thread figure beside it.  single and the
    result of parallel_fn are (items, seconds, sample)."""
    from oracle import parallel

    items, sec, sample = parallel_fn()
    s_items, s_sec, s_sample = single
    return dict(value=round(items / sec, 1), unit=unit, cores=nthreads, kind="oracle",
                sample=sample, cpu_model=parallel.cpu_model(),
                affinity_cores=parallel.host_cores(),
                single_thread=dict(value=round(s_items / s_sec, 1), cores=1, sample=s_sample))


def cpu_baseline_deposit(wl, order, T, target_s):
    """The fp64 oracle as it stands on a bounded prefix sample of the same
    particles, its tile sort (keys + stable counting sort) and deposit: on one
    thread, and on every host core (per-thread ranges, private J added in
    thread order)."""
    import oracle
    from oracle import parallel

    def run(m):
        x = [a[:m] for a in wl.x_next]
        t0 = time.perf_counter()
        oracle.tile_sort(wl.dim, wl.n, order, T, x)
        oracle.deposit(wl.dim, wl.n, order, x, [v[:m] for v in wl.v], wl.q[:m], wl.w[:m])
        return time.perf_counter() - t0

    cal = min(wl.count, 1 << 20)
    per = run(cal) / cal
    m = int(min(wl.count, max(cal, target_s / per)))
    sec = run(m)
    single = (m, sec, f"first {m} of {wl.count} particles of the step input: oracle tile sort "
                      f"(keys + stable counting sort) + fp64 deposit, {sec:.1f} s, 1 thread")
    nth = parallel.thread_count(3 * 8 * wl.n[0] * wl.n[1] * wl.n[2])

    def run_par():
        t0 = time.perf_counter()
        parallel.deposit_step(wl.dim, wl.n, order, T, wl.x_next, wl.v, wl.q, wl.w, nth)
        sec = time.perf_counter() - t0
        return wl.count, sec, (f"all {wl.count} particles of the step input: oracle tile sort + "
                               f"fp64 deposit on {nth} threads (per-thread ranges, private fp64 "
                               f"J added in thread order), {sec:.1f} s")

    return cpu_baseline(single, run_par, nth, "particles/s")


# ----------------------------------------------------------------- deposit family

def bench_deposit(args, torch, pcg, name):
    import numpy as np

    import synthetic

    info = synthetic.WORKLOADS[name]
    order = info["order"]
    T = args.tile or (info.get("T") or 8)
    D = info["D"]
    progress(f"generating {name}")
    wl = synthetic.workload(name)
    n, dim, cnt = wl.n, wl.dim, wl.count
    progress(f"{cnt} particles generated; set-up sort")
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    # previous step's state: sorted on x, pushed to x_next (library sort, untimed)
    x0 = [t(a) for a in wl.x]
    arrays = [t(a) for a in wl.x_next] + [t(a) for a in wl.v] + [t(wl.q), t(wl.w)]
    _, _, off0, cur = pcg.pcg_tile_sort(dim, n, order, T, x0, arrays)
    del x0, arrays
    torch.cuda.synchronize()
    nt = pcg.ntiles(dim, n, T)
    J = torch.zeros(3, n[2], n[1], n[0], dtype=torch.float32, device=dev)
    esc = torch.zeros(1, dtype=torch.int64, device=dev)
    lay = pcg.Layout(T=T, order=order, tile_offsets=off0, n_partitioned=cnt, drift=D,
                     block=args.block)
    dws = torch.empty(max(pcg.pcg_deposit_workspace_bytes(dim, n, lay), 256), dtype=torch.uint8,
                      device=dev)
    # sort outputs (the next step's state), preallocated
    perm = torch.empty(cnt, dtype=torch.int32, device=dev)
    keys = torch.empty(cnt, dtype=torch.int32, device=dev)
    off1 = torch.empty(nt + 1, dtype=torch.int32, device=dev)
    nxt = [torch.empty_like(a) for a in cur]
    sws = torch.empty(pcg.pcg_sort_workspace_bytes(dim, n, cnt, T), dtype=torch.uint8, device=dev)
    rws = torch.empty(pcg.pcg_deposit_regroup_workspace_bytes(dim, n, lay, cnt), dtype=torch.uint8,
                      device=dev)
    xs, vs, q, w = cur[:dim], cur[dim:dim + 3], cur[dim + 3], cur[dim + 4]

    def deposit():
        pcg.deposit_currents(dim, n, order, xs, vs, q, w, J, lay, esc, dws)

    def resort():
        # the pushed particles are grouped by the previous layout: re-sort from it
        pcg.pcg_tile_sort(dim, n, order, T, xs, cur, outs=nxt, want_perm=False,
                          want_keys=False, tile_offsets=off1, workspace=sws, prev=lay)

    def step():
        # deposit with the layout the particles are grouped by, and regroup them
        # by their pushed positions (the next step's layout), in one pass
        J.zero_()
        pcg.deposit_currents_regroup(dim, n, order, xs, vs, q, w, J, lay, cur, outs=nxt,
                                     tile_offsets=off1, workspace=rws)

    progress("timing steps")
    ms, wall, kt = time_steps(torch, pcg, step, args.steps, args.warmup)
    progress(f"{ms:.4f} ms per step")
    # escape count of one deposit of this input
    esc.zero_()
    deposit()
    torch.cuda.synchronize()
    n_esc = int(esc.item())

    # algorithmic bytes per launch (SoA fp32 fields the kernel must move)
    jbytes = 3 * n[0] * n[1] * n[2] * 4
    pbytes = (dim + 5) * 4
    alg = {
        # particle fields read once + J read-modify-write
        "deposit_tiled": cnt * pbytes + 2 * jbytes,
        # the same, plus every field written once to its new slot
        "deposit_regroup": cnt * 2 * pbytes + 2 * jbytes,
        # positions read (per-chunk direction counts are negligible)
        "sort_inc_count": cnt * dim * 4,
        # every field read once and written once
        "sort_inc_move": cnt * 2 * pbytes,
        "sort_keys": cnt * (dim * 4 + 4),
        "sort_permute": cnt * (4 + 2 * pbytes),
        "sort_offsets": cnt * 4 + (nt + 1) * 4,
    }
    # the step re-sorts from the previous layout: the general sort's launches
    # are the gated fallback
    kernels = kernel_table(kt, args.steps, alg, gated=True)
    dominant = max(kt, key=lambda nm: kt[nm]["total_ms"])
    roof_dom = (roofline_entry(kt, dominant, bytes_per_launch=alg[dominant])
                if dominant in alg else None)

    extra = {}
    progress("timing the step with cold caches")
    evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    extra["cold_step_ms"] = time_cold(torch, step, args.steps, evict)
    extra["cold_deposit_ms"] = time_cold(torch, lambda: (J.zero_(), deposit()), args.steps, evict)
    del evict
    # the deposit alone (deposit_currents on the same input), with its own tap
    progress("timing the deposit alone")
    dep_ms, _, kt_dep = time_steps(torch, pcg, lambda: (J.zero_(), deposit()), args.steps, 1)
    roof = roofline_entry(kt_dep, "deposit_tiled", bytes_per_launch=alg["deposit_tiled"])
    # traffic records are kept per tile size for the blob (its T is swept)
    tkey = f"{name}_T{T}" if name == "tsc3d_128_blob" else name
    for r in (roof, roof_dom):
        if r:
            r["traffic"] = measured_traffic(r["kernel"], tkey)
    extra["deposit_only_particles_per_s"] = round(cnt / (dep_ms * 1e-3), 1)
    extra["deposit_only_ms"] = round(dep_ms, 4)
    if not args.no_flat:
        def flat():
            J.zero_()
            pcg.deposit_currents(dim, n, order, xs, vs, q, w, J, None)
        fl_ms = time_plain(torch, flat, max(3, args.steps // 4))
        extra["flat_deposit_particles_per_s"] = round(cnt / (fl_ms * 1e-3), 1)
        extra["tiled_speedup_vs_flat"] = round(fl_ms / dep_ms, 2)
    sort_ms = time_plain(torch, resort, args.steps)
    unfused_ms = time_plain(torch, lambda: (J.zero_(), deposit(), resort()), args.steps)
    extra["unfused_step_ms"] = round(unfused_ms, 4)
    cold_ms = time_plain(torch, lambda: pcg.pcg_tile_sort(
        dim, n, order, T, xs, cur, outs=nxt, perm=perm, sorted_keys=keys, tile_offsets=off1,
        workspace=sws), max(3, args.steps // 4))
    extra["sort_without_prev_layout_ms"] = round(cold_ms, 4)
    extra["sort_only_ms"] = round(sort_ms, 4)
    extra["escaped_particles"] = n_esc
    extra["deposit_roofline"] = roof
    extra["dominant_kernel"] = dominant
    wk = {"cic2d_512_ppc16": "2-D CIC current deposit + tile sort, 512^2 periodic, 16 ppc",
          "cic3d_128_ppc32": "3-D CIC current deposit + tile sort, 128^3 periodic, 32 ppc, "
                             "2% pushed 2-4 cells",
          "tsc3d_128_blob": "3-D TSC current deposit + tile sort, 128^3 periodic, clustered "
                            "(Gaussian blob)"}[name]
    config = dict(workload=wk, particles=cnt, grid=n[:dim], order=order, tile=T, drift=D,
                  block=args.block or 512,
                  step="zero J + fused tiled deposit and regroup (incremental tile sort)")
    cpu = None
    if not args.no_cpu_baseline:
        progress("timing the oracle on the host")
        cpu = cpu_baseline_deposit(wl, order, T, args.cpu_seconds)
    return dict(value=cnt / (ms * 1e-3), ms=ms, wall=wall, dtype="f32", config=config,
                roofline=roof_dom if roof_dom else roof, kernels=kernels, extra=extra,
                cpu=cpu, unit="particles/s")


def bench_zigzag(args, torch, pcg):
    """Charge-conserving zigzag deposit on the cic3d_128_ppc32 particles, each
    moved by its velocity (x_prev = x - v, unwrapped).  The particles are
    grouped by a layout keyed on their previous positions, as the last step's
    sort left them; one step deposits their currents with that layout and
    regroups them by the new positions (incremental tile sort from it)."""
    import numpy as np

    import synthetic

    # every move is under a cell and the layout is keyed on one end of it, so
    # the window needs no drift
    T = args.tile or 8
    D = args.drift if args.drift >= 0 else 0
    progress("generating cic3d_128_ppc32 (zigzag moves)")
    wl = synthetic.workload("cic3d_128_ppc32")
    n, cnt = wl.n, wl.count
    xp = synthetic.previous_positions(wl.x, scale_v=1.0, v=wl.v)
    key0 = [np.mod(a, np.float32(n[k])).astype(np.float32) for k, a in enumerate(xp)]
    key0 = [np.where(a >= n[k], np.float32(0), a) for k, a in enumerate(key0)]
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    arrays = [t(a) for a in wl.x] + [t(a) for a in xp] + [t(wl.q), t(wl.w)]
    _, _, off0, cur = pcg.pcg_tile_sort(3, n, 1, T, [t(a) for a in key0], arrays)
    del arrays
    torch.cuda.synchronize()
    nt = pcg.ntiles(3, n, T)
    J = torch.zeros(3, n[2], n[1], n[0], dtype=torch.float32, device=dev)
    esc = torch.zeros(1, dtype=torch.int64, device=dev)
    lay = pcg.Layout(T=T, order=1, tile_offsets=off0, n_partitioned=cnt, drift=D)
    off1 = torch.empty(nt + 1, dtype=torch.int32, device=dev)
    nxt = [torch.empty_like(a) for a in cur]
    sws = torch.empty(pcg.pcg_sort_workspace_bytes(3, n, cnt, T), dtype=torch.uint8, device=dev)
    x, xpd, q, w = cur[0:3], cur[3:6], cur[6], cur[7]

    def deposit():
        pcg.deposit_currents_zigzag(n, x, xpd, q, w, J, lay, esc)

    def unfused():
        J.zero_()
        deposit()
        pcg.pcg_tile_sort(3, n, 1, T, x, cur, outs=nxt, want_perm=False, want_keys=False,
                          tile_offsets=off1, workspace=sws, prev=lay)

    def step():
        # deposit with the layout of the previous positions and regroup by the
        # new ones, in one pass over the particle arrays
        J.zero_()
        pcg.deposit_currents_zigzag_regroup(n, x, xpd, q, w, J, lay, cur, outs=nxt,
                                            tile_offsets=off1, workspace=sws)

    progress("timing steps")
    ms, wall, kt = time_steps(torch, pcg, step, args.steps, args.warmup)
    progress(f"{ms:.4f} ms per step")
    esc.zero_()
    deposit()
    torch.cuda.synchronize()
    n_esc = int(esc.item())
    jbytes = 3 * n[0] * n[1] * n[2] * 4
    alg = {
        # x, x_prev, q, w read once + J read-modify-write
        "zigzag_tiled": cnt * 8 * 4 + 2 * jbytes,
        # the same, plus every field written once to its new slot
        "zigzag_regroup": cnt * 2 * 8 * 4 + 2 * jbytes,
        "sort_inc_count": cnt * 3 * 4,
        "sort_inc_move": cnt * 2 * 8 * 4,
    }
    kernels = kernel_table(kt, args.steps, alg, gated=True)
    roof = roofline_entry(kt, "zigzag_regroup", bytes_per_launch=alg["zigzag_regroup"])
    if roof:
        roof["traffic"] = measured_traffic("zigzag_regroup", "zigzag3d_128_ppc32")
    extra = dict(escaped_particles=n_esc)
    extra["unfused_step_ms"] = round(time_plain(torch, unfused, args.steps), 4)
    _, _, kt_dep = time_steps(torch, pcg, lambda: (J.zero_(), deposit()), args.steps, 1)
    extra["deposit_roofline"] = roofline_entry(kt_dep, "zigzag_tiled",
                                               bytes_per_launch=alg["zigzag_tiled"])
    if extra["deposit_roofline"]:
        extra["deposit_roofline"]["traffic"] = measured_traffic("zigzag_tiled",
                                                                "zigzag3d_128_ppc32")
    progress("timing the step with cold caches")
    evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    extra["cold_step_ms"] = time_cold(torch, step, args.steps, evict)
    del evict
    dep_ms = time_plain(torch, lambda: (J.zero_(), deposit()), args.steps)
    extra["deposit_only_ms"] = round(dep_ms, 4)
    if not args.no_flat:
        def flat():
            J.zero_()
            pcg.deposit_currents_zigzag(n, x, xpd, q, w, J, None)
        fl_ms = time_plain(torch, flat, max(3, args.steps // 4))
        extra["flat_deposit_ms"] = round(fl_ms, 4)
        extra["tiled_speedup_vs_flat"] = round(fl_ms / dep_ms, 2)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        progress("timing the oracle on the host")

        def run(m):
            t0 = time.perf_counter()
            oracle.tile_sort(3, n, 1, T, [a[:m] for a in wl.x])
            oracle.deposit_zigzag(n, [a[:m] for a in wl.x], [a[:m] for a in xp], wl.q[:m],
                                  wl.w[:m])
            return time.perf_counter() - t0

        cal = 1 << 20
        per = run(cal) / cal
        m = int(min(cnt, max(cal, args.cpu_seconds / per)))
        sec = run(m)
        single = (m, sec, f"first {m} of {cnt} particles: oracle tile sort + fp64 zigzag "
                          f"deposit, {sec:.1f} s, 1 thread")
        from oracle import parallel

        nth = parallel.thread_count(3 * 8 * n[0] * n[1] * n[2])

        def run_par():
            t0 = time.perf_counter()
            parallel.zigzag_step(n, T, wl.x, xp, wl.q, wl.w, nth)
            sec = time.perf_counter() - t0
            return cnt, sec, (f"all {cnt} particles: oracle tile sort + fp64 zigzag deposit on "
                              f"{nth} threads (per-thread ranges, private fp64 J added in thread "
                              f"order), {sec:.1f} s")

        cpu = cpu_baseline(single, run_par, nth, "particles/s")
    config = dict(workload="3-D charge-conserving zigzag current deposit + tile sort, 128^3 "
                           "periodic, 32 ppc, each particle moved by its velocity",
                  particles=cnt, grid=n, tile=T, drift=D,
                  step="zero J + fused tiled zigzag deposit (layout of the previous "
                       "positions) and regroup (incremental tile sort on the new positions)")
    return dict(value=cnt / (ms * 1e-3), ms=ms, wall=wall, dtype="f32", config=config,
                roofline=roof, kernels=kernels, extra=extra, cpu=cpu, unit="particles/s")


# ----------------------------------------------------------------- mass matrix

def bench_mass(args, torch, pcg, scalar=False, f64=False):
    """The ECSIM mass matrix, or with scalar=True the scalar one (coefficient q w:
    x, q, w are read and sorted, 27 values per node row); f64: M and all
    arithmetic in fp64 (the fp64 entry points)."""
    import numpy as np

    import synthetic

    progress("generating mass_64_ppc64")
    wl = synthetic.workload("mass_64_ppc64")
    n, cnt = wl.n, wl.count
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x = [t(a) for a in wl.x]
    mdt = torch.float64 if f64 else torch.float32
    if scalar:
        shuffled = x + [t(wl.q), t(wl.w)]
        M = torch.zeros(n[2], n[1], n[0], 27, dtype=mdt, device=dev)
    else:
        shuffled = x + [t(b) for b in wl.B] + [t(wl.beta), t(wl.q), t(wl.w)]
        M = torch.zeros(n[2], n[1], n[0], 27, 3, 3, dtype=mdt, device=dev)
    nc = n[0] * n[1] * n[2]
    perm = torch.empty(cnt, dtype=torch.int32, device=dev)
    keys = torch.empty(cnt, dtype=torch.int32, device=dev)
    sws = torch.empty(pcg.pcg_sort_workspace_bytes(3, n, cnt, 1), dtype=torch.uint8, device=dev)
    mws = torch.empty(max(pcg.pcg_mass_workspace_bytes(n), 256), dtype=torch.uint8, device=dev)
    # the previous step's state: cell-sorted particles and their layout (set-up,
    # untimed: a cold sort of the shuffled input)
    off0 = torch.empty(nc + 1, dtype=torch.int32, device=dev)
    cur = [torch.empty_like(a) for a in shuffled]
    pcg.pcg_tile_sort(3, n, 1, 1, x, shuffled, outs=cur, perm=perm, sorted_keys=keys,
                      tile_offsets=off0, workspace=sws)
    torch.cuda.synchronize()
    prev = pcg.Layout(T=1, order=1, tile_offsets=off0, n_partitioned=cnt, drift=0)
    off1 = torch.empty(nc + 1, dtype=torch.int32, device=dev)
    nxt = [torch.empty_like(a) for a in cur]
    cells = pcg.Layout(T=1, order=1, tile_offsets=off1, n_partitioned=cnt, drift=0)

    def assemble(variant):
        if scalar:
            pcg.assemble_mass_matrix_scalar(n, nxt[0:3], nxt[3], nxt[4], M, cells, variant,
                                            workspace=mws)
        else:
            pcg.assemble_mass_matrix(n, nxt[0:3], nxt[3:6], nxt[6], nxt[7], nxt[8], M, cells,
                                     variant, workspace=mws)

    def step():
        # re-sort by cell from the previous layout, then assemble M from
        # scratch (the column kernel stores every row without reading it)
        pcg.pcg_tile_sort(3, n, 1, 1, cur[0:3], cur, outs=nxt, want_perm=False, want_keys=False,
                          tile_offsets=off1, workspace=sws, prev=prev)
        assemble(pcg.PCG_MASS_MFMA | pcg.PCG_MASS_OVERWRITE)

    progress("timing steps")
    ms, wall, kt = time_steps(torch, pcg, step, args.steps, args.warmup)
    progress(f"{ms:.4f} ms per step")
    mbytes = M.numel() * M.element_size()
    sfx = "_f64" if f64 else ""
    kname = ("mass_scalar_mfma" if scalar else "mass_mfma") + sfx
    wname = "mass_scalar_64_ppc64" if scalar else ("mass_f64_64_ppc64" if f64 else "mass_64_ppc64")
    mfma_peak = MFMA_FP64_PEAK_TFLOPS if f64 else MFMA_FP32_PEAK_TFLOPS
    # per particle: 8x8 node pairs x 2 flops (scalar) or x 9 components x 2 flops
    flops = cnt * (128.0 if scalar else 1152.0)
    # algorithmic HBM bytes: the particle values once (x, q, w; tensor: + B,
    # beta) and every row of M written once (assembled from scratch)
    pbytes = 20 if scalar else 36
    if scalar:
        roof = roofline_entry(kt, kname, bytes_per_launch=cnt * pbytes + mbytes)
    else:
        roof = roofline_entry(kt, kname, flops_per_launch=flops, mfma_peak=mfma_peak)
    if roof:
        roof["traffic"] = measured_traffic(kname, wname)
    kernels = kernel_table(kt, args.steps, {}, gated=True)
    extra = {}
    progress("timing with cold caches")
    evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    extra["cold_step_ms"] = time_cold(torch, step, args.steps, evict)
    extra["cold_assembly_ms"] = time_cold(
        torch, lambda: assemble(pcg.PCG_MASS_MFMA | pcg.PCG_MASS_OVERWRITE), args.steps, evict)
    del evict
    for nm, var in (("valu", pcg.PCG_MASS_VALU), ("mfma", pcg.PCG_MASS_MFMA)):
        mm = time_plain(torch, lambda: assemble(var | pcg.PCG_MASS_OVERWRITE), 5)
        extra[f"mass_{nm}_ms"] = round(mm, 4)
    extra["mfma_speedup_vs_valu"] = round(extra["mass_valu_ms"] / extra["mass_mfma_ms"], 2)
    extra["cold_cell_sort_ms"] = round(time_plain(torch, lambda: pcg.pcg_tile_sort(
        3, n, 1, 1, x, shuffled, outs=cur, perm=perm, sorted_keys=keys, tile_offsets=off0,
        workspace=sws), 3), 4)
    if kname in kt and not scalar:
        sec = kt[kname]["avg_us"] * 1e-6
        hbm = (cnt * pbytes + mbytes) / sec / 1e9
        extra["mass_hbm_roofline"] = dict(bound="hbm", achieved=round(hbm, 1), peak=HBM_PEAK_GBS,
                                          unit="GB/s", frac=round(hbm / HBM_PEAK_GBS, 4))
    if kname in kt and scalar:
        tf = flops / (kt[kname]["avg_us"] * 1e-6) / 1e12
        extra["mass_mfma_roofline"] = dict(bound="mfma", achieved=round(tf, 2),
                                           peak=MFMA_FP32_PEAK_TFLOPS, unit="TFLOP/s",
                                           frac=round(tf / MFMA_FP32_PEAK_TFLOPS, 4))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        progress("timing the oracle on the host")

        def run_oracle(m):
            if scalar:
                oracle.mass_matrix_scalar(n, [a[:m] for a in wl.x], wl.q[:m], wl.w[:m])
            else:
                oracle.mass_matrix(n, [a[:m] for a in wl.x], [b[:m] for b in wl.B], wl.q[:m],
                                   wl.w[:m], wl.beta[:m])

        m = 1 << 20
        t0 = time.perf_counter()
        run_oracle(m)
        per = (time.perf_counter() - t0) / m
        m2 = int(min(cnt, max(m, args.cpu_seconds / per)))
        t0 = time.perf_counter()
        run_oracle(m2)
        sec = time.perf_counter() - t0
        single = (m2, sec, f"first {m2} of {cnt} particles: fp64 per-particle outer products, "
                           f"{sec:.1f} s, 1 thread")
        from oracle import parallel

        nth = parallel.thread_count(M.numel() * 8)
        m3 = int(min(cnt, m2 * nth))

        def run_par():
            xs = [a[:m3] for a in wl.x]
            t0 = time.perf_counter()
            if scalar:
                parallel.mass(n, xs, wl.q[:m3], wl.w[:m3], nth)
            else:
                parallel.mass(n, xs, wl.q[:m3], wl.w[:m3], nth, B=[b[:m3] for b in wl.B],
                              beta=wl.beta[:m3])
            sec = time.perf_counter() - t0
            return m3, sec, (f"first {m3} of {cnt} particles: fp64 per-particle outer products "
                             f"on {nth} threads (per-thread ranges, private fp64 M added in "
                             f"thread order), {sec:.1f} s")

        cpu = cpu_baseline(single, run_par, nth, "particles/s")
    if scalar:
        config = dict(workload="scalar 3-D CIC mass matrix (coefficient q w) 64^3, 64 ppc "
                               "(cell sort + MFMA assembly)",
                      particles=cnt, grid=n,
                      step="zero M + cell re-sort of x, q, w from the previous layout + "
                           "scalar MFMA assembly")
    else:
        prec = "fp64 " if f64 else ""
        config = dict(workload=f"ECSIM 3-D CIC mass matrix {prec}64^3, 64 ppc (cell sort + "
                               "MFMA assembly)",
                      particles=cnt, grid=n,
                      step=f"zero M + cell re-sort from the previous layout + {prec}MFMA "
                           "assembly")
    return dict(value=cnt / (ms * 1e-3), ms=ms, wall=wall, dtype="f64" if f64 else "f32",
                config=config,
                roofline=roof, kernels=kernels, extra=extra, cpu=cpu, unit="particles/s")


# ----------------------------------------------------------------- 1-D sweep

def bench_sweep(args, torch, pcg):
    import numpy as np

    import synthetic

    s = synthetic.workload("sweep1d_2000")
    dev = torch.device("cuda:0")
    x0 = torch.from_numpy(s.x0).to(dev)
    v = torch.from_numpy(s.v).to(dev)
    H = torch.empty(s.nb, dtype=torch.float32, device=dev)
    step = lambda: pcg.deposit_sweep1d(s.nb, x0, v, s.T, s.dt, s.hw, H)
    ms, wall, kt = time_steps(torch, pcg, step, args.steps, args.warmup)
    kernels = {nm: dict(avg_us=round(kk["avg_us"], 2)) for nm, kk in kt.items()}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        reps = 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 2.0:
            oracle.sweep1d(s.nb, s.x0, s.v, s.T, s.dt, s.hw)
            reps += 1
        sec = (time.perf_counter() - t0) / reps
        cpu = dict(value=round(s.x0.size * s.T / sec, 1), unit="particle-steps/s", cores=1,
                   kind="oracle", sample=f"the whole workload, {reps} repetitions")
    return dict(value=s.x0.size * s.T / (ms * 1e-3), ms=ms, wall=wall, dtype="f64",
                config=dict(workload="1-D windowed CIC sweep, 2000 particles, 50 steps, 1024 bins"),
                roofline=None, kernels=kernels, extra={}, cpu=cpu, unit="particle-steps/s")


# -------------------------------------------------- scalar mass matrix, TSC weights

def bench_mass_tsc(args, torch, pcg, tensor=False):
    """Mass matrix with TSC weights on the mass_64_ppc64 particles, scalar or (tensor)
    ECSIM: re-sort by support base (T = 1, order = 2) from the previous layout,
    then assemble."""
    import numpy as np

    import synthetic

    progress("generating mass_64_ppc64")
    wl = synthetic.workload("mass_64_ppc64")
    n, cnt = wl.n, wl.count
    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x = [t(a) for a in wl.x]
    if tensor:
        shuffled = x + [t(wl.q), t(wl.w)] + [t(b) for b in wl.B] + [t(wl.beta)]
        M = torch.zeros(n[2], n[1], n[0], 125, 3, 3, dtype=torch.float32, device=dev)
    else:
        shuffled = x + [t(wl.q), t(wl.w)]
        M = torch.zeros(n[2], n[1], n[0], 125, dtype=torch.float32, device=dev)
    nc = n[0] * n[1] * n[2]
    perm = torch.empty(cnt, dtype=torch.int32, device=dev)
    keys = torch.empty(cnt, dtype=torch.int32, device=dev)
    sws = torch.empty(pcg.pcg_sort_workspace_bytes(3, n, cnt, 1), dtype=torch.uint8, device=dev)
    off0 = torch.empty(nc + 1, dtype=torch.int32, device=dev)
    cur = [torch.empty_like(a) for a in shuffled]
    pcg.pcg_tile_sort(3, n, 2, 1, x, shuffled, outs=cur, perm=perm, sorted_keys=keys,
                      tile_offsets=off0, workspace=sws)
    torch.cuda.synchronize()
    prev = pcg.Layout(T=1, order=2, tile_offsets=off0, n_partitioned=cnt, drift=0)
    off1 = torch.empty(nc + 1, dtype=torch.int32, device=dev)
    nxt = [torch.empty_like(a) for a in cur]
    groups = pcg.Layout(T=1, order=2, tile_offsets=off1, n_partitioned=cnt, drift=0)

    def assemble(variant):
        if tensor:
            pcg.assemble_mass_matrix_tsc(n, nxt[0:3], nxt[5:8], nxt[8], nxt[3], nxt[4], M, groups,
                                         variant)
        else:
            pcg.assemble_mass_matrix_scalar_tsc(n, nxt[0:3], nxt[3], nxt[4], M, groups, variant)

    def step():
        pcg.pcg_tile_sort(3, n, 2, 1, cur[0:3], cur, outs=nxt, want_perm=False, want_keys=False,
                          tile_offsets=off1, workspace=sws, prev=prev)
        assemble(pcg.PCG_MASS_MFMA | pcg.PCG_MASS_OVERWRITE)  # clears M, then adds

    progress("timing steps")
    ms, wall, kt = time_steps(torch, pcg, step, args.steps, args.warmup)
    progress(f"{ms:.4f} ms per step")
    kname = "mass_tsc_tensor_mfma" if tensor else "mass_tsc_mfma"
    wname = "mass_tsc_64_ppc64" if tensor else "mass_tsc_scalar_64_ppc64"
    # dense 27 x 27 node pairs x 2 flops (x 9 components for the tensor)
    flops = cnt * 27.0 * 27.0 * 2.0 * (9.0 if tensor else 1.0)
    roof = roofline_entry(kt, kname, flops_per_launch=flops)
    if roof:
        roof["traffic"] = measured_traffic(kname, wname)
    kernels = kernel_table(kt, args.steps, {}, gated=True)
    extra = {}
    progress("timing with cold caches")
    evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device=dev)
    extra["cold_step_ms"] = time_cold(torch, step, args.steps, evict)
    del evict
    for nm, var in (("valu", pcg.PCG_MASS_VALU), ("mfma", pcg.PCG_MASS_MFMA)):
        extra[f"mass_{nm}_ms"] = round(time_plain(
            torch, lambda: assemble(var | pcg.PCG_MASS_OVERWRITE), 5), 4)
    extra["mfma_speedup_vs_valu"] = round(extra["mass_valu_ms"] / extra["mass_mfma_ms"], 2)
    # device atomics of the brick flush, at most: every node pair that a
    # brick's groups reach (5 b + 4 per axis for b groups), x 9 components for
    # the tensor; entries that stay zero are skipped
    edge = (2, 2, 2) if tensor else (4, 4, 2)
    per_brick = 9 if tensor else 1
    bricks = 1
    for k in range(3):
        bricks *= -(-n[k] // edge[k])
        per_brick *= 5 * edge[k] + 4
    extra["flush_atomics_per_launch_max"] = bricks * per_brick
    extra["flush_atomics_per_group_max"] = round(bricks * per_brick / nc, 1)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        progress("timing the oracle on the host")
        def run_oracle(k):
            if tensor:
                oracle.mass_matrix_tsc(n, [a[:k] for a in wl.x], [b[:k] for b in wl.B], wl.q[:k],
                                       wl.w[:k], wl.beta[:k])
            else:
                oracle.mass_matrix_scalar_tsc(n, [a[:k] for a in wl.x], wl.q[:k], wl.w[:k])

        m = 1 << 16
        t0 = time.perf_counter()
        run_oracle(m)
        per = (time.perf_counter() - t0) / m
        m2 = int(min(cnt, max(m, args.cpu_seconds / per)))
        t0 = time.perf_counter()
        run_oracle(m2)
        sec = time.perf_counter() - t0
        single = (m2, sec, f"first {m2} of {cnt} particles: fp64 per-particle 27 x 27 outer "
                           f"products, {sec:.1f} s, 1 thread")
        from oracle import parallel

        nth = parallel.thread_count(M.numel() * 8)
        m3 = int(min(cnt, m2 * nth))

        def run_par():
            xs = [a[:m3] for a in wl.x]
            t0 = time.perf_counter()
            if tensor:
                parallel.mass(n, xs, wl.q[:m3], wl.w[:m3], nth, B=[b[:m3] for b in wl.B],
                              beta=wl.beta[:m3], order=2)
            else:
                parallel.mass(n, xs, wl.q[:m3], wl.w[:m3], nth, order=2)
            sec = time.perf_counter() - t0
            return m3, sec, (f"first {m3} of {cnt} particles: fp64 per-particle 27 x 27 outer "
                             f"products on {nth} threads (per-thread ranges, private fp64 M "
                             f"added in thread order), {sec:.1f} s")

        cpu = cpu_baseline(single, run_par, nth, "particles/s")
    kind = "ECSIM 3-D TSC mass matrix" if tensor else "scalar 3-D TSC mass matrix (coefficient q w)"
    config = dict(workload=f"{kind} 64^3, 64 ppc (support-group sort + MFMA assembly)",
                  particles=cnt, grid=n,
                  step="zero M + support-group re-sort of x, q, w" + (", B, beta" if tensor else "")
                       + " from the previous layout + "
                       "MFMA assembly with an atomic flush")
    return dict(value=cnt / (ms * 1e-3), ms=ms, wall=wall, dtype="f32", config=config,
                roofline=roof, kernels=kernels, extra=extra, cpu=cpu, unit="particles/s")


# ------------------------------------------------------------- 1-D sweep, reverse

FP64_VECTOR_OPS = 39.3e12   # MI355X fp64 vector instructions x lanes per s (78.6 TFLOP/s / 2)
SELECT_OPS = 9              # fp64 ops of one particle-step's selection test (see DESIGN)


def bench_sweep_grad(args, torch, pcg):
    """The page's gradient at its timing-table size: deposit_sweep1d_loss_grad
    (forward sweep into H, seed 2 (H - target), reverse gather into dx0)."""
    import numpy as np

    import synthetic

    progress("generating sweep1d_grad_1e7")
    s = synthetic.workload("sweep1d_grad_1e7")
    dev = torch.device("cuda:0")
    x0 = torch.from_numpy(s.x0).to(dev)
    v = torch.from_numpy(s.v).to(dev)
    target = torch.from_numpy(np.random.default_rng(7).random(s.nb)).to(dev)
    H = torch.empty(s.nb, dtype=torch.float32, device=dev)
    dx0 = torch.empty_like(x0)
    n, T = s.x0.size, s.T
    step = lambda: pcg.deposit_sweep1d_loss_grad(s.nb, x0, v, T, s.dt, s.hw, target, H, dx0)
    ms, wall, kt = time_steps(torch, pcg, step, args.steps, args.warmup)
    progress(f"{ms:.4f} ms per gradient")
    kernels = {nm: dict(avg_us=round(kk["avg_us"], 2)) for nm, kk in kt.items()}
    roof = None
    if "sweep1d_grad" in kt:
        sec = kt["sweep1d_grad"]["avg_us"] * 1e-6
        ops = SELECT_OPS * n * T / sec
        roof = dict(bound="alu", achieved=round(ops / 1e12, 3), peak=FP64_VECTOR_OPS / 1e12,
                    unit="T fp64 ops/s", frac=round(ops / FP64_VECTOR_OPS, 4),
                    traffic=measured_traffic("sweep1d_grad", "sweep1d_grad_1e7"),
                    kernel="sweep1d_grad", avg_us=round(kt["sweep1d_grad"]["avg_us"], 2))
    extra = dict(page_gpu_gradient_ms={"jax_compacted": 52.6, "enzyme_atomics": 146.9},
                 page_gpu="unnamed 16 GB NVIDIA GPU (context, not this machine)",
                 selected_particle_steps=int(np.count_nonzero(dx0.cpu().numpy())))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        progress("timing the oracle on the host")
        m = 200_000
        t0 = time.perf_counter()
        Ho = oracle.sweep1d(s.nb, s.x0[:m], s.v[:m], T, s.dt, s.hw)
        oracle.sweep1d_grad(s.nb, s.x0[:m], s.v[:m], T, s.dt, s.hw,
                            2.0 * (Ho - target.cpu().numpy()))
        per = (time.perf_counter() - t0) / m
        m2 = int(min(n, max(m, args.cpu_seconds / per)))
        t0 = time.perf_counter()
        Ho = oracle.sweep1d(s.nb, s.x0[:m2], s.v[:m2], T, s.dt, s.hw)
        oracle.sweep1d_grad(s.nb, s.x0[:m2], s.v[:m2], T, s.dt, s.hw,
                            2.0 * (Ho - target.cpu().numpy()))
        sec = time.perf_counter() - t0
        single = (m2 * T, sec, f"first {m2} of {n} particles, forward + reverse, {sec:.1f} s, "
                               "1 thread")
        from oracle import parallel

        nth = parallel.thread_count(1)
        m3 = int(min(n, m2 * nth))
        tg = target.cpu().numpy()

        def run_par():
            t0 = time.perf_counter()
            parallel.sweep_loss_grad(s.nb, s.x0[:m3], s.v[:m3], T, s.dt, s.hw, tg, nth)
            sec = time.perf_counter() - t0
            return m3 * T, sec, (f"first {m3} of {n} particles, forward + reverse on {nth} "
                                 f"threads (per-thread ranges, histograms added in thread "
                                 f"order), {sec:.1f} s")

        cpu = cpu_baseline(single, run_par, nth, "particle-steps/s")
    config = dict(workload="1-D windowed sweep loss gradient: 10^7 particles, 50 steps, 1024 "
                           "bins (forward, seed, reverse gather)",
                  particles=n, steps=T, bins=s.nb)
    # the page's fastest GPU gradient at this size, as the same rate (another
    # machine: context)
    page_rate = n * T / 52.6e-3
    extra["vs_baseline_is"] = "value / the page's 52.6 ms JAX gradient as particle-steps/s"
    return dict(value=n * T / (ms * 1e-3), ms=ms, wall=wall, dtype="f64", config=config,
                roofline=roof, kernels=kernels, extra=extra, cpu=cpu,
                unit="particle-steps/s", vs_baseline=round(n * T / (ms * 1e-3) / page_rate, 2))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(splitting the grid over GPUs is described, not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch

    import particle_cell_grid_amd as pcg

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    copy_gbs = None
    if not args.no_copy_bandwidth:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda:0")
        b = torch.empty_like(a)
        copy_ms = time_plain(torch, lambda: b.copy_(a), 10)
        copy_gbs = round(2 * a.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1)
        del a, b
    if args.workload in ("cic2d_512_ppc16", "cic3d_128_ppc32", "tsc3d_128_blob"):
        r = bench_deposit(args, torch, pcg, args.workload)
    elif args.workload == "mass_64_ppc64":
        r = bench_mass(args, torch, pcg)
    elif args.workload == "mass_f64_64_ppc64":
        r = bench_mass(args, torch, pcg, f64=True)
    elif args.workload == "mass_tsc_scalar_64_ppc64":
        r = bench_mass_tsc(args, torch, pcg)
    elif args.workload == "mass_tsc_64_ppc64":
        r = bench_mass_tsc(args, torch, pcg, tensor=True)
    elif args.workload == "sweep1d_grad_1e7":
        r = bench_sweep_grad(args, torch, pcg)
    elif args.workload == "mass_scalar_64_ppc64":
        r = bench_mass(args, torch, pcg, scalar=True)
    elif args.workload == "zigzag3d_128_ppc32":
        r = bench_zigzag(args, torch, pcg)
    else:
        r = bench_sweep(args, torch, pcg)
    line = {
        "metric": METRIC if args.workload == HEADLINE else f"{args.workload}: {r['unit']}",
        "value": round(r["value"], 1),
        "unit": r["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": r.get("vs_baseline"),
        "dtype": r["dtype"],
        "data": "synthetic",
        "config": r["config"],
        "roofline": r["roofline"],
        "cpu_baseline": r["cpu"],
        "kernels": r["kernels"],
        "extra": dict(r["extra"], device_copy_GBps=copy_gbs,
                      kernel_timing="kernel durations from a second pass of the same K steps "
                                    "with per-launch HIP events on the launch stream; "
                                    "ms_per_step from the first, uninstrumented pass"),
        "wall_s_timed": round(r["wall"], 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
