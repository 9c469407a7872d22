"""Benchmark of the tiled f32 path on one MI355X.

One step is one tm_scale2d call on the 4096 x 4096 f32 matrix (X ~ N(0,1), Y = 1.5 X, 32 x 128
tiles, aligned path, 16-byte vectors): the host promise check, the tile schedule (a view with
contiguous rows is one flat row of 1 KiB work items) and the unmasked streaming kernel.  `value` is that step's throughput in GB/s of algorithmic traffic (64 MiB read +
64 MiB written, decimal GB), timed with HIP events on the launch stream over K steps that rotate
through enough buffer sets (1 GiB) that neither L2 nor the 256 MiB Infinity Cache holds a set
between its uses: the bytes come from HBM.

The same JSON line carries
  roofline      the step kernel against the 8 TB/s HBM3E peak (achieved = algorithmic bytes per
                launch / mean launch time, the event-timed region over its K launches), and its
                HBM traffic from rocprofv3 counters when profiles/ holds counters taken on the
                current kernel source;
  cpu_baseline  the CPU oracle (plain single-threaded C) on the same matrix on this host; the
                same leg checks the timed kernel's output against the oracle's, bit for bit;
  paths         every other path of the method, each on its own workload shape, its headline
                the median over 10 batches of 50 launches: the ragged path on the same shape, the
                three 1-D access variants and the 1-D ragged path, the ragged 4100 x 1000 map (as
                one flat row, and over padded rows, where the 2-D edge tiles run), row and column sums (naive and
                LDS walks; the LDS walk's one-pass form on 16 x 2^20), the masked row max, the
                softmax row statistics (also over 8 rows of 2^18, in one pass and split with a
                workspace), the per-channel bias add, a tile-size sweep and the transpose /
                NCHW -> NHWC conversion (64 channels, and 3 channels both ways).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--paths all|none] [--cpu-seconds S]
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_GBS = 8000.0            # MI355X HBM3E, published
ROTATE_BYTES = 1 << 30       # bytes touched per rotation of buffer sets
BATCHES, BATCH_LAUNCHES = 10, 50   # step batch statistics
METRIC = "achieved HBM GB/s and % of 8 TB/s peak, aligned vs ragged, per config"
STEP_KERNEL_SOURCES = ["edge_masking_vector_amd/csrc/mapflat.hip", "edge_masking_vector_amd/csrc/device.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_scale2d_4096_aligned.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--paths", choices=["main", "all", "none"], default="main",
                    help="other paths to time after the step: main (every path but the tile sweep, "
                         "whose 8192x8192 launches share the step's kernel), all (main plus the sweep), "
                         "or none")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--path-batches", type=int, default=BATCHES,
                    help="after each path's timed region, this many batches of %d launches for its median "
                         "and minimum per-launch time (0: mean only)" % BATCH_LAUNCHES)
    ap.add_argument("--sweep-out", default=None,
                    help="with --paths all: write the full tile-size sweep table (JSON) to this file")
    ap.add_argument("--size-curve", default=None,
                    help="also time the step's call (aligned scale, 32x128 tiles) on square matrices from "
                         "512 to 16384 and write per-size times and a least-squares fit of "
                         "time = bytes / bandwidth + fixed cost (JSON) to this file")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the step, time K runtime device-to-device copies of the same 64 MiB "
                         "buffers: the plain copy of known size that scales rocprofv3's byte counters")
    return ap.parse_args()


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def gbs(nbytes, seconds):
    return nbytes / seconds / 1e9


PREROLL = 2   # untimed launches queued ahead of a timed region


class Timer:
    """HIP events on the launch stream around K back-to-back launches: nothing else is enqueued in
    between, so the host stays ahead of the GPU and the mean is the kernels' own duration.

    After the synchronize that opens a region, PREROLL untimed launches (buffer sets -PREROLL ..
    -1 of the rotation) are enqueued before the start event.  The GPU is then already busy when
    the start event is reached, and the host's latency to issue the first timed launch (several
    microseconds through Python) is not counted as a step: without it, 20 timed steps of 21.4 us
    measured 21.7 us each.

    The events are created with hipEventDisableSystemFence, which HIP provides for events that
    only time work: recording one then skips the system-scope memory fence (a cache writeback and
    invalidation on this GPU) that a default event performs.  The end event still waits for every
    launch before it, so the region holds all of their work.  A region still carries the events'
    own cost: two events recorded back to back on a busy GPU measure 3.3 us apart (4.3 us with
    default events), so a 20-launch region reads about 0.15 us per launch above the kernels'
    durations (20.97 against 21.04 us per launch for the step with default events; 200-launch
    regions 20.93 us either way)."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.hip = _hip_runtime(torch)
        self.region = _timing_events(self.hip)

    def run(self, launch, n):
        torch, hip = self.torch, self.hip
        s = ctypes.c_void_p(self.stream.cuda_stream)
        torch.cuda.synchronize()
        for i in range(-PREROLL, 0):
            launch(i)
        _hip_check(hip.hipEventRecord(self.region[0], s), "hipEventRecord")
        for i in range(n):
            launch(i)
        _hip_check(hip.hipEventRecord(self.region[1], s), "hipEventRecord")
        _hip_check(hip.hipEventSynchronize(self.region[1]), "hipEventSynchronize")
        ms = ctypes.c_float()
        _hip_check(hip.hipEventElapsedTime(ctypes.byref(ms), self.region[0], self.region[1]), "hipEventElapsedTime")
        torch.cuda.synchronize()
        return ms.value * 1e-3   # seconds for n launches


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000   # hip_runtime_api.h: hipEventDisableSystemFence
_HIP = []


def _hip_runtime(torch):
    """The HIP runtime torch loaded (the same library, so the same streams and events)."""
    if not _HIP:
        hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
        hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        _HIP.append(hip)
    return _HIP[0]


def _hip_check(err, what):
    if err != 0:
        raise RuntimeError("%s failed with HIP error %d" % (what, err))


_EVENTS = []


def _timing_events(hip):
    """One pair of timing events for every region (created once, kept until the process ends)."""
    if not _EVENTS:
        for _ in range(2):
            e = ctypes.c_void_p()
            _hip_check(hip.hipEventCreateWithFlags(ctypes.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE),
                       "hipEventCreateWithFlags")
            _EVENTS.append(e)
    return _EVENTS[0], _EVENTS[1]


def rotated(torch, host, n_sets, dev, extra=0):
    """n_sets device copies of `host` (plus `extra` floats of slack at the end of each).  Output
    buffers are allocated zero-filled (torch.zeros), so that, like the inputs, every page they span
    has been written before anything is timed."""
    base = torch.from_numpy(host).to(dev)
    sets = []
    for _ in range(n_sets):
        t = torch.empty(host.size + extra, dtype=torch.float32, device=dev)
        t[:host.size].copy_(base)
        sets.append(t)
    return sets


def sets_for(bytes_per_set):
    return max(2, -(-ROTATE_BYTES // max(bytes_per_set, 1)))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this benchmark runs on exactly one GPU (the tiled maps and reductions have "
              "no cross-GPU step here); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        return 2

    import torch

    from edge_masking_vector_amd import _build, inputs
    if not (os.path.exists(_build.LIB) and os.path.exists(_build.EXT)):
        _build.build()
    from edge_masking_vector_amd import tilemap as tm

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    K, W = args.steps, args.warmup

    # ---- the step: aligned scale on 4096 x 4096 ---------------------------------------------------
    M = N = 4096
    TM, TN, alpha = 32, 128, 1.5
    step_bytes = 2 * M * N * 4
    xh = inputs.scale_input(M, N)
    R = sets_for(step_bytes)
    xs = rotated(torch, xh, R, dev)
    ys = [torch.zeros_like(x) for x in xs]

    def step(i):
        st = tm.tm_scale2d(xs[i % R], N, ys[i % R], N, M, N, alpha, TM, TN, 1, tm.TM_VAR_VEC4, stream)
        if st != tm.TM_OK:
            raise tm.TilemapError(st)

    # The other paths are measured first, so the step is timed in the state a sustained workload
    # leaves the GPU in: the first timed region of a process measured 1-2% slower than batches
    # timed later in the same process (the kernel trace shows the kernels themselves slower, with
    # no gaps between them).
    paths = (run_paths(torch, tm, inputs, dev, stream, K, W, args.sweep_out, sweep=args.paths == "all",
                       path_batches=args.path_batches)
             if args.paths != "none" else None)

    for i in range(W):
        step(i)
    total = Timer(torch, stream).run(step, K)
    ms_per_step = total / K * 1e3
    value = gbs(step_bytes, total / K)
    mean_launch = total / K   # one kernel launch per step
    achieved = gbs(step_bytes, mean_launch)
    # Batch statistics, after the timed region: BATCHES batches of BATCH_LAUNCHES launches, each
    # bracketed by its own events.
    batch = sorted(Timer(torch, stream).run(step, BATCH_LAUNCHES) / BATCH_LAUNCHES for _ in range(BATCHES))

    if args.size_curve:
        size_curve(torch, tm, inputs, dev, stream, args.size_curve)

    calib = None
    if args.calibrate_copy:
        copy = lambda i: ys[i % R].copy_(xs[i % R])
        for i in range(W):
            copy(i)
        t = Timer(torch, stream).run(copy, K) / K
        calib = {"mean_us": round(t * 1e6, 3), "gbs": round(gbs(step_bytes, t), 1),
                 "bytes_read": step_bytes // 2, "bytes_written": step_bytes // 2}

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_source_sha256") == source_digest(STEP_KERNEL_SOURCES):
            traffic = tr.get("traffic_bytes_per_launch")

    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
                "kernel": "map_flat<scale, 16-byte chunks> (mapflat.hip: one 1 KiB work item per one-wave workgroup)",
                "algorithmic_bytes_per_launch": step_bytes,
                "mean_launch_us": round(mean_launch * 1e6, 3),
                "batches": {"count": BATCHES, "launches_each": BATCH_LAUNCHES,
                            "median_launch_us": round(float(np.median(batch)) * 1e6, 3),
                            "min_launch_us": round(batch[0] * 1e6, 3)}}

    # ---- CPU baseline: the oracle on the same matrix, single-threaded ----------------------------
    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        yh = np.empty_like(xh)
        oracle.scale2d(xh, N, yh, N, M, N, alpha)
        got = ys[0].cpu().numpy()
        if not np.array_equal(got.view(np.uint32), yh.view(np.uint32)):
            print("bench.py: the timed kernel's output differs from the oracle", file=sys.stderr)
            return 1
        # one thread, pinned to one of the cores this process may use
        allowed = os.sched_getaffinity(0)
        core = min(allowed)
        os.sched_setaffinity(0, {core})
        try:
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.scale2d(xh, N, yh, N, M, N, alpha)
                reps += 1
                el = time.perf_counter() - t0
                if el >= args.cpu_seconds:
                    break
        finally:
            os.sched_setaffinity(0, allowed)
        cpu = {"value": round(gbs(step_bytes * reps, el), 3), "unit": "GB/s", "cores": 1,
               "kind": "oracle",
               "sample": "oracle scale2d over the full 4096x4096 f32 matrix, %d repetitions in %.1f s "
                         "on host core %d, one of %d this process may use (%s)"
                         % (reps, el, core, len(allowed), cpu_model())}

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "scale2d Y = 1.5*X, 4096x4096 f32 row-major (X ~ N(0,1)), 32x128 tiles, "
                               "aligned path, 16-byte vectors",
                   "M": M, "N": N, "TM": TM, "TN": TN, "aligned": 1, "variant": "VEC4",
                   "buffer_sets": R, "parallelism": "single GPU",
                   "timed_after": "the other paths" if paths is not None else "start-up",
                   "frac_of_peak": round(value / PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if paths is not None:
        ceiling = paths["ceiling_probe_copy_512MiB"]
        roofline["ceiling_gbs"] = max(ceiling["tm_copy2d_gbs"], ceiling["runtime_copy_gbs"])
        roofline["frac_of_ceiling"] = round(achieved / roofline["ceiling_gbs"], 4)
        line["paths"] = paths
    if calib is not None:
        line["calibration_copy"] = calib
    print(json.dumps(line), flush=True)
    return 0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for l in f:
                if l.startswith("model name"):
                    return l.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def run_paths(torch, tm, inputs, dev, stream, K, W, sweep_out=None, sweep=True, path_batches=BATCHES):
    """Every other path, each on its workload shape, K launches after W warm-ups (the tile sweep
    only if `sweep`)."""
    out = {}

    def timed(name, nbytes, n_sets, launch, note, plan=None):
        """W warm-ups, then K launches timed as one region (mean_us), then path_batches batches of
        BATCH_LAUNCHES launches that carry on the rotation through the buffer sets.  The headline
        (us, gbs, frac) is the median over the batches, which does not depend on --steps: with
        K = 20 a 4 us kernel's mean still carried host launch gaps.  Without batches it is the
        mean."""
        for i in range(W):
            launch(i % n_sets)
        mean = Timer(torch, stream).run(lambda i: launch(i % n_sets), K) / K
        rec = {"bytes": nbytes, "note": note, "mean_us": round(mean * 1e6, 3)}
        if plan is not None:
            rec["plan"] = plan
        head, how = mean, "mean of %d launches" % K
        if path_batches > 0:
            batch = []
            for b in range(path_batches):
                first = K + b * BATCH_LAUNCHES
                batch.append(Timer(torch, stream).run(lambda i: launch((first + i) % n_sets),
                                                      BATCH_LAUNCHES) / BATCH_LAUNCHES)
            head = float(np.median(batch))
            how = "median of %d batches of %d launches" % (path_batches, BATCH_LAUNCHES)
            rec["median_us"] = round(head * 1e6, 3)
            rec["min_us"] = round(min(batch) * 1e6, 3)
        rec["us"] = round(head * 1e6, 3)
        rec["gbs"] = round(gbs(nbytes, head), 1)
        rec["frac"] = round(gbs(nbytes, head) / PEAK_GBS, 4)
        rec["timing"] = how
        out[name] = rec

    def ok(st):
        if st != tm.TM_OK:
            raise tm.TilemapError(st)

    walk_names = {tm.TM_MAP_FLAT: "flat", tm.TM_MAP_SPAN: "span", tm.TM_MAP_TILES: "tiles"}

    def map_plan(expect, x, ldx, y, ldy, M, N, TM, TN, aligned, var):
        """The plan the map call will run (tm_map_walk), checked against the path's label."""
        st, walk, items = tm.tm_map_walk(0, x, ldx, y, ldy, M, N, TM, TN, aligned, var)
        ok(st)
        if walk_names.get(walk) != expect:
            raise RuntimeError("map %dx%d strides %d / %d runs the %s plan, labelled %s"
                               % (M, N, ldx, ldy, walk_names.get(walk), expect))
        return {"walk": expect, "items": items}

    # ceiling probe: the aligned copy and the runtime's device-to-device copy of 8192 x 8192 f32
    # (256 MiB read + 256 MiB written per launch, twice the Infinity Cache)
    M = N = 8192
    nb = 2 * M * N * 4
    R = sets_for(nb)
    xs = rotated(torch, inputs.uniform(10, M * N, -1.0, 1.0), R, dev)
    ys = [torch.zeros_like(x) for x in xs]
    timed("_probe_tm", nb, R, lambda i: ok(tm.tm_copy2d(xs[i], N, ys[i], N, M, N, 32, 128, 1,
                                                         tm.TM_VAR_VEC4, stream)), "")
    timed("_probe_rt", nb, R, lambda i: ys[i].copy_(xs[i]), "")
    a, b = out.pop("_probe_tm"), out.pop("_probe_rt")
    out["ceiling_probe_copy_512MiB"] = {
        "tm_copy2d_gbs": a["gbs"], "tm_copy2d_us": a["us"], "runtime_copy_gbs": b["gbs"],
        "runtime_copy_us": b["us"], "bytes": nb,
        "note": "8192x8192 f32: tm_copy2d aligned 32x128 vec4, and torch's device-to-device copy"}
    del xs, ys

    # 4096 x 4096 scale: ragged path (aligned=0) and scalar accesses
    M = N = 4096
    xh = inputs.scale_input(M, N)
    nb = 2 * M * N * 4
    R = sets_for(nb)
    xs = rotated(torch, xh, R, dev)
    ys = [torch.zeros_like(x) for x in xs]
    timed("scale_4096_ragged_vec4", nb, R,
          lambda i: ok(tm.tm_scale2d(xs[i], N, ys[i], N, M, N, 1.5, 32, 128, 0, tm.TM_VAR_VEC4, stream)),
          "same shape, ragged path (per-tile whole-tile test)")
    timed("scale_4096_aligned_scalar", nb, R,
          lambda i: ok(tm.tm_scale2d(xs[i], N, ys[i], N, M, N, 1.5, 32, 128, 1, tm.TM_VAR_SCALAR, stream)),
          "same shape, aligned path, one element per thread (4-byte accesses, 256-thread workgroups)")
    timed("ceiling_vendor_copy_64MiB", nb, R, lambda i: ys[i].copy_(xs[i]),
          "torch device-to-device copy of the same 64 MiB (ROCm's copy kernel), for context")
    del xs, ys

    # 1-D a*2+1 over 2**20 elements: three access variants (aligned) and the ragged VEC4 path
    n = 1 << 20
    a = inputs.map1d_input(n)
    nb = 2 * n * 4
    R = sets_for(nb)
    xs = rotated(torch, a, R, dev)
    ys = [torch.zeros_like(x) for x in xs]
    for name, var, TN, aligned, how in (
            ("map1d_scalar", tm.TM_VAR_SCALAR, 256, 1, "one element per thread (the page's scalar kernel)"),
            ("map1d_vec4_understated", tm.TM_VAR_VEC4_UNDERSTATED, 1024, 1,
             "4 elements per thread as four 4-byte accesses (alignment under-stated)"),
            ("map1d_vec4", tm.TM_VAR_VEC4, 1024, 1, "4 elements per thread as one 16-byte access"),
            ("map1d_vec4_ragged", tm.TM_VAR_VEC4, 1024, 0, "16-byte accesses")):
        timed(name, nb, R,
              lambda i, var=var, TN=TN, aligned=aligned: ok(tm.tm_map_affine(
                  xs[i], n, ys[i], n, 1, n, 2.0, 1.0, 1, TN, aligned, var, stream)),
              "1M-element a*2+1, %s, TN=%d, %s" % ("aligned" if aligned else "ragged path", TN, how))
    del xs, ys

    # ragged 4100 x 1000 affine under 64 x 64, and its aligned counterpart 4096 x 1024
    for (M, N, aligned, var, name) in ((4100, 1000, 0, tm.TM_VAR_VEC4, "affine_4100x1000_ragged_vec4"),
                                       (4100, 1000, 0, tm.TM_VAR_SCALAR, "affine_4100x1000_ragged_scalar"),
                                       (4096, 1024, 1, tm.TM_VAR_VEC4, "affine_4096x1024_aligned_vec4")):
        xh = inputs.ragged_input(M, N)
        nb = 2 * M * N * 4
        R = sets_for(nb)
        xs = rotated(torch, xh, R, dev)
        ys = [torch.zeros_like(x) for x in xs]
        timed(name, nb, R,
              lambda i, M=M, N=N, aligned=aligned, var=var: ok(tm.tm_map_affine(
                  xs[i], N, ys[i], N, M, N, 0.75, -0.25, 64, 64, aligned, var, stream)),
              "y = fmaf(x, 0.75, -0.25), 64x64 tiles; rows contiguous (row stride N), so the view is "
              "planned as one flat row whose only ragged edge is its end",
              plan=map_plan("flat", xs[0], N, ys[0], N, M, N, 64, 64, aligned, var))
        del xs, ys
    # the same ragged map over padded rows.  The view is one span of 1 KiB items on y's 1 KiB grid
    # whose columns past N are masked when the padding is under a line or at most an eighth of the
    # row, or (rows off the line grid) wider: rows off the 16-byte grid (row stride 1001), on it
    # (1004), a scale-sized view (4100 x 4100 at row stride 4104), strides that differ between x
    # and y, and 600 floats of padding (waves wholly inside it exit at once).  Different strides
    # over 16-byte rows under 1024 floats, and wide padding between rows on the line grid, keep the 2-D
    # tile plan, whose edge tiles (the bottom 4 rows, the right 40 or 4 columns) take the masked
    # body.
    for (M, N, ldx, ldy, TM, TN, var, name, expect, what) in (
            (4100, 1000, 1001, 1001, 64, 64, tm.TM_VAR_AUTO, "affine_4100x1000_ld1001_ragged_2d", "span",
             "one span of 1 KiB items, columns past N masked (rows off the 16-byte grid)"),
            (4100, 1000, 1004, 1004, 64, 64, tm.TM_VAR_VEC4, "affine_4100x1000_ld1004_ragged_2d", "span",
             "one span of 1 KiB items, columns past N masked"),
            (4100, 4100, 4104, 4104, 32, 128, tm.TM_VAR_VEC4, "scale_4100x4100_ld4104_ragged_2d", "span",
             "one span of 1 KiB items, columns past N masked"),
            (4100, 4100, 4104, 4108, 32, 128, tm.TM_VAR_VEC4, "scale_4100x4100_ldx4104_ldy4108_ragged_2d", "span",
             "one span over y, x's rows 4 floats shorter"),
            (4100, 4100, 4700, 4700, 32, 128, tm.TM_VAR_VEC4, "scale_4100x4100_ld4700_ragged_2d", "span",
             "one span, 600 floats of padding between rows (waves wholly inside it exit at once)"),
            (4100, 4100, 4104, 4104, 32, 128, tm.TM_VAR_AUTO, "scale_4100x4100_ld4104_xoff1_ragged_2d", "span",
             "one span over y, x's view one float past y's 16-byte phase: x's chunks are 4-byte "
             "aligned 16-byte loads"),
            (4100, 1000, 1004, 1008, 64, 64, tm.TM_VAR_VEC4, "affine_4100x1000_ldx1004_ldy1008_ragged_tiles", "tiles",
             "the 2-D tile plan (different strides, 16-byte rows under 1024 floats): 16-byte chunks, 4-row "
             "bottom and 64x40 right-edge tiles masked"),
            (4100, 4100, 5120, 5120, 32, 128, tm.TM_VAR_VEC4, "scale_4100x4100_ld5120_ragged_tiles", "tiles",
             "the 2-D tile plan (rows on the 128-byte line grid, 1020 floats of padding): 16-byte "
             "chunks, 32x128 tiles, 4-row bottom and 4-column right edge tiles masked")):
        xoff = 1 if "xoff1" in name else 0   # x's view this many floats into its buffer
        xh = inputs.matrix(inputs.ragged_input(M, N, seed=12), M, N, ldx)
        xh = np.concatenate([np.zeros(xoff, np.float32), xh])
        nb = 2 * M * N * 4
        R = sets_for(M * ldx * 4 + M * ldy * 4)
        xs = [x[xoff:] for x in rotated(torch, xh, R, dev)]
        ys = [torch.zeros(M * ldy, device=dev) for _ in range(R)]
        timed(name, nb, R,
              lambda i, M=M, N=N, ldx=ldx, ldy=ldy, TM=TM, TN=TN, var=var: ok(tm.tm_map_affine(
                  xs[i], ldx, ys[i], ldy, M, N, 0.75, -0.25, TM, TN, 0, var, stream)),
              "ragged path, %dx%d tiles, row strides %d / %d (padded rows): %s; bytes count the %dx%d "
              "elements only" % (TM, TN, ldx, ldy, what, M, N),
              plan=map_plan(expect, xs[0], ldx, ys[0], ldy, M, N, TM, TN, 0, var))
        del xs, ys

    # row and column sums of 4096 x 4096 U[0,1)
    M = N = 4096
    xh = inputs.colrow_input(M, N)
    R = sets_for(M * N * 4)
    xs = rotated(torch, xh, R, dev)
    outs = [torch.zeros(N, device=dev) for _ in range(R)]
    nb = M * N * 4 + N * 4
    walk = tm.tm_row_walk(M, N, N, 4, 1024, 1, xs[0])
    timed("rowsum_4096", nb, R,
          lambda i: ok(tm.tm_rowsum(xs[i], N, outs[i], M, N, 4, 1024, 1, stream)),
          "row walk, 4x1024 tiles, aligned: %d-column tiles, %d whole + %d (tm_row_walk), %d lanes per row"
          % (walk[1], walk[2], walk[3], walk[4]))
    for name, walk, TM, TN in (("colsum_naive_4096", tm.TM_COL_NAIVE, 256, 1),
                               ("colsum_naive_xcd_4096", tm.TM_COL_NAIVE_XCD, 256, 1),
                               ("colsum_lds_4096", tm.TM_COL_LDS, 256, 64)):
        wsb = tm.tm_colsum_workspace_bytes(M, N, TM, TN, walk)
        wss = [torch.zeros(wsb // 4, device=dev) for _ in range(R)]
        st, form, srows, scols, slabs, strips = tm.tm_col_walk(xs[0], N, outs[0], M, N, TM, TN,
                                                               walk == tm.TM_COL_LDS and 1 or 0, walk,
                                                               wss[0], wsb)
        ok(st)
        geometry = ("the naive walk: %d-row slabs of one column per workgroup" % srows
                    if walk != tm.TM_COL_LDS else
                    "the LDS walk's own %d-row slabs by %d-column strips (%d x %d workgroups%s)"
                    % (srows, scols, slabs, strips,
                       ", one 16-byte column chunk per thread" if form == tm.TM_COLFORM_STRIPS else ""))
        timed(name, nb, R,
              lambda i, walk=walk, TM=TM, TN=TN, wsb=wsb, wss=wss: ok(tm.tm_colsum(
                  xs[i], N, outs[i], M, N, TM, TN, walk == tm.TM_COL_LDS and 1 or 0, walk, wss[i], wsb,
                  stream)),
              "column walk, caller tile %dx%d (the promise), %s; both passes (workspace %d B not counted)"
              % (TM, TN, geometry, wsb))
        del wss
    reads_only = {k: round(gbs(M * N * 4, out[k]["us"] * 1e-6), 1)
                  for k in ("rowsum_4096", "colsum_naive_4096", "colsum_naive_xcd_4096", "colsum_lds_4096")}
    out["reads_only_gbs_4096"] = reads_only
    del xs, outs
    # column sums of a short, wide matrix (16 x 2^20): the LDS walk's one-pass form
    M, N = 16, 1 << 20
    xh = inputs.uniform(11, M * N, 0.0, 1.0)
    R = sets_for(M * N * 4)
    xs = rotated(torch, xh, R, dev)
    outs = [torch.zeros(N, device=dev) for _ in range(R)]
    assert tm.tm_colsum_workspace_bytes(M, N, 16, 64, tm.TM_COL_LDS) == 0
    timed("colsum_lds_16x1048576", M * N * 4 + N * 4, R,
          lambda i: ok(tm.tm_colsum(xs[i], N, outs[i], M, N, 16, 64, 1, tm.TM_COL_LDS, None, 0, stream)),
          "one pass: each thread adds a 16-byte column chunk down the 16 rows (no workspace)")
    del xs, outs

    # masked row max: 8192 x 1000 ragged (BC = 64: 15 whole tiles + 40 columns), aligned 8192 x 1024
    for (M, N, aligned, name) in ((8192, 1000, 0, "rowmax_8192x1000_ragged"),
                                  (8192, 1024, 1, "rowmax_8192x1024_aligned")):
        sh = inputs.scores_input(M, N)
        R = sets_for(M * N * 4)
        ss = rotated(torch, sh, R, dev)
        outs = [torch.zeros(M, device=dev) for _ in range(R)]
        nb = M * N * 4 + M * 4
        st, bc, nfull, rem, lanes = tm.tm_row_walk(M, N, N, 16, 64, aligned, ss[0])
        ok(st)
        walk = "%d-column tiles: %d whole + %s (tm_row_walk), %d lanes per row" % (
            bc, nfull, "one masked tile of %d columns" % rem if rem else "no remainder", lanes)
        timed(name, nb, R,
              lambda i, M=M, N=N, aligned=aligned: ok(tm.tm_rowmax_masked(ss[i], N, outs[i], M, N, 16, 64,
                                                                          aligned, stream)),
              "16x64 tiles, %s; -1e30 fill" % walk)
        ls = [torch.zeros(M, device=dev) for _ in range(R)]
        timed(name.replace("rowmax", "softmax_stats"), nb + M * 4, R,
              lambda i, M=M, N=N, aligned=aligned: ok(tm.tm_softmax_stats(ss[i], N, outs[i], ls[i], M, N, 16,
                                                                          64, aligned, stream)),
              "row maximum and sum of exp(s - max), 16x64 tiles, %s" % walk)
        del ss, outs, ls
    # a few long rows: softmax statistics over 8 rows of 2^18 scores, in one pass (one workgroup
    # per row) and with a workspace (row segments on separate workgroups, then one combine)
    M, N = 8, 1 << 18
    sh = inputs.uniform(6, M * N, -10.0, -1.0)
    R = sets_for(M * N * 4)
    ss = rotated(torch, sh, R, dev)
    outs = [torch.zeros(M, device=dev) for _ in range(R)]
    ls = [torch.zeros(M, device=dev) for _ in range(R)]
    wsb = tm.tm_rows_workspace_bytes(M, N)
    ws = torch.zeros(wsb // 4, device=dev)
    nb = M * N * 4 + 2 * M * 4
    timed("softmax_stats_8x262144_one_pass", nb, R,
          lambda i: ok(tm.tm_softmax_stats(ss[i], N, outs[i], ls[i], M, N, 1, 64, 0, stream)),
          "one workgroup per row")
    timed("softmax_stats_8x262144_split", nb, R,
          lambda i: ok(tm.tm_softmax_stats_ws(ss[i], N, outs[i], ls[i], M, N, 1, 64, 0, ws, wsb, stream)),
          "tm_softmax_stats_ws: %d-element row segments on separate workgroups, then a combine "
          "(workspace %d B not counted)" % (N * M * 8 // wsb, wsb))
    del ss, outs, ls, ws
    # per-channel bias add on the NHWC tensor (32, 64, 56, 56) read as a 100352 x 64 NC view
    M, N = 32 * 56 * 56, 64
    xh = inputs.uniform(7, M * N, -1.0, 1.0)
    nb = 2 * M * N * 4 + N * 4
    R = sets_for(nb)
    xs = rotated(torch, xh, R, dev)
    ys = [torch.zeros_like(x) for x in xs]
    bias = torch.from_numpy(inputs.uniform(8, N, -1.0, 1.0)).to(dev)
    timed("channel_bias_add_nhwc_32x64x56x56", nb, R,
          lambda i: ok(tm.tm_channel_affine(xs[i], N, None, bias, ys[i], N, M, N, 64, 64, 1,
                                            tm.TM_VAR_VEC4, stream)),
          "y[n, c] = x[n, c] + bias[c] on the NC view of an NHWC tensor, 64x64 tiles")
    del xs, ys

    # tile-size sweep: every tile that keeps the promise for Y = 1.5 X on 8192 x 8192 (512 MiB
    # touched per launch, more than the Infinity Cache holds)
    if sweep:
        sweep_paths(torch, tm, inputs, dev, stream, out, sweep_out)
    transpose_paths(torch, tm, inputs, dev, stream, timed, ok)
    torch.cuda.synchronize()
    return out


def size_curve(torch, tm, inputs, dev, stream, path):
    """Y = 1.5 X (aligned, VEC4, 32x128 tiles) on n x n for n = 512 .. 16384, each size over buffer
    sets rotated through at least 1 GiB; fits time = bytes / bandwidth + fixed cost (least squares
    over the sizes of at least 64 MiB moved, where the fit is not dominated by the fixed cost)."""
    rows = []
    for n in (512, 1024, 2048, 2944, 4096, 5760, 8192, 11520, 16384):  # multiples of the tile
        nb = 2 * n * n * 4
        R = sets_for(nb)
        xs = [torch.empty(n * n, device=dev).uniform_(-1.0, 1.0) for _ in range(R)]
        ys = [torch.zeros_like(x) for x in xs]

        def launch(i):
            st = tm.tm_scale2d(xs[i % R], n, ys[i % R], n, n, n, 1.5, 32, 128, 1, tm.TM_VAR_VEC4, stream)
            if st != tm.TM_OK:
                raise tm.TilemapError(st)
        K = max(20, min(400, int(2e9 // nb)))
        for i in range(10):
            launch(i)
        t = Timer(torch, stream).run(launch, K) / K
        rows.append({"n": n, "bytes": nb, "us": round(t * 1e6, 3), "gbs": round(gbs(nb, t), 1),
                     "launches": K, "buffer_sets": R})
        del xs, ys
    big = [r for r in rows if r["bytes"] >= 64 << 20]
    A = np.array([[r["bytes"], 1.0] for r in big])
    b = np.array([r["us"] * 1e-6 for r in big])
    (inv_bw, fixed), *_ = np.linalg.lstsq(A, b, rcond=None)
    with open(path, "w") as f:
        json.dump({"workload": "scale2d Y = 1.5 X, n x n f32, aligned, VEC4, 32x128 tiles",
                   "sizes": rows, "fit": {"bandwidth_gbs": round(1.0 / inv_bw / 1e9, 1),
                                          "fixed_us": round(fixed * 1e6, 3),
                                          "sizes_used": [r["n"] for r in big]}}, f, indent=1)


def sweep_paths(torch, tm, inputs, dev, stream, out, sweep_out):
    def ok(st):
        if st != tm.TM_OK:
            raise tm.TilemapError(st)
    M = N = 8192
    x = torch.from_numpy(inputs.scale_input(M, N, seed=9)).to(dev)
    y = torch.empty_like(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st, TMb, TNb, us, table = tm.tm_autotune_map(1, x, N, y, N, M, N, 1.5, 0.0, 1, tm.TM_VAR_AUTO, 5, e0, e1,
                                                 stream)
    ok(st)
    nb = 2 * M * N * 4
    runs = sorted((t, 1 << i, 1 << j) for i, row in enumerate(table) for j, t in enumerate(row) if t > 0)
    gb = sorted(gbs(nb, t * 1e-6) for t, _, _ in runs)
    out["tile_sweep_scale_8192"] = {
        "tiles_run": len(runs), "median_gbs": round(float(np.median(gb)), 1),
        "fastest_gbs": round(gb[-1], 1), "slowest_gbs": round(gb[0], 1),
        "spread": round(gb[-1] / gb[0] - 1.0, 4),
        "note": "tm_autotune_map over every menu tile keeping the promise, 5 launches each.  The tile "
                "only states the promise: every tile runs the same 1 KiB work items, so the spread is "
                "launch-to-launch noise and no tile is better than another (tm_autotune_map still "
                "reports the fastest of its run, here %dx%d)" % (TMb, TNb)}
    if sweep_out:
        with open(sweep_out, "w") as f:
            json.dump({"workload": "scale2d 8192x8192 f32, aligned", "bytes_per_launch": nb,
                       "us_per_launch": {"%dx%d" % (a, b): round(t, 3) for t, a, b in runs}}, f, indent=1)
    del x, y


def transpose_paths(torch, tm, inputs, dev, stream, timed, ok):
    # transpose 4096 x 4096 (64x64 tiles) and the NCHW -> NHWC conversion of [32][64][56*56]
    M = N = 4096
    xh = inputs.scale_input(M, N)
    nb = 2 * M * N * 4
    R = sets_for(nb)
    xs = rotated(torch, xh, R, dev)
    ys = [torch.zeros_like(x) for x in xs]
    timed("transpose_4096_aligned", nb, R,
          lambda i: ok(tm.tm_transpose(xs[i], N, 0, ys[i], M, 0, 1, M, N, 64, 64, 1, stream)),
          "y = x^T, 64x64 tiles staged through LDS")
    del xs, ys
    B, C, HW = 32, 64, 56 * 56
    xh = inputs.uniform(6, B * C * HW, -1.0, 1.0)
    nb = 2 * B * C * HW * 4
    R = sets_for(nb)
    xs = rotated(torch, xh, R, dev)
    ys = [torch.zeros_like(x) for x in xs]
    timed("nchw_to_nhwc_32x64x56x56", nb, R,
          lambda i: ok(tm.tm_transpose(xs[i], HW, C * HW, ys[i], C, HW * C, B, C, HW, 64, 64, 1, stream)),
          "batched transpose [B][C][HW] -> [B][HW][C]")
    del xs, ys
    # three channels (RGB images, 32 x 3 x 224 x 224) both ways: the packed side (rows of 3 floats)
    # moves as one contiguous block per work item
    B, C, HW = 32, 3, 224 * 224
    xh = inputs.uniform(8, B * C * HW, -1.0, 1.0)
    nb = 2 * B * C * HW * 4
    R = sets_for(nb)
    xs = rotated(torch, xh, R, dev)
    ys = [torch.zeros_like(x) for x in xs]
    timed("nchw_to_nhwc_32x3x224x224", nb, R,
          lambda i: ok(tm.tm_transpose(xs[i], HW, C * HW, ys[i], C, HW * C, B, C, HW, 1, 64, 0, stream)),
          "batched transpose [B][3][HW] -> [B][HW][3], ragged path, packed side as one block")
    timed("nhwc_to_nchw_32x3x224x224", nb, R,
          lambda i: ok(tm.tm_transpose(xs[i], C, HW * C, ys[i], HW, C * HW, B, HW, C, 64, 1, 0, stream)),
          "batched transpose [B][HW][3] -> [B][3][HW], ragged path, packed side as one block")
    del xs, ys


if __name__ == "__main__":
    sys.exit(main())
