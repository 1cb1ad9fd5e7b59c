#!/usr/bin/env python3
"""Bench of the bucketed gradient synchronisation on one MI355X.

Metric: grad-sync GB/s and % of HBM peak; ms per bucketed sync. The default
workload is BERT-large-shaped gradients (391 fp32 tensors, 335,141,888
parameters), R = 8 replicas resident in HBM, bucket cap 25 MiB (37 buckets),
hooks firing last parameter first. One step = one whole synchronisation:
391 mark_ready calls (each bucket is launched on the side stream as it
completes, in bucket order) and finalize (the compute stream joins the side
stream).

Algorithmic bytes per step = 2 * R * S (every replica's gradients read once and
written once; S = bytes of one replica's gradients). ``value`` is that divided
by the wall-clock time per step.

Other workloads (not the default line): ``--config 1`` (nn.Linear(10,10), R=2:
microseconds per synchronised sync), ``--config 2`` (ResNet-50 shapes),
``--config 4`` (no_sync: BERT-base shapes, R=16, 8 bf16 micro-steps, then one
sync), ``--config 5`` (overlap with a bf16 MLP backward), ``--config 6`` (the
blog's 48 MiB payload, R=4, as 12 x 4 MiB or, with ``--blog-param-mib 1``,
48 x 1 MiB parameters; cap 4 MiB unless ``--cap-mib``), ``--cap-mib``,
``--mode staged|view``, ``--n-side``, ``--graph`` (replays of one captured
sync), ``--hooks many`` (all hooks in one call), ``--unused-frac`` (used
flags), ``--wg-per-cu`` (reduction workgroups per compute unit).
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
MiB = 1 << 20


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--blog-param-mib", type=int, default=4, choices=[1, 4],
                    help="--config 6: the 48 MiB payload as 12 x 4 MiB or 48 x 1 MiB parameters")
    ap.add_argument("--cap-mib", type=float, default=None)
    ap.add_argument("--replicas", type=int, default=None,
                    help="--config 2/3/6: replica count instead of the workload's (1..64; above 16 the "
                         "generic-R kernel runs)")
    ap.add_argument("--mode", choices=["fused", "staged", "view"], default="fused",
                    help="view = gradient_as_bucket_view (gradients live in flat bucket storages)")
    ap.add_argument("--n-side", type=int, default=2,
                    help="side streams; buckets go round-robin over them (0: reduce on the compute "
                         "stream itself, no cross-stream events)")
    ap.add_argument("--launch-blocks", type=int, default=None,
                    help="cap on workgroups per reduction launch (0 = whole GPU); "
                         "default 0, and for --config 5 a sweep")
    ap.add_argument("--fused-last-step", action="store_true",
                    help="--config 4: the synchronising micro-step is accumulated by the reduction "
                         "itself (ddpb_set_sync_step) instead of a separate accumulation pass")
    ap.add_argument("--step-lists", action="store_true",
                    help="--config 4: pass the step tensors as R x P lists on every call instead of "
                         "step tables checked and marshalled once")
    ap.add_argument("--wg-per-cu", type=int, default=None, choices=[0, 1, 2],
                    help="reduction workgroups per compute unit (0 = no limit); default the "
                         "library's (1), and for --config 5 a sweep of 1 and 0")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="configs 2/3/6: skip the product-native ceiling (the same tensors at R = 1)")
    ap.add_argument("--first-on-compute", action="store_true",
                    help="configs 2/3/6: the compute stream itself comes first in the side-stream list, "
                         "so bucket 0 (and every (n_side+1)-th) needs no cross-stream event")
    ap.add_argument("--roctx", action="store_true",
                    help="configs 2/3/6: bind with DDPB_BIND_ROCTX (host-side ranges for rocprofv3 "
                         "--marker-trace); --config 5: a range around each timed phase")
    ap.add_argument("--cpu-sample-gb", type=float, default=24.0,
                    help="cap on the algorithmic bytes (2*R*S) of the oracle's sample")
    ap.add_argument("--nosync-sample-mib", type=float, default=30.0,
                    help="--config 4: fp32 MiB per replica of the oracle's sample (whole buckets, at least one)")
    ap.add_argument("--overlap-sample-mib", type=float, default=256.0,
                    help="--config 5: fp32 MiB per replica of the oracle's sample (whole buckets, at least one)")
    ap.add_argument("--cpu-min-seconds", type=float, default=10.0,
                    help="the oracle repeats the sample's sync until this much CPU time")
    ap.add_argument("--no-time-launches", action="store_true",
                    help="do not record per-launch events (roofline becomes null)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one whole sync into a HIP graph after warm-up and time its replays "
                         "(no per-launch events: roofline becomes null)")
    ap.add_argument("--unused-frac", type=float, default=0.0,
                    help="fraction of (replica, variable) pairs marked unused before every sync "
                         "(seeded; at least one replica uses each variable)")
    ap.add_argument("--shuffle-params", action="store_true",
                    help="--config 5: define the parameters in a seeded shuffled order, so that the "
                         "reverse definition order no longer follows the backward")
    ap.add_argument("--rebuild", action="store_true",
                    help="--config 5: plan the first iteration as one bucket, then rebuild the buckets "
                         "from the recorded hook order before timing")
    ap.add_argument("--hooks", choices=["each", "many"], default="each",
                    help="each = one mark_ready call per hook from Python; many = the whole hook "
                         "order in one mark_ready_many call (no binding overhead per hook)")
    return ap.parse_args()


from ddp_bucketed_gradient_amd.profiling import stored_figure_current, union_length  # noqa: E402


def overlap_from_profiles(workload: str, setting: str):
    """The timeline figure of a --config 5 phase (share of the reduction
    kernels' time concurrent with backward kernels) from the kernel and
    marker trace summarised under profiles/; only while the built kernels are
    the ones measured."""
    p = os.path.join(ROOT, "profiles", "overlap.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        e = json.load(f).get(workload)
    if not e or not stored_figure_current(e):
        return None
    ph = e["phases"].get(setting)
    return dict(ph, profile=e["profile"]) if ph else None


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE and
    stored under profiles/; only used while the built kernels are the ones
    measured (the device code's hash)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(f"{kernel}:{workload}")
    if not e or not stored_figure_current(e):
        return None
    return e.get("bytes_per_launch")


COPY_BYTES = 4_000_000_000


def torch_copy_GBps(torch, nbytes: int = COPY_BYTES) -> float:
    """Bandwidth of torch's device-to-device copy of nbytes (read + write
    bytes / time; the runtime's blit kernel). Context only: a hand-written
    streaming kernel beats it, so it is no ceiling. Its 4 GB dispatches also
    calibrate the HBM byte counters of a rocprofv3 --pmc run of the bench."""
    n = nbytes // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def cpu_baseline_sync(w, host_in, nvars_sample, sample_bytes, min_seconds):
    """Times the oracle (plain NumPy, single-threaded) on the first buckets of
    the same workload and inputs."""
    import numpy as np
    from oracle import reducer as OR
    numels = w.numels()
    P = len(numels)
    first_v = P - nvars_sample
    sub = numels[first_v:]
    red = OR.Reducer(sub, w.R, w.cap_bytes)
    grads = [[host_in[v][r].copy() for v in range(first_v, P)] for r in range(w.R)]
    red.bind(grads)
    red.sync()                       # untimed: first touch of the oracle's bucket buffers
    reps = 0
    t0 = time.perf_counter()
    while True:                      # whole syncs until about min_seconds of CPU work
        red.sync()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    gbs = 2 * w.R * sample_bytes * reps / dt / 1e9
    return gbs, dt, red.B, reps


def cpu_baseline_threads(w, host_in, nvars_sample, min_seconds, threads):
    """The same oracle on the same sample, its variables dealt round-robin (by
    size) to `threads` independent oracle reducers that run concurrently (NumPy
    releases the GIL inside its array operations). Values are elementwise, so
    the split changes no result, only which thread computes it."""
    import threading
    from oracle import reducer as OR
    numels = w.numels()
    P = len(numels)
    vs = sorted(range(P - nvars_sample, P), key=lambda v: -numels[v])
    groups = [g for g in (vs[i::threads] for i in range(threads)) if g]
    reds = []
    for g in groups:
        red = OR.Reducer([numels[v] for v in g], w.R, w.cap_bytes)
        red.bind([[host_in[v][r].copy() for v in g] for r in range(w.R)])
        red.sync()                   # untimed, as in the single-thread figure
        reds.append(red)
    reps = [0] * len(reds)
    stop = threading.Event()

    def work(i):
        while not stop.is_set():
            reds[i].sync()
            reps[i] += 1

    ths = [threading.Thread(target=work, args=(i,)) for i in range(len(reds))]
    t0 = time.perf_counter()
    for t in ths:
        t.start()
    time.sleep(min_seconds)
    stop.set()
    for t in ths:
        t.join()
    dt = time.perf_counter() - t0
    done = sum(2 * w.R * 4 * sum(numels[v] for v in g) * n for g, n in zip(groups, reps))
    return done / dt / 1e9, dt, len(reds), min(reps)


def sync_workload(args, WC):
    """The workload of --config 2, 3 or 6, with --cap-mib and --replicas applied
    (both also rename it, so stored figures keyed by name do not carry over)."""
    if args.config == 2:
        w = WC.RESNET50
    elif args.config == 6:
        w = WC.BLOG_COARSE4 if args.blog_param_mib == 4 else WC.BLOG_FINE1
    else:
        w = WC.BERT_LARGE
    if args.cap_mib is not None:
        w = WC.Workload(w.cfg, f"{w.name.split('_cap')[0]}_cap{args.cap_mib:g}", w.params, w.R,
                        cap_bytes=int(args.cap_mib * MiB))
    if args.replicas is not None:
        if not 1 <= args.replicas <= 64:
            raise SystemExit("bench.py: --replicas must be in 1..64")
        w = WC.Workload(w.cfg, re.sub(r"_r\d+", f"_r{args.replicas}", w.name, count=1), w.params, args.replicas,
                        cap_bytes=w.cap_bytes)
    return w


def time_syncs(torch, red, run_step, steps, compute, timed_launches):
    """Times `steps` calls of run_step (one whole sync each) on the compute
    stream: wall clock between two device synchronisations, one event per
    sync boundary (median and p95), host time inside the calls, and -- with
    per-launch events -- the union of each sync's launch intervals."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    per_step = []                       # (starts, durations) of every launch, per step
    ring = 64                           # iterations whose launch events the library keeps
    read = 0                            # timed steps whose launch times were collected
    torch.cuda.synchronize()            # barrier (one process) + device sync
    t0 = time.perf_counter()
    host_s = 0.0
    evs[0].record(compute)
    for k in range(steps):
        h0 = time.perf_counter()
        run_step()
        host_s += time.perf_counter() - h0
        evs[k + 1].record(compute)
        # Collect launch times of steps that are about to leave the library's
        # ring, well behind the device, so the host never waits on recent work.
        while timed_launches and k - read >= ring - 8:
            per_step.append(red.launch_times_ms(k - read, True))
            read += 1
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    while timed_launches and read < steps:
        per_step.append(red.launch_times_ms(steps - 1 - read, True))
        read += 1
    sync_ms = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(steps))
    half = len(sync_ms) // 2
    return {"wall_ms": (t1 - t0) * 1e3 / steps,
            "ev_ms": evs[0].elapsed_time(evs[-1]) / steps,
            "med_ms": sync_ms[half] if len(sync_ms) % 2 else 0.5 * (sync_ms[half - 1] + sync_ms[half]),
            "p95_ms": sync_ms[-(-95 * len(sync_ms) // 100) - 1],            # nearest rank
            "host_s": host_s,
            "launch_ms": [d for _, ds in per_step for d in ds],
            "busy_ms": sum(union_length(st, ds) for st, ds in per_step)}


def product_ceiling(torch, D, grads, numels, R, cap, compute, sides, steps, warmup):
    """The practical ceiling of an in-place pass over the same bytes with the
    product's own kernel: every replica's tensor of every variable becomes a
    variable of one reducer with R = 1 (the mean of one replica is the
    replica, so each element is read once and written back once, the sync's
    1:1 mix with one stream per wave instead of R), numbered variable-major so
    that reverse order visits the R copies of each variable together, under R
    times the cap, so its buckets hold what the R-replica buckets hold. Same
    streams and launch timing; all hooks in one call. The best of one
    workgroup per CU and no limit."""
    P = len(numels)
    shapes = [(numels[v],) for v in range(P) for _ in range(R)]
    flat = [[grads[r][v].view(-1) for v in range(P) for r in range(R)]]
    order = list(range(P * R))[::-1]
    red = D.Reducer(shapes, 1, cap * R)
    red.bind(flat, compute_stream=compute, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
    # all hooks in one call: R times as many variables would otherwise make
    # the Python hook loop, not the device, the bottleneck
    def one():
        red.mark_ready_many(order)
        red.finalize()

    best = None
    for wg in (1, 0):
        red.set_workgroups_per_cu(wg)
        for _ in range(warmup):
            one()
        t = time_syncs(torch, red, one, steps, compute, True)
        if best is None or t["wall_ms"] < best[1]["wall_ms"]:
            best = (wg, t)
    wg, t = best
    alg = 2 * R * 4 * sum(numels)
    out = {"GBps": round(alg / (t["wall_ms"] * 1e-3) / 1e9, 1), "ms_per_sync": round(t["wall_ms"], 4),
           "GBps_union": round(alg * steps / (t["busy_ms"] * 1e-3) / 1e9, 1),
           "buckets": red.num_buckets, "workgroups_per_cu": wg,
           "what": f"fused_mean_kernel at R = 1 over the same {R} x {P} tensors (in place, each byte read "
                   f"once and written once), cap {R} x the sync's, same side streams, hooks in one call"}
    red.close()
    return out


def run_sync_bench(args, torch, D, WG, WC):
    w = sync_workload(args, WC)
    params = w.params()
    numels = w.numels()
    P, R = len(numels), w.R
    S = 4 * sum(numels)
    mode = D.MODE_STAGED if args.mode == "staged" else D.MODE_FUSED
    log(f"workload {w.name}: P={P} R={R} S={S / 1e6:.1f} MB cap={w.cap_bytes} mode={args.mode}")

    red = D.Reducer([p.shape for p in params], R, w.cap_bytes)
    B = red.num_buckets
    timed_launches = not (args.no_time_launches or args.graph)
    flags = D.BIND_TIME_LAUNCHES if timed_launches else 0
    if args.roctx:
        flags |= D.BIND_ROCTX
    # The compute stream and the side streams are consecutive streams of
    # torch's pool, so the HIP runtime places them on distinct hardware queues
    # (it hands out its 4 queues round-robin); the legacy null stream stays idle.
    compute = torch.cuda.Stream()
    sides = [torch.cuda.Stream() for _ in range(args.n_side)] if args.n_side > 0 else [compute]
    if args.first_on_compute and args.n_side > 0:
        sides = [compute] + sides        # bucket 0 (and every n_side+1-th) runs on the compute stream
    torch.cuda.set_stream(compute)
    if args.mode == "view":        # gradient_as_bucket_view: gradients are views of flat storages
        views = red.bind_bucket_views(compute_stream=compute, side_streams=sides, flags=flags)
        grads = [[x.view(-1) for x in row] for row in views]
    else:
        grads = [[torch.empty(n, dtype=torch.float32, device="cuda") for n in numels] for _ in range(R)]
    for r in range(R):
        for v, n in enumerate(numels):
            WG.normal(WG.seed_of(w.cfg, r, v), n, "cuda", out=grads[r][v])
    torch.cuda.synchronize()
    log("inputs generated on the device")
    if args.mode != "view":
        red.bind(grads, compute_stream=compute, side_streams=sides, mode=mode, flags=flags)
    red.set_launch_blocks(args.launch_blocks or 0)
    wg_per_cu = 1 if args.wg_per_cu is None else args.wg_per_cu
    red.set_workgroups_per_cu(wg_per_cu)
    order = w.ready_order()
    used = None
    if args.unused_frac > 0:
        import numpy as np
        rng = np.random.default_rng(7)
        used = rng.random((R, P)) >= args.unused_frac
        used[rng.integers(0, R, size=P), np.arange(P)] = True     # every variable used somewhere
        log(f"unused pairs: {int((~used).sum())} of {R * P}")
    if args.hooks == "many":
        order_arr = list(order)

        def one_sync():
            if used is not None:
                red.set_local_used(used)
            red.mark_ready_many(order_arr)
            red.finalize()
    else:
        def one_sync():
            if used is not None:
                red.set_local_used(used)
            red.sync(order)

    # snapshot of the oracle's sample (first buckets), before any sync
    cpu = None
    cpu_threads = None
    host_in = None
    nvars_sample = 0
    sample_bytes = 0
    if not args.no_cpu_baseline and args.unused_frac > 0:
        log("no CPU baseline with --unused-frac (the oracle leg times the plain sync)")
    elif not args.no_cpu_baseline:
        budget = args.cpu_sample_gb * 1e9 / (2 * R)
        for b in range(B):
            vars_b, nb = red.lib.get_bucket(red.h, b)
            if sample_bytes > 0 and sample_bytes + nb > budget:
                break
            sample_bytes += nb
            nvars_sample += len(vars_b)
        sample_vars = list(range(P - nvars_sample, P))
        host_in = {v: [grads[r][v].cpu().numpy() for r in range(R)] for v in sample_vars}
        log(f"oracle sample: {nvars_sample} tensors, {sample_bytes / 1e6:.1f} MB per replica")

    for _ in range(args.warmup):
        one_sync()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")
    run_step = one_sync
    if args.graph:                      # replays repeat the captured device work only
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=compute):
            one_sync()
        torch.cuda.synchronize()
        run_step = graph.replay
        for _ in range(args.warmup):
            run_step()
        torch.cuda.synchronize()
        log("captured one sync into a graph")

    t = time_syncs(torch, red, run_step, args.steps, compute, timed_launches)
    wall_ms, launch_ms, busy_ms = t["wall_ms"], t["launch_ms"], t["busy_ms"]
    log(f"timed {args.steps} steps: {wall_ms:.3f} ms/step wall, {t['ev_ms']:.3f} ms/step events")

    alg = 2 * R * S
    if used is not None:
        # unused pairs are not read; every variable is used by some replica,
        # so the mean is still written to every replica
        import numpy as np
        alg = 4 * int((used * np.asarray(numels, dtype=np.int64)[None, :]).sum()) + R * S
    value = alg / (wall_ms * 1e-3) / 1e9
    kernel = {"fused": "fused_mean_kernel", "view": "fused_mean_kernel(bucket view)",
              "staged": "pack+mean+copyback"}[args.mode]
    roofline = None
    if launch_ms:
        n_launch = len(launch_ms)
        assert n_launch == B * args.steps, (n_launch, B, args.steps)
        avg_ms = sum(launch_ms) / n_launch
        bytes_per_launch = alg / B
        # Three bases for the kernel's rate. With one side stream the launches
        # never overlap and the union of their intervals is the sum of their
        # durations; with several, consecutive launches run concurrently, so
        # the union is the time the kernel occupied the GPU (`achieved`), each
        # launch's own duration is stretched by its neighbour (per launch), and
        # the wall clock adds the gaps between syncs.
        achieved = alg * args.steps / (busy_ms * 1e-3) / 1e9
        per_launch = bytes_per_launch / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    # stored counters cover every variable used by every replica
                    "traffic": traffic_from_profiles(kernel, w.name) if used is None else None,
                    "kernel": kernel,
                    "basis": "union of each sync's launch intervals (HIP events on the dispatches, "
                             "side streams)",
                    "frac_union": round(achieved / HBM_PEAK_GBPS, 4),
                    "frac_per_launch": round(per_launch / HBM_PEAK_GBPS, 4),
                    "frac_wall": round(value / HBM_PEAK_GBPS, 4),
                    "launches": n_launch, "avg_launch_us": round(avg_ms * 1e3, 2),
                    "alg_bytes_per_launch": bytes_per_launch,
                    "busy_us_per_step": round(busy_ms * 1e3 / args.steps, 2),
                    "launch_concurrency": round(sum(launch_ms) / busy_ms, 3)}

    if host_in is not None:
        log("timing the oracle on the host sample")
        gbs, dt, nb, reps = cpu_baseline_sync(w, host_in, nvars_sample, sample_bytes, args.cpu_min_seconds)
        cpu = {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{w.name}: first {nb} of {B} buckets ({nvars_sample} tensors, "
                         f"{sample_bytes / 1e6:.1f} MB per replica, R={R}) from the same device inputs; "
                         f"NumPy single thread, {reps} sync(s) in {dt:.1f} s"}
        nthr = max(1, min(16, len(os.sched_getaffinity(0))))
        if nthr > 1:
            log(f"timing the oracle on the same sample in {nthr} threads")
            gbs_t, dt_t, ng, reps_t = cpu_baseline_threads(w, host_in, nvars_sample, args.cpu_min_seconds, nthr)
            cpu_threads = {"value": round(gbs_t, 3), "unit": "GB/s", "cores": ng, "kind": "oracle",
                           "sample": f"same sample, its tensors dealt to {ng} oracle reducers in threads; "
                                     f"at least {reps_t} sync(s) each in {dt_t:.1f} s"}
        del host_in

    ceiling = None
    if not args.no_ceiling and used is None and not args.graph:
        log("product ceiling: the same tensors at R = 1")
        ceiling = product_ceiling(torch, D, grads, numels, R, w.cap_bytes, compute, sides, args.steps,
                                  max(1, args.warmup))
    copy_gbps = torch_copy_GBps(torch)
    out = {
        "metric": "grad-sync GB/s and % HBM peak; ms per bucketed sync, BERT-large R=8"
        if w.cfg == 3 and R == 8 else f"grad-sync GB/s; ms per bucketed sync, {w.name}",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "tensors": P, "params": sum(numels), "replicas": R,
                   "bucket_cap_bytes": w.cap_bytes, "buckets": B, "mode": args.mode,
                   "side_streams": args.n_side, "first_bucket_on_compute_stream": bool(args.first_on_compute),
                   "hooks": args.hooks, "graph": args.graph,
                   "unused_frac": args.unused_frac, "workgroups_per_cu": wg_per_cu,
                   "launch_timing_events": timed_launches,
                   "alg_bytes_per_step": alg},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "ceiling": ceiling,
        "pct_of_ceiling": round(100 * value / ceiling["GBps"], 2) if ceiling else None,
        "torch_copy_GBps": round(copy_gbps, 1),
        "ms_per_step_events": round(t["ev_ms"], 4),
        "ms_per_sync_median": round(t["med_ms"], 4),
        "ms_per_sync_p95": round(t["p95_ms"], 4),
        "host_ms_per_step": round(t["host_s"] * 1e3 / args.steps, 4),
        "host_us_per_hook": round(t["host_s"] * 1e6 / (args.steps * P), 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_threads,
    }
    return out


def _pool_streams(torch, n_side):
    compute = torch.cuda.Stream()
    sides = [torch.cuda.Stream() for _ in range(n_side)] if n_side > 0 else [compute]
    torch.cuda.set_stream(compute)
    return compute, sides


def time_oracle_threads(make_unit, groups, min_seconds):
    """Runs make_unit(group)() repeatedly in one thread per group (NumPy
    releases the GIL inside its array operations) for about min_seconds; the
    unit returns its algorithmic bytes. Returns GB/s, seconds, the least
    number of units any thread finished."""
    import threading
    units = [make_unit(g) for g in groups]
    for u in units:
        u()                          # untimed: first touch of the oracle's buffers
    done = [0] * len(units)
    reps = [0] * len(units)
    stop = threading.Event()

    def work(i):
        while not stop.is_set():
            done[i] += units[i]()
            reps[i] += 1

    ths = [threading.Thread(target=work, args=(i,)) for i in range(len(units))]
    t0 = time.perf_counter()
    for th in ths:
        th.start()
    if len(ths) == 1:
        while time.perf_counter() - t0 < min_seconds and reps[0] == 0:
            time.sleep(0.01)
    time.sleep(max(0.0, min_seconds - (time.perf_counter() - t0)))
    stop.set()
    for th in ths:
        th.join()
    dt = time.perf_counter() - t0
    return sum(done) / dt / 1e9, dt, min(reps)


def nosync_oracle_unit(numels_s, R, k, cap, host_steps):
    """One optimizer step of config 4 in the oracle, on the sample's variables:
    k bf16 micro-steps accumulated in fp32 (the first assigns), then the
    bucketed sync. host_steps[t][r][j]: uint16 bf16 bits of variable j."""
    import numpy as np
    from oracle import reducer as OR
    orc = OR.Reducer(numels_s, R, cap)
    acc = [[np.zeros(n, np.float32) for n in numels_s] for _ in range(R)]
    orc.bind(acc)
    N = sum(numels_s)
    nbytes = R * N * (6 + 10 * (k - 1)) + 2 * R * 4 * N

    def unit():
        orc.set_sync(False)
        for t in range(k):
            if t == k - 1:
                orc.set_sync(True)
            orc.no_sync_accumulate(host_steps[t], first=(t == 0))
        orc.sync()
        return nbytes
    unit.reducer = orc               # (its gradients, for checking the unit)
    return unit


def run_nosync_bench(args, torch, D, WG, WC):
    """One step = k micro-steps: k-1 local backward passes accumulate under
    no_sync, the k-th accumulates with sync on and runs the bucketed sync."""
    w = WC.BERT_BASE_NOSYNC
    numels = w.numels()
    P, R, k = len(numels), w.R, w.micro_steps
    N = sum(numels)
    S = 4 * N
    log(f"workload {w.name}: P={P} R={R} k={k} N={N}")
    grads = [[torch.zeros(n, dtype=torch.float32, device="cuda") for n in numels] for _ in range(R)]
    # each replica's step gradients of one micro-step are one flat bf16 draw
    # (three dispatches), the variables views into it
    flats = [[WG.flat_step(4, r, t, N, "cuda") for r in range(R)] for t in range(k)]
    steps = [[WG.flat_views(flats[t][r], numels) for r in range(R)] for t in range(k)]
    torch.cuda.synchronize()
    log("inputs generated on the device")
    compute, sides = _pool_streams(torch, args.n_side)
    red = D.Reducer([p.shape for p in w.params()], R, w.cap_bytes)
    red.bind(grads, compute_stream=compute, side_streams=sides, flags=D.BIND_TIME_LAUNCHES)
    wg_per_cu = 1 if args.wg_per_cu is None else args.wg_per_cu
    red.set_workgroups_per_cu(wg_per_cu)
    order = w.ready_order()
    acc_ms = []
    # The step tensors are the same every optimizer step: check and marshal
    # their addresses once (about 2 ms of Python per micro-step otherwise,
    # which makes the loop host-bound); --step-lists passes the lists.
    step_args = steps if args.step_lists else [red.step_table(steps[t]) for t in range(k)]
    host_s = []

    def one_step(timed, n):
        h0 = time.perf_counter()
        for t in range(k):
            if t == k - 1:
                red.set_sync(True)
                if args.fused_last_step:       # the sync accumulates this step itself
                    red.set_sync_step(step_args[t], first_step=(t == 0))
                    red.sync(order)
                    continue
            e0 = e1 = None
            if timed:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(compute)
            red.no_sync_accumulate(step_args[t], first_step=(t == 0))
            if timed:
                e1.record(compute)
                acc_ms.append((n, t, e0, e1))
            red.sync(order)                    # hooks: no-ops until the last micro-step
        red.set_sync(False)
        if timed:
            host_s.append(time.perf_counter() - h0)

    red.set_sync(False)
    for i in range(args.warmup):
        one_step(False, i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(True, i)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    acc_first = [a.elapsed_time(b) for _, t, a, b in acc_ms if t == 0]
    acc_rest = [a.elapsed_time(b) for _, t, a, b in acc_ms if t > 0]
    # per optimizer step: the mean of its later micro-steps (a slow run shows here)
    by_step = [round(sum(a.elapsed_time(b) for n2, t, a, b in acc_ms if n2 == n and t > 0) /
                     max(1, sum(1 for n2, t, _, _ in acc_ms if n2 == n and t > 0)), 4) for n in range(args.steps)]
    # the last sync's launches overlap on the side streams: their union is
    # the time the reduction occupied the GPU
    st, ds = red.launch_times_ms(0, True)
    sync_ms = union_length(st, ds)
    # accumulation bytes of every micro-step, plus the sync's read and write of
    # every replica -- which the fused last step folds into its accumulation
    alg = R * N * (6 + 10 * (k - 1)) + (0 if args.fused_last_step else 2 * R * S)
    value = alg / (wall_ms * 1e-3) / 1e9
    avg_rest = sum(acc_rest) / len(acc_rest)
    bytes_rest = 10 * R * N
    achieved = bytes_rest / (avg_rest * 1e-3) / 1e9
    sync_kernel = "fused_acc_mean_kernel<bf16,add>" if args.fused_last_step else "fused_mean_kernel"
    sync_bytes = 10 * R * N if args.fused_last_step else 2 * R * S

    cpu = cpu_threads = None
    if not args.no_cpu_baseline:
        # the oracle on the first buckets' variables (the last-defined ones),
        # from the same device inputs
        budget = args.nosync_sample_mib * MiB
        nvars, sb = 0, 0
        for b in range(red.num_buckets):
            vars_b, nb = red.lib.get_bucket(red.h, b)
            if sb > 0 and sb + nb > budget:
                break
            sb += nb
            nvars += len(vars_b)
        vs = list(range(P - nvars, P))
        numels_s = [numels[v] for v in vs]
        log(f"oracle sample: {nvars} tensors, {sb / 1e6:.1f} MB per replica (fp32), R={R}, k={k}")
        host = [[[steps[t][r][v].view(torch.int16).cpu().numpy().view("uint16") for v in vs] for r in range(R)]
                for t in range(k)]
        gbs, dt, reps = time_oracle_threads(lambda g: nosync_oracle_unit(numels_s, R, k, w.cap_bytes, host),
                                            [0], args.cpu_min_seconds)
        cpu = {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{w.name}: first buckets ({nvars} tensors, {sb / 1e6:.1f} MB per replica) of the same "
                         f"device inputs; {k} micro-steps accumulated and one bucketed sync per unit, on the "
                         f"line's byte count; NumPy single thread, {reps} unit(s) in {dt:.1f} s"}
        nthr = max(1, min(16, len(os.sched_getaffinity(0))))
        if nthr > 1:
            order_v = sorted(range(len(vs)), key=lambda j: -numels_s[j])
            groups = [g for g in (order_v[i::nthr] for i in range(nthr)) if g]
            gbs_t, dt_t, reps_t = time_oracle_threads(
                lambda g: nosync_oracle_unit([numels_s[j] for j in g], R, k, w.cap_bytes,
                                             [[[host[t][r][j] for j in g] for r in range(R)] for t in range(k)]),
                groups, args.cpu_min_seconds)
            cpu_threads = {"value": round(gbs_t, 3), "unit": "GB/s", "cores": len(groups), "kind": "oracle",
                           "sample": f"same sample, its tensors dealt to {len(groups)} oracle reducers in threads; "
                                     f"at least {reps_t} unit(s) each in {dt_t:.1f} s"}
        del host
    copy_gbps = torch_copy_GBps(torch)
    return {
        "metric": f"grad-sync GB/s; ms per optimizer step (k={k} no_sync micro-steps + 1 sync), {w.name}",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "tensors": P, "params": N, "replicas": R, "micro_steps": k,
                   "step_dtype": "bf16", "buckets": red.num_buckets, "workgroups_per_cu": wg_per_cu,
                   "fused_last_step": args.fused_last_step, "step_tables": not args.step_lists,
                   "launch_timing_events": True, "alg_bytes_per_step": alg},
        "host_ms_per_step": round(1e3 * sum(host_s) / len(host_s), 4),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "accumulate_first_ms": round(sum(acc_first) / len(acc_first), 4),
        "accumulate_ms": round(avg_rest, 4),
        "accumulate_ms_by_step": by_step,
        "accumulate_ms_min_max": [round(min(acc_rest), 4), round(max(acc_rest), 4)],
        "sync_kernel": sync_kernel,
        "sync_busy_ms_last": round(sync_ms, 4),
        # the fused last step reads the accumulators and the bf16 steps and writes the mean
        "sync_busy_GBps_last": round(sync_bytes / (sync_ms * 1e-3) / 1e9, 1),
        "sync_traffic_bytes_per_launch": traffic_from_profiles(sync_kernel, w.name),
        "torch_copy_GBps": round(copy_gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profiles("accumulate_kernel<bf16,add>", w.name),
                     "kernel": "accumulate_kernel<bf16,add>",
                     "basis": "one launch per micro-step on the compute stream (events around it)",
                     "alg_bytes_per_launch": bytes_rest, "avg_launch_us": round(avg_rest * 1e3, 2)},
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_threads,
    }


def run_overlap_bench(args, torch, D, WG, WC):
    """Bucketed sync on side streams overlapping a synthetic bf16 backward of a
    24-layer MLP (d 2048, FFN 8192, 8192 tokens) on the compute stream, which
    writes replica 0's fp32 gradients layer by layer; replicas 1..7 are
    resident."""
    w = WC.MLP_OVERLAP
    params = w.params()
    numels = w.numels()
    P, R = len(numels), w.R
    S = 4 * sum(numels)
    L, d, f, T = 24, 2048, 8192, 8192
    cap = w.cap_bytes if args.cap_mib is None else int(args.cap_mib * MiB)
    log(f"workload {w.name}: P={P} R={R} S={S / 1e6:.1f} MB cap={cap}")
    grads = [[torch.empty(n, dtype=torch.float32, device="cuda") for n in numels] for _ in range(R)]
    for r in range(1, R):
        for v, n in enumerate(numels):
            WG.normal(WG.seed_of(5, r, v), n, "cuda", out=grads[r][v])
    g = torch.Generator(device="cuda").manual_seed(5)
    bf = torch.bfloat16
    X = [torch.randn(T, d, device="cuda", dtype=bf, generator=g) for _ in range(L)]
    H = [torch.randn(T, f, device="cuda", dtype=bf, generator=g) for _ in range(L)]
    W1 = [torch.randn(f, d, device="cuda", dtype=bf, generator=g) * 0.02 for _ in range(L)]
    W2 = [torch.randn(d, f, device="cuda", dtype=bf, generator=g) * 0.02 for _ in range(L)]
    dY0 = torch.randn(T, d, device="cuda", dtype=bf, generator=g)
    torch.cuda.synchronize()
    log("inputs generated on the device")
    compute, sides = _pool_streams(torch, args.n_side)
    # definition order: the architecture's, or a seeded shuffle of it; the
    # reducer numbers variables in definition order (dpos: layer-order index ->
    # reducer index), while the backward below walks the layers
    perm = WG.permutation(55, P) if args.shuffle_params else list(range(P))
    dpos = [0] * P
    for k, v in enumerate(perm):
        dpos[v] = k
    shapes_def = [params[v].shape for v in perm]
    grads_def = [[row[v] for v in perm] for row in grads]
    red = D.Reducer(shapes_def, R, (1 << 62) if args.rebuild else cap)
    # DDPB_BIND_OVERLAP: the library's setting for a reduction beside a
    # backward (no per-CU limit); the sweep below sets each value explicitly
    bind_flags = D.BIND_TIME_LAUNCHES | D.BIND_OVERLAP
    red.bind(grads_def, compute_stream=compute, side_streams=sides, flags=bind_flags)
    g0 = [grads[0][v].view(params[v].shape) for v in range(P)]
    order = [dpos[v] for v in w.ready_order()]

    def backward(hook):
        dY = dY0
        for l in range(L - 1, -1, -1):
            vW1, vb1, vW2, vb2 = 4 * l, 4 * l + 1, 4 * l + 2, 4 * l + 3
            torch.sum(dY, dim=0, dtype=torch.float32, out=g0[vb2])
            hook(vb2)
            torch.mm(dY.t(), H[l], torch.float32, out=g0[vW2])
            hook(vW2)
            dH = torch.mm(dY, W2[l])
            torch.sum(dH, dim=0, dtype=torch.float32, out=g0[vb1])
            hook(vb1)
            torch.mm(dH.t(), X[l], torch.float32, out=g0[vW1])
            hook(vW1)
            dY = torch.mm(dH, W1[l])

    def none(v):
        pass

    def hook(v):
        red.mark_ready(dpos[v])

    if args.rebuild:                    # one iteration as a single bucket records the hook order
        backward(hook)
        red.finalize()
        red.rebuild_buckets(cap)
        red.bind(grads_def, compute_stream=compute, side_streams=sides, flags=bind_flags)
        torch.cuda.synchronize()
        log(f"rebuilt into {red.num_buckets} buckets from the recorded hook order")

    def timed(fn, reps, phase):
        """ms per call of fn; with --roctx the timed calls sit in a host-side
        range named after the phase, for a marker trace."""
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with roctx_range(args.roctx, f"bench {phase}"):
            e0.record(compute)
            for _ in range(reps):
                fn()
            e1.record(compute)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    def both():
        backward(hook)
        red.finalize()

    t_bwd = timed(lambda: backward(none), args.steps, "backward alone")
    flops = 4 * 2 * T * d * f * L
    alg = 2 * R * S
    sweep = {}
    # (workgroups per CU, launch-block cap) pairs: the library's default, no
    # limit on workgroups per CU, and capped grids
    wgs = [args.wg_per_cu] if args.wg_per_cu is not None else [1, 0]
    caps = [args.launch_blocks] if args.launch_blocks is not None else [0, 32, 128]
    for wg in wgs:
        for mb in caps:
            red.set_workgroups_per_cu(wg)
            red.set_launch_blocks(mb)
            t_red = timed(lambda: red.sync(order), args.steps, f"reduction alone wg{wg} blocks{mb}")
            t_both = timed(both, args.steps, f"both wg{wg} blocks{mb}")
            hidden = max(0.0, min(1.0, (t_bwd + t_red - t_both) / t_red))
            sweep[f"wg{wg}_blocks{mb}"] = {
                "workgroups_per_cu": wg, "launch_blocks": mb,
                "t_reduction_ms": round(t_red, 4), "t_both_ms": round(t_both, 4), "hidden": round(hidden, 4),
                "reduction_kernel_ms_in_overlap": round(sum(red.launch_times_ms(0)), 4)}
            log(f"workgroups_per_cu={wg} launch_blocks={mb}: reduction {t_red:.3f} ms alone, "
                f"both {t_both:.3f} ms, hidden {hidden:.3f}")
    best = min(sweep, key=lambda k: sweep[k]["t_both_ms"])
    b = sweep[best]
    # Control: one bucket (cap above S) can only launch after the last hook,
    # so nothing overlaps and the hidden fraction should be about 0; it runs
    # with the best setting of the sweep.
    red.set_launch_blocks(0)
    red1 = D.Reducer(shapes_def, R, 1 << 62)
    red1.bind(grads_def, compute_stream=compute, side_streams=sides, flags=bind_flags)
    red1.set_workgroups_per_cu(b["workgroups_per_cu"])
    red1.set_launch_blocks(b["launch_blocks"])

    def both1():
        backward(lambda v: red1.mark_ready(dpos[v]))
        red1.finalize()

    t_red1 = timed(lambda: red1.sync(order), args.steps, "control reduction alone")
    t_both1 = timed(both1, args.steps, "control both")
    control = {"buckets": red1.num_buckets, "t_reduction_ms": round(t_red1, 4), "t_both_ms": round(t_both1, 4),
               "hidden": round(max(0.0, min(1.0, (t_bwd + t_red1 - t_both1) / t_red1)), 4)}
    log(f"single-bucket control: reduction {t_red1:.3f} ms alone, both {t_both1:.3f} ms, "
        f"hidden {control['hidden']:.3f}")
    red1.close()
    cpu = cpu_threads = None
    if not args.no_cpu_baseline:
        # the oracle's sync (pack, fixed-order mean, copy-back) on the first
        # buckets' variables, from the device's gradients as they now stand
        import numpy as np
        from oracle import reducer as OR
        nvars, sb = 0, 0
        for bb in range(red.num_buckets):
            vars_b, nb = red.lib.get_bucket(red.h, bb)
            if sb > 0 and sb + nb > args.overlap_sample_mib * MiB:
                break
            sb += nb
            nvars += len(vars_b)
        vs = list(range(P - nvars, P))           # reducer (definition-order) indices
        host = [[grads_def[r][v].cpu().numpy().copy() for v in vs] for r in range(R)]
        numels_s = [host[0][j].size for j in range(len(vs))]

        def sync_unit(js):
            orc = OR.Reducer([numels_s[j] for j in js], R, cap)
            orc.bind([[np.array(host[r][j], copy=True) for j in js] for r in range(R)])
            nbytes = 2 * R * 4 * sum(numels_s[j] for j in js)

            def unit():
                orc.sync()
                return nbytes
            return unit

        log(f"oracle sample: {nvars} tensors, {sb / 1e6:.1f} MB per replica, R={R}")
        gbs, dt, reps = time_oracle_threads(sync_unit, [list(range(len(vs)))], args.cpu_min_seconds)
        cpu = {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{w.name}: first {nvars} tensors ({sb / 1e6:.1f} MB per replica, R={R}) of the "
                         f"same gradients; the bucketed sync (pack, mean, copy-back) on the line's 2*R*S "
                         f"numerator, to set beside reduction_GBps; NumPy single thread, {reps} sync(s) in "
                         f"{dt:.1f} s"}
        nthr = max(1, min(16, len(os.sched_getaffinity(0))))
        if nthr > 1:
            order_v = sorted(range(len(vs)), key=lambda j: -numels_s[j])
            groups = [g for g in (order_v[i::nthr] for i in range(nthr)) if g]
            gbs_t, dt_t, reps_t = time_oracle_threads(sync_unit, groups, args.cpu_min_seconds)
            cpu_threads = {"value": round(gbs_t, 3), "unit": "GB/s", "cores": len(groups), "kind": "oracle",
                           "sample": f"same sample, its tensors dealt to {len(groups)} oracle reducers in "
                                     f"threads; at least {reps_t} sync(s) each in {dt_t:.1f} s"}
        del host
    return {
        "metric": f"fraction of reduction hidden under backward; ms per step, {w.name}",
        "value": b["hidden"], "unit": "fraction", "n_gpus": 1, "steps": args.steps, "warmup": 2,
        "ms_per_step": b["t_both_ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 GEMM / f32 reduce", "data": "synthetic",
        "config": {"workload": w.name, "tensors": P, "replicas": R, "bucket_cap_bytes": cap,
                   "buckets": red.num_buckets, "tokens": T, "side_streams": args.n_side,
                   "workgroups_per_cu": b["workgroups_per_cu"], "launch_blocks": b["launch_blocks"],
                   "shuffled_definition_order": args.shuffle_params, "rebuilt": args.rebuild},
        "t_backward_ms": round(t_bwd, 4), "t_reduction_ms": b["t_reduction_ms"], "t_both_ms": b["t_both_ms"],
        "backward_TFLOPs": round(flops / (t_bwd * 1e-3) / 1e12, 1),
        "reduction_GBps": round(alg / (b["t_reduction_ms"] * 1e-3) / 1e9, 1),
        "sweep": sweep,
        "single_bucket_control": control,
        # rocprofv3 timeline of the same workload (kernel intervals inside the
        # phase's marker range), stored under profiles/
        "timeline": {"best": overlap_from_profiles(w.name, best), "control": overlap_from_profiles(w.name, "control")}
        if not (args.shuffle_params or args.rebuild or args.cap_mib is not None) else None,
        "roofline": None, "cpu_baseline": cpu, "cpu_baseline_threads": cpu_threads,
    }


_ROCTX = None


class roctx_range:
    """A host-side roctx range (rocprofv3 --marker-trace) when `on`, through
    the same roctx library the native code links."""

    def __init__(self, on: bool, name: str):
        self.on, self.name = on, name

    def __enter__(self):
        global _ROCTX
        if self.on:
            if _ROCTX is None:
                import ctypes
                _ROCTX = ctypes.CDLL("/opt/rocm/lib/librocprofiler-sdk-roctx.so.1")
                _ROCTX.roctxRangePushA.argtypes = [ctypes.c_char_p]
            _ROCTX.roctxRangePushA(self.name.encode())
        return self

    def __exit__(self, *exc):
        if self.on:
            _ROCTX.roctxRangePop()
        return False


def run_latency_bench(args, torch, D, WG, WC):
    """nn.Linear(10,10) gradients (bias 10 + weight 100 floats), R = 2, one
    440-byte bucket: a latency-bound sync, reported in microseconds. Each
    timed sync is followed by a device synchronisation, so the figure is
    hooks + launch + kernel + join as a caller waiting for the result sees it."""
    w = WC.LINEAR10
    params = w.params()
    numels = w.numels()
    R = w.R
    compute, sides = _pool_streams(torch, args.n_side)
    grads = [[torch.empty(n, dtype=torch.float32, device="cuda") for n in numels] for _ in range(R)]
    for r in range(R):
        for v, n in enumerate(numels):
            WG.normal(WG.seed_of(1, r, v), n, "cuda", out=grads[r][v])
    red = D.Reducer([p.shape for p in params], R, w.cap_bytes)
    red.bind(grads, compute_stream=compute, side_streams=sides)
    wg_per_cu = 1 if args.wg_per_cu is None else args.wg_per_cu
    red.set_workgroups_per_cu(wg_per_cu)
    order = w.ready_order()
    for _ in range(args.warmup):
        red.sync(order)
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        red.sync(order)
        torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / args.steps
    log(f"timed {args.steps} syncs: {us:.1f} us each (synchronised)")
    # the oracle on the same sync, one host core (cpu_baseline leg)
    from oracle import reducer as OR
    host = [[g.cpu().numpy().copy() for g in row] for row in grads]
    orc = OR.Reducer(numels, R, w.cap_bytes)
    orc.bind(host)
    n_cpu = 0
    c0 = time.perf_counter()
    while time.perf_counter() - c0 < 1.0:
        orc.sync(order)
        n_cpu += 1
    cpu_us = (time.perf_counter() - c0) * 1e6 / n_cpu
    return {
        "metric": f"us per bucketed sync (latency bound), {w.name}",
        "value": round(us, 2), "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "tensors": len(numels), "replicas": R, "bucket_cap_bytes": w.cap_bytes,
                   "buckets": red.num_buckets, "bytes_per_replica": 4 * sum(numels),
                   "side_streams": args.n_side, "workgroups_per_cu": wg_per_cu},
        "roofline": None,
        "cpu_baseline": {"value": round(cpu_us, 2), "unit": "us", "cores": 1, "kind": "oracle",
                         "sample": f"whole workload, {n_cpu} syncs"},
    }


def main():
    args = parse()
    if args.graph and args.unused_frac > 0:
        print("bench.py: --graph and --unused-frac cannot be combined (an iteration with used flags "
              "is not captured)", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library emulates the R data-parallel "
              "replicas inside one GPU's HBM and has no collective between GPUs; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    import ddp_bucketed_gradient_amd as D
    from workloads import gen as WG, configs as WC
    torch.cuda.set_device(0)
    if args.config == 1:
        out = run_latency_bench(args, torch, D, WG, WC)
    elif args.config in (2, 3, 6):
        out = run_sync_bench(args, torch, D, WG, WC)
    elif args.config == 4:
        out = run_nosync_bench(args, torch, D, WG, WC)
    else:
        out = run_overlap_bench(args, torch, D, WG, WC)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
