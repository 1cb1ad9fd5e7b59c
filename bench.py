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

Other workloads (not the default line): ``--config 2`` (ResNet-50 shapes),
``--config 4`` (no_sync: BERT-base shapes, R=16, 8 bf16 micro-steps, then one
sync), ``--config 5`` (overlap with a bf16 MLP backward), ``--cap-mib``,
``--mode staged``, ``--n-side``.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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
    ap.add_argument("--config", type=int, default=3, choices=[2, 3, 4, 5])
    ap.add_argument("--cap-mib", type=float, default=None)
    ap.add_argument("--mode", choices=["fused", "staged"], default="fused")
    ap.add_argument("--n-side", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-gb", type=float, default=8.0,
                    help="algorithmic bytes (2*R*S) of the oracle's timed sample")
    ap.add_argument("--no-time-launches", action="store_true",
                    help="do not record per-launch events (roofline becomes null)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    p = os.path.join(ROOT, "ddp_bucketed_gradient_amd", "csrc", "kernels.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE and
    stored under profiles/; only used while the kernel source is unchanged."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        d = json.load(f)
    e = d.get(f"{kernel}:{workload}")
    if not e or e.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return e.get("bytes_per_launch")


def hbm_copy_ceiling(torch, gb: float = 2.0) -> float:
    """Plain device-to-device copy bandwidth (read + write bytes / time)."""
    n = int(gb * 1e9 / 4)
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


def cpu_baseline_sync(w, host_in, nvars_sample, sample_bytes):
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
    t0 = time.perf_counter()
    red.sync()
    dt = time.perf_counter() - t0
    gbs = 2 * w.R * sample_bytes / dt / 1e9
    return gbs, dt, red.B


def run_sync_bench(args, torch, D, WG, WC):
    if args.config == 2:
        w = WC.RESNET50
    else:
        w = WC.BERT_LARGE
    if args.cap_mib is not None:
        w = WC.Workload(w.cfg, f"{w.name.split('_cap')[0]}_cap{args.cap_mib:g}", w.params, w.R,
                        cap_bytes=int(args.cap_mib * MiB))
    params = w.params()
    numels = w.numels()
    P, R = len(numels), w.R
    S = 4 * sum(numels)
    mode = D.MODE_STAGED if args.mode == "staged" else D.MODE_FUSED
    log(f"workload {w.name}: P={P} R={R} S={S / 1e6:.1f} MB cap={w.cap_bytes} mode={args.mode}")

    grads = [[torch.empty(n, dtype=torch.float32, device="cuda") for n in numels] for _ in range(R)]
    for r in range(R):
        for v, n in enumerate(numels):
            WG.normal(WG.seed_of(w.cfg, r, v), n, "cuda", out=grads[r][v])
    torch.cuda.synchronize()
    log("inputs generated on the device")

    red = D.Reducer([p.shape for p in params], R, w.cap_bytes)
    B = red.num_buckets
    flags = 0 if args.no_time_launches else D.BIND_TIME_LAUNCHES
    sides = [torch.cuda.Stream() for _ in range(args.n_side)]
    red.bind(grads, side_streams=sides, mode=mode, flags=flags)
    order = w.ready_order()

    # snapshot of the oracle's sample (first buckets), before any sync
    cpu = None
    host_in = None
    nvars_sample = 0
    sample_bytes = 0
    if not args.no_cpu_baseline:
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
        red.sync(order)
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    compute = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    launch_ms = []
    torch.cuda.synchronize()            # barrier (one process) + device sync
    t0 = time.perf_counter()
    ev0.record(compute)
    for k in range(args.steps):
        red.sync(order)
        if flags and k >= 1:
            launch_ms += red.launch_times_ms(1)   # step k-1; step k keeps the GPU busy
    ev1.record(compute)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if flags:
        launch_ms += red.launch_times_ms(0)
    wall_ms = (t1 - t0) * 1e3 / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    log(f"timed {args.steps} steps: {wall_ms:.3f} ms/step wall, {ev_ms:.3f} ms/step events")

    alg = 2 * R * S
    value = alg / (wall_ms * 1e-3) / 1e9
    kernel = "fused_mean_kernel" if mode == D.MODE_FUSED else "pack+mean+copyback"
    roofline = None
    if launch_ms:
        n_launch = len(launch_ms)
        assert n_launch == B * args.steps, (n_launch, B, args.steps)
        avg_ms = sum(launch_ms) / n_launch
        bytes_per_launch = alg / B
        achieved = bytes_per_launch / (avg_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4),
                    "traffic": traffic_from_profiles(kernel, w.name),
                    "kernel": kernel, "launches": n_launch, "avg_launch_us": round(avg_ms * 1e3, 2),
                    "alg_bytes_per_launch": bytes_per_launch}

    if host_in is not None:
        log("timing the oracle on the host sample")
        gbs, dt, nb = cpu_baseline_sync(w, host_in, nvars_sample, sample_bytes)
        cpu = {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{w.name}: first {nb} of {B} buckets ({nvars_sample} tensors, "
                         f"{sample_bytes / 1e6:.1f} MB per replica, R={R}) from the same device inputs; "
                         f"NumPy single thread, {dt:.1f} s"}
        del host_in

    copy_gbps = hbm_copy_ceiling(torch)
    out = {
        "metric": "grad-sync GB/s and % HBM peak; ms per bucketed sync, BERT-large R=8"
        if w.cfg == 3 else f"grad-sync GB/s; ms per bucketed sync, {w.name}",
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
                   "side_streams": args.n_side, "alg_bytes_per_step": alg},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "hbm_copy_GBps": round(copy_gbps, 1),
        "ms_per_step_events": round(ev_ms, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: this build emulates the R data-parallel "
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
    if args.config in (2, 3):
        out = run_sync_bench(args, torch, D, WG, WC)
    elif args.config == 4:
        from bench_extra import run_nosync_bench
        out = run_nosync_bench(args, torch, D, WG, WC)
    else:
        from bench_extra import run_overlap_bench
        out = run_overlap_bench(args, torch, D, WG, WC)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
