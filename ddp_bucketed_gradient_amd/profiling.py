"""Figures from rocprofv3 output, for the bench's roofline and overlap claims.

Measurement support only: nothing here takes part in a synchronisation. Three
summaries, each printed as a small Markdown table (the text committed under
``profiles/``) and as one JSON object:

* ``trace``   -- a kernel trace (``--kernel-trace``): the launches of one
  kernel grouped into syncs of ``--per-sync`` consecutive dispatches; per
  timed sync the union of their [start, end) intervals (launches on several
  side streams overlap), the average launch duration, and the fraction of HBM
  peak each basis gives for the sync's algorithmic bytes.
* ``overlap`` -- a kernel trace and a marker trace (``--marker-trace``): the
  reduction launches that ran inside marker ranges matching ``--phase``, and
  how much of their time intersects other kernels (all of them, and those
  matching ``--compute``), the timeline evidence of overlap with a backward.
* ``traffic`` -- two counter runs (``--pmc FETCH_SIZE`` and ``--pmc
  WRITE_SIZE``): HBM bytes per launch of a kernel, each counter scaled by what
  it reads for device copies of known size in the same run.

Usage: ``python -m ddp_bucketed_gradient_amd.profiling {trace,overlap,traffic} ...``
(``--help`` on each).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from typing import List, Optional, Sequence, Tuple

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def kernel_source_hash() -> str:
    """sha256 prefix of the sources that decide what the kernels read and
    write: the kernels and their launcher, the segment planner and the
    descriptor layout they share (not the readiness state machine)."""
    h = hashlib.sha256()
    for name in ("kernels.hip", "core.hpp", "plan.cpp"):
        with open(os.path.join(ROOT, "ddp_bucketed_gradient_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def device_code_hash(lib_path: Optional[str] = None) -> Optional[str]:
    """sha256 prefix of the gfx950 device code in the built library (its
    `.hip_fatbin` section): it changes exactly when a kernel's compiled code
    changes, not when only host code does. None if the library is missing."""
    import struct
    path = lib_path or os.path.join(ROOT, "ddp_bucketed_gradient_amd", "lib", "libddpb.so")
    if not os.path.exists(path):
        return None
    with open(path, "rb") as f:
        d = f.read()
    if d[:4] != b"\x7fELF" or d[4] != 2:
        return None
    shoff = struct.unpack_from("<Q", d, 0x28)[0]
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", d, 0x3A)
    secs = [struct.unpack_from("<IIQQQQIIQQ", d, shoff + i * shentsize) for i in range(shnum)]
    stroff = secs[shstrndx][4]
    for sec in secs:
        name = d[stroff + sec[0]:d.index(b"\0", stroff + sec[0])]
        if name == b".hip_fatbin":
            return hashlib.sha256(d[sec[4]:sec[4] + sec[5]]).hexdigest()[:16]
    return None


def stored_figure_current(entry: dict) -> bool:
    """Whether a figure stored under profiles/ was measured with the kernels
    now built: by the device-code hash when the entry has one, else by the
    kernel-source hash."""
    if entry.get("device_code_sha256_16"):
        return entry["device_code_sha256_16"] == device_code_hash()
    return entry.get("kernel_source_sha256_16") == kernel_source_hash()


def union_length(starts: Sequence[float], durs: Sequence[float]) -> float:
    """Length of the union of the intervals [s, s + d)."""
    return sum(e - s for s, e in merge([(s, s + d) for s, d in zip(starts, durs)]))


def merge(iv: Sequence[Tuple[float, float]]) -> List[Tuple[float, float]]:
    """Disjoint sorted union of [s, e) intervals."""
    out: List[Tuple[float, float]] = []
    for s, e in sorted(iv):
        if out and s <= out[-1][1]:
            if e > out[-1][1]:
                out[-1] = (out[-1][0], e)
        else:
            out.append((s, e))
    return out


def intersection_length(a: Tuple[float, float], merged: List[Tuple[float, float]]) -> float:
    """Length of [a0, a1) inside the disjoint sorted intervals `merged`."""
    import bisect
    s, e = a
    i = max(0, bisect.bisect_right([m[0] for m in merged], s) - 1)
    total = 0.0
    while i < len(merged) and merged[i][0] < e:
        lo, hi = max(s, merged[i][0]), min(e, merged[i][1])
        if hi > lo:
            total += hi - lo
        i += 1
    return total


def _find(path: str, suffix: str) -> str:
    if os.path.isfile(path):
        return path
    hits = sorted(glob.glob(os.path.join(path, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {path}")
    return hits[-1]


def read_dispatches(trace: str) -> List[dict]:
    """Kernel dispatch rows (name, dispatch id, start, end in ns) of a kernel
    trace CSV, in dispatch order."""
    rows = []
    with open(_find(trace, "kernel_trace.csv"), newline="") as f:
        for r in csv.DictReader(f):
            rows.append({"name": r["Kernel_Name"], "id": int(r["Dispatch_Id"]),
                         "start": int(r["Start_Timestamp"]), "end": int(r["End_Timestamp"])})
    rows.sort(key=lambda r: r["id"])
    return rows


def read_markers(trace: str) -> List[dict]:
    rows = []
    with open(_find(trace, "marker_api_trace.csv"), newline="") as f:
        for r in csv.DictReader(f):
            rows.append({"name": r.get("Function") or r.get("Name") or "",
                         "start": int(r["Start_Timestamp"]), "end": int(r["End_Timestamp"])})
    return rows


# --- trace -------------------------------------------------------------------------

def trace_summary(dispatches: List[dict], kernel: str, per_sync: int, timed: int, alg_bytes: float,
                  peak: float = HBM_PEAK_GBPS) -> dict:
    """The last `timed` syncs of `per_sync` launches each of the kernels whose
    name matches `kernel`: busy time as the union of each sync's launch
    intervals, the average launch, and the fraction of peak on each basis
    (alg_bytes = algorithmic bytes of one sync)."""
    ks = [d for d in dispatches if re.search(kernel, d["name"])]
    need = per_sync * timed
    if len(ks) < need:
        raise ValueError(f"{len(ks)} launches of {kernel!r}, need {need}")
    ks = ks[len(ks) - need:]
    busy_ns, durs, spans = 0.0, [], []
    for k in range(timed):
        g = ks[k * per_sync:(k + 1) * per_sync]
        busy_ns += union_length([d["start"] for d in g], [d["end"] - d["start"] for d in g])
        durs += [d["end"] - d["start"] for d in g]
        spans.append(max(d["end"] for d in g) - min(d["start"] for d in g))
    avg_ns = sum(durs) / len(durs)
    busy_per_sync = busy_ns / timed
    span_ns = ks[-1]["end"] - ks[0]["start"]           # first launch start to last launch end
    gbps_union = alg_bytes / busy_per_sync              # bytes per ns = GB/s
    gbps_launch = (alg_bytes / per_sync) / avg_ns
    gbps_span = alg_bytes * timed / span_ns
    return {"kernel": kernel, "launches": need, "syncs": timed, "avg_launch_us": round(avg_ns / 1e3, 2),
            "busy_us_per_sync": round(busy_per_sync / 1e3, 2),
            "span_us_per_sync": round(span_ns / timed / 1e3, 2),
            "launch_concurrency": round(sum(durs) / busy_ns, 3),
            "GBps_union": round(gbps_union, 1), "frac_union": round(gbps_union / peak, 4),
            "GBps_per_launch": round(gbps_launch, 1), "frac_per_launch": round(gbps_launch / peak, 4),
            "GBps_span": round(gbps_span, 1), "frac_span": round(gbps_span / peak, 4)}


# --- overlap -----------------------------------------------------------------------

def overlap_summary(dispatches: List[dict], markers: List[dict], reduction: str, phase: str,
                    compute: str) -> dict:
    """Reduction launches inside marker ranges named like `phase`: the share of
    their time during which another kernel (any, and one matching `compute`)
    was running."""
    windows = [(m["start"], m["end"]) for m in markers if re.search(phase, m["name"])]
    if not windows:
        raise ValueError(f"no marker range matches {phase!r}")
    inside = lambda d: any(s <= d["start"] and d["end"] <= e for s, e in windows)  # noqa: E731
    red = [d for d in dispatches if re.search(reduction, d["name"]) and inside(d)]
    others = [d for d in dispatches if not re.search(reduction, d["name"]) and inside(d)]
    comp = [d for d in others if re.search(compute, d["name"])]
    m_all = merge([(d["start"], d["end"]) for d in others])
    m_comp = merge([(d["start"], d["end"]) for d in comp])
    total = sum(d["end"] - d["start"] for d in red)
    with_all = sum(intersection_length((d["start"], d["end"]), m_all) for d in red)
    with_comp = sum(intersection_length((d["start"], d["end"]), m_comp) for d in red)
    return {"phase": phase, "windows": len(windows), "reduction_launches": len(red),
            "reduction_kernel_ms": round(total / 1e6, 3), "compute_kernels": len(comp),
            "frac_concurrent_with_any_kernel": round(with_all / total, 4) if total else None,
            "frac_concurrent_with_compute": round(with_comp / total, 4) if total else None}


def update_overlap_json(path: str, workload: str, setting: str, summary: dict, profile: str):
    """Store one phase's overlap figures under `workload` in overlap.json (the
    file bench.py reads for the --config 5 line), stamped with the hashes of
    the kernels now built; the other phases of an entry measured with other
    kernels are dropped."""
    d = {}
    if os.path.exists(path):
        with open(path) as f:
            d = json.load(f)
    dev, src = device_code_hash(), kernel_source_hash()
    e = d.get(workload)
    if not e or e.get("device_code_sha256_16") != dev:
        e = {"phases": {}}
    e.update({"device_code_sha256_16": dev, "kernel_source_sha256_16": src, "profile": profile})
    e["phases"][setting] = {k: summary[k] for k in ("reduction_launches", "reduction_kernel_ms",
                                                    "frac_concurrent_with_any_kernel",
                                                    "frac_concurrent_with_compute")}
    d[workload] = e
    with open(path, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
        f.write("\n")


# --- host ranges ---------------------------------------------------------------------

def ranges_summary(dispatches: List[dict], markers: List[dict], kernel: str) -> dict:
    """The library's roctx ranges (DDPB_BIND_ROCTX) against the device: per
    range kind, count and average / min / max duration; and for the last
    sync (from the last `ddpb launch` range that opens a sync, i.e. the
    first launch after a finalize join, to that sync's join) the host's span,
    the device span of the kernels those launches issued (the matching
    dispatches of `kernel`, one per single-bucket launch range, in order) and
    how long after its range opened each kernel started."""
    lr = sorted((m for m in markers if m["name"].startswith("ddpb ")), key=lambda m: m["start"])
    kinds: dict = {}
    for m in lr:
        n = m["name"]
        kind = "launch 0-0" if n == "ddpb launch 0-0" else ("launch b-b" if n.startswith("ddpb launch") else n[5:])
        kinds.setdefault(kind, []).append((m["end"] - m["start"]) / 1e3)
    out = {"ranges": {k: {"calls": len(v), "avg_us": round(sum(v) / len(v), 1), "min_us": round(min(v), 1),
                          "max_us": round(max(v), 1)} for k, v in kinds.items()}}
    joins = [i for i, m in enumerate(lr) if m["name"] == "ddpb finalize join"]
    if not joins:
        return out
    last = joins[-1]
    first = joins[-2] + 1 if len(joins) > 1 else 0
    launches = [m for m in lr[first:last] if m["name"].startswith("ddpb launch")]
    ks = [d for d in dispatches if re.search(kernel, d["name"]) and d["start"] >= launches[0]["start"]]
    ks = ks[:len(launches)]
    if len(ks) < len(launches):
        return out
    delays = [(k["start"] - m["start"]) / 1e3 for k, m in zip(ks, launches)]
    out.update({"last_sync_launch_ranges": len(launches),
                "last_sync_host_span_us": round((lr[last]["end"] - launches[0]["start"]) / 1e3, 1),
                "last_sync_device_span_us": round((max(k["end"] for k in ks) - min(k["start"] for k in ks)) / 1e3, 1),
                "kernel_start_after_range_open_us": [round(min(delays), 1), round(max(delays), 1)]})
    return out


# --- traffic -----------------------------------------------------------------------

def read_counter(run: str, counter: str) -> List[Tuple[str, float]]:
    """(kernel name, counter value) per dispatch of a counter-collection CSV."""
    out = []
    with open(_find(run, "counter_collection.csv"), newline="") as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name", counter) == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def counter_summary(rows: List[Tuple[str, float]], kernel: str) -> dict:
    """Sum and per-dispatch mean of one counter over the dispatches of the
    kernels whose name matches `kernel`."""
    vals = [v for name, v in rows if re.search(kernel, name)]
    if not vals:
        raise ValueError(f"no dispatch of {kernel!r} in the counter run")
    return {"dispatches": len(vals), "total": sum(vals), "per_dispatch": round(sum(vals) / len(vals), 1)}


def traffic_summary(fetch: List[Tuple[str, float]], write: List[Tuple[str, float]], kernel: str,
                    copy_bytes: float, alg_bytes_per_launch: float, copy_kernel: str = "copyBuffer") -> dict:
    """HBM bytes per launch of `kernel` from the FETCH_SIZE and WRITE_SIZE
    runs (KiB per dispatch). Each counter is scaled by copy_bytes over what it
    reads for the largest dispatches of the copy kernel (copies of copy_bytes
    each in the same run)."""
    def scale(rows):
        vals = sorted(v for n, v in rows if re.search(copy_kernel, n))
        if not vals:
            raise ValueError("no copy dispatches to calibrate against")
        top = [v for v in vals if v >= 0.99 * vals[-1]]
        return copy_bytes / (1024.0 * sum(top) / len(top)), len(top), sum(top) / len(top)

    def per_launch(rows):
        vals = [v for n, v in rows if re.search(kernel, n)]
        if not vals:
            raise ValueError(f"no dispatch of {kernel!r}")
        return sum(vals) / len(vals), len(vals)

    sf, nf, kf = scale(fetch)
    sw, nw, kw = scale(write)
    f_kib, nlf = per_launch(fetch)
    w_kib, nlw = per_launch(write)
    fb, wb = f_kib * 1024 * sf, w_kib * 1024 * sw
    return {"kernel": kernel, "kernel_source_sha256_16": kernel_source_hash(),
            "device_code_sha256_16": device_code_hash(),
            "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
            "bytes_per_launch": round(fb + wb), "alg_bytes_per_launch": round(alg_bytes_per_launch),
            "traffic_over_algorithmic": round((fb + wb) / alg_bytes_per_launch, 4),
            "fetch_scale": round(sf, 4), "write_scale": round(sw, 4), "launches": min(nlf, nlw),
            "copy_dispatches_used": f"{nf} / {nw} copies of {copy_bytes:.0f} B",
            "copy_fetch_kib": round(kf), "copy_write_kib": round(kw)}


def update_traffic_json(path: str, key: str, entry: dict):
    d = {}
    if os.path.exists(path):
        with open(path) as f:
            d = json.load(f)
    d[key] = entry
    with open(path, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
        f.write("\n")


# --- CLI ---------------------------------------------------------------------------

def _table(d: dict) -> str:
    lines = ["| field | value |", "|---|---|"]
    lines += [f"| {k} | {v} |" for k, v in d.items()]
    return "\n".join(lines)


def main(argv: Optional[Sequence[str]] = None) -> int:
    ap = argparse.ArgumentParser(prog="python -m ddp_bucketed_gradient_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace", help="per-sync union of a kernel's launches from a kernel trace")
    t.add_argument("dir")
    t.add_argument("--kernel", required=True, help="regex on the kernel name")
    t.add_argument("--per-sync", type=int, required=True, help="launches per sync (buckets)")
    t.add_argument("--timed", type=int, required=True, help="timed syncs (the last ones in the trace)")
    t.add_argument("--alg-bytes", type=float, required=True, help="algorithmic bytes of one sync")
    t.add_argument("--peak", type=float, default=HBM_PEAK_GBPS)
    o = sub.add_parser("overlap", help="reduction time concurrent with other kernels, inside marker ranges")
    o.add_argument("dir")
    o.add_argument("--reduction", default="fused_mean_kernel")
    o.add_argument("--phase", required=True, help="regex on the marker range names")
    o.add_argument("--compute", default="Cijk|gemm|Gemm|GEMM", help="regex on the compute kernels' names")
    o.add_argument("--update", default=None, help="overlap.json to store the phase in")
    o.add_argument("--key", default=None, help="with --update: the workload's key")
    o.add_argument("--setting", default=None, help="with --update: the phase's name in the entry")
    o.add_argument("--profile", default=None, help="with --update: the summary file it comes from")
    g = sub.add_parser("ranges", help="the library's roctx ranges against the kernels they issued")
    g.add_argument("dir")
    g.add_argument("--kernel", default="fused_mean_kernel")
    n = sub.add_parser("counters", help="totals of counters over a kernel's dispatches in a --pmc run")
    n.add_argument("dir")
    n.add_argument("--counter", action="append", required=True, help="counter name as in the CSV (repeatable)")
    n.add_argument("--kernel", required=True, help="regex on the kernel name")
    c = sub.add_parser("traffic", help="HBM bytes per launch from FETCH_SIZE and WRITE_SIZE runs")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--copy-bytes", type=float, default=4e9)
    c.add_argument("--alg-bytes-per-launch", type=float, required=True)
    c.add_argument("--key", default=None, help="with --update: the entry's key (kernel:workload)")
    c.add_argument("--update", default=None, help="traffic.json to add the entry to")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        out = trace_summary(read_dispatches(a.dir), a.kernel, a.per_sync, a.timed, a.alg_bytes, a.peak)
    elif a.cmd == "overlap":
        out = overlap_summary(read_dispatches(a.dir), read_markers(a.dir), a.reduction, a.phase, a.compute)
        if a.update:
            if not (a.key and a.setting and a.profile):
                ap.error("--update needs --key, --setting and --profile")
            update_overlap_json(a.update, a.key, a.setting, out, a.profile)
    elif a.cmd == "counters":
        out = {name: counter_summary(read_counter(a.dir, name), a.kernel) for name in a.counter}
    elif a.cmd == "ranges":
        out = ranges_summary(read_dispatches(a.dir), read_markers(a.dir), a.kernel)
    else:
        out = traffic_summary(read_counter(a.fetch, "FETCH_SIZE"), read_counter(a.write, "WRITE_SIZE"),
                              a.kernel, a.copy_bytes, a.alg_bytes_per_launch)
        if a.update:
            if not a.key:
                ap.error("--update needs --key")
            update_traffic_json(a.update, a.key, out)
    print(_table(out))
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
