"""CPU tests of the profiling summaries (ddp_bucketed_gradient_amd.profiling)
on small synthetic rocprofv3 CSV files: interval unions and intersections by
brute force, the per-sync grouping of a kernel trace, marker-delimited overlap
and the copy-calibrated counter traffic."""
import csv
import json

import numpy as np
import pytest

from ddp_bucketed_gradient_amd import profiling as PF


def _brute_union(iv, res=1):
    """Length of a union of integer intervals by marking unit cells."""
    if not iv:
        return 0
    lo, hi = min(s for s, _ in iv), max(e for _, e in iv)
    cells = np.zeros(hi - lo, bool)
    for s, e in iv:
        cells[s - lo:e - lo] = True
    return int(cells.sum())


@pytest.mark.parametrize("seed", range(20))
def test_union_and_intersection_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    iv = [(int(s), int(s + d)) for s, d in zip(rng.integers(0, 200, 12), rng.integers(0, 40, 12))]
    assert PF.union_length([s for s, _ in iv], [e - s for s, e in iv]) == _brute_union(iv)
    other = [(int(s), int(s + d)) for s, d in zip(rng.integers(0, 200, 9), rng.integers(1, 30, 9))]
    m = PF.merge(other)
    for a in iv:
        both = _brute_union([a]) + _brute_union(other) - _brute_union([a] + other)
        assert PF.intersection_length(a, m) == both


def _write_trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id",
                    "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp"])
        for i, (name, s, e) in enumerate(rows):
            w.writerow(["KERNEL_DISPATCH", "Agent 1", 1, 1, 1, i + 1, 7, name, i + 1, s, e])


def test_trace_summary_groups_syncs_and_takes_unions(tmp_path):
    # two warm-up syncs, then two timed syncs of three launches, two streams overlapping
    rows = [("gen", 0, 50)]
    t = 100
    for sync in range(4):
        rows += [("void ddpb::fused_mean_kernel<8, true>(x)", t, t + 100),
                 ("void ddpb::fused_mean_kernel<8, true>(x)", t + 50, t + 150),
                 ("copyBuffer", t + 160, t + 170),
                 ("void ddpb::fused_mean_kernel<8, true>(x)", t + 150, t + 200)]
        t += 1000
    _write_trace(tmp_path / "run_kernel_trace.csv", rows)
    d = PF.read_dispatches(str(tmp_path))
    out = PF.trace_summary(d, "fused_mean_kernel", per_sync=3, timed=2, alg_bytes=800.0, peak=8.0)
    assert out["busy_us_per_sync"] == 0.2                     # union 200 ns of 250 ns of launches
    assert out["avg_launch_us"] == round(250 / 3 / 1e3, 2)
    assert out["GBps_union"] == 4.0 and out["frac_union"] == 0.5
    assert out["launch_concurrency"] == 1.25
    assert out["span_us_per_sync"] == round((1000 + 200) / 2 / 1e3, 2)
    with pytest.raises(ValueError):
        PF.trace_summary(d, "fused_mean_kernel", per_sync=3, timed=5, alg_bytes=1.0)


def test_overlap_summary_counts_only_the_phase_windows(tmp_path):
    rows = [("fused_mean_kernel<8,true>", 0, 100),             # outside every window
            ("Cijk_gemm", 1000, 1100),
            ("fused_mean_kernel<8,true>", 1050, 1150),         # 50 with the GEMM
            ("reduce_kernel", 1140, 1200),                     # +10 with another kernel
            ("fused_mean_kernel<8,true>", 1300, 1400)]         # alone
    _write_trace(tmp_path / "run_kernel_trace.csv", rows)
    with open(tmp_path / "run_marker_api_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Domain", "Function", "Start_Timestamp", "End_Timestamp"])
        w.writerow(["MARKER_CORE_API", "bench both wg0 blocks0", 900, 2000])
        w.writerow(["MARKER_CORE_API", "bench reduction alone wg0 blocks0", 0, 500])
    out = PF.overlap_summary(PF.read_dispatches(str(tmp_path)), PF.read_markers(str(tmp_path)),
                             "fused_mean_kernel", "^bench both", "Cijk")
    assert out["reduction_launches"] == 2
    assert out["frac_concurrent_with_compute"] == 0.25
    assert out["frac_concurrent_with_any_kernel"] == 0.3


def test_traffic_summary_calibrates_on_copies(tmp_path):
    def counters(path, name, copy_kib, vals):
        with open(path, "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            k = 0
            for v in copy_kib:
                k += 1
                w.writerow([k, "__amd_rocclr_copyBuffer", name, v])
            for v in vals:
                k += 1
                w.writerow([k, "accumulate_kernel<true, false>", name, v])
    counters(tmp_path / "f_counter_collection.csv", "FETCH_SIZE", [1000.0, 1000.0, 3.0], [10.0, 30.0])
    counters(tmp_path / "w_counter_collection.csv", "WRITE_SIZE", [2000.0, 2000.0], [10.0, 10.0])
    out = PF.traffic_summary(PF.read_counter(str(tmp_path / "f_counter_collection.csv"), "FETCH_SIZE"),
                             PF.read_counter(str(tmp_path / "w_counter_collection.csv"), "WRITE_SIZE"),
                             "accumulate_kernel", copy_bytes=2048000.0, alg_bytes_per_launch=51200.0)
    assert out["fetch_scale"] == 2.0 and out["write_scale"] == 1.0
    assert out["fetch_bytes_per_launch"] == 20 * 1024 * 2 and out["write_bytes_per_launch"] == 10 * 1024
    assert out["traffic_over_algorithmic"] == 1.0
    p = tmp_path / "traffic.json"
    PF.update_traffic_json(str(p), "k:w", out)
    assert json.loads(p.read_text())["k:w"]["bytes_per_launch"] == 51200


def test_overlap_json_update_keeps_phases_of_the_same_kernels(tmp_path):
    p = tmp_path / "overlap.json"
    ph = {"reduction_launches": 2, "reduction_kernel_ms": 0.2, "frac_concurrent_with_any_kernel": 0.3,
          "frac_concurrent_with_compute": 0.25, "phase": "x", "windows": 1, "compute_kernels": 1}
    PF.update_overlap_json(str(p), "w", "wg0", ph, "profiles/x.md")
    PF.update_overlap_json(str(p), "w", "control", dict(ph, frac_concurrent_with_compute=0.0), "profiles/x.md")
    e = json.loads(p.read_text())["w"]
    assert set(e["phases"]) == {"wg0", "control"}
    assert e["phases"]["control"]["frac_concurrent_with_compute"] == 0.0
    assert PF.stored_figure_current(e)
    # an entry measured with other kernels loses its phases at the next update
    e["device_code_sha256_16"] = "0" * 16
    p.write_text(json.dumps({"w": e}))
    PF.update_overlap_json(str(p), "w", "wg1", ph, "profiles/x.md")
    assert set(json.loads(p.read_text())["w"]["phases"]) == {"wg1"}


def test_ranges_summary_matches_launch_ranges_to_their_kernels():
    # two syncs of two single-bucket launches each; kernels start 5 and 7 us after their ranges open
    mk = lambda n, s, e: {"name": n, "start": s, "end": e}  # noqa: E731
    markers = [mk("ddpb launch 0-0", 0, 40_000), mk("ddpb launch 1-1", 50_000, 80_000),
               mk("ddpb finalize join", 90_000, 100_000),
               mk("ddpb launch 0-0", 200_000, 230_000), mk("ddpb launch 1-1", 240_000, 260_000),
               mk("ddpb finalize join", 270_000, 290_000), mk("bench other", 0, 1)]
    disp = [{"name": "fused_mean_kernel<8, true>", "id": i, "start": s, "end": s + 300_000}
            for i, s in enumerate([5_000, 57_000, 205_000, 247_000])]
    disp.append({"name": "other", "id": 9, "start": 201_000, "end": 202_000})
    out = PF.ranges_summary(disp, markers, "fused_mean_kernel")
    assert out["ranges"]["launch 0-0"] == {"calls": 2, "avg_us": 35.0, "min_us": 30.0, "max_us": 40.0}
    assert out["ranges"]["launch b-b"]["calls"] == 2 and out["ranges"]["finalize join"]["avg_us"] == 15.0
    assert out["last_sync_launch_ranges"] == 2
    assert out["last_sync_host_span_us"] == 90.0
    assert out["last_sync_device_span_us"] == 342.0
    assert out["kernel_start_after_range_open_us"] == [5.0, 7.0]


def test_counter_summary_sums_a_kernels_dispatches(tmp_path):
    with open(tmp_path / "r_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerow([1, "copyBuffer", "TCC_EA0_WRREQ_sum", 7.0])
        w.writerow([2, "fused_mean_kernel<8, true>", "TCC_EA0_WRREQ_sum", 10.0])
        w.writerow([2, "fused_mean_kernel<8, true>", "TCC_EA0_WRREQ_64B_sum", 4.0])
        w.writerow([3, "fused_mean_kernel<8, true>", "TCC_EA0_WRREQ_sum", 20.0])
    rows = PF.read_counter(str(tmp_path), "TCC_EA0_WRREQ_sum")
    assert PF.counter_summary(rows, "fused_mean") == {"dispatches": 2, "total": 30.0, "per_dispatch": 15.0}
    assert PF.counter_summary(PF.read_counter(str(tmp_path), "TCC_EA0_WRREQ_64B_sum"), "fused")["total"] == 4.0
    with pytest.raises(ValueError):
        PF.counter_summary(rows, "accumulate")
